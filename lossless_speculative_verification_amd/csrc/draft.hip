// Kernels of the draft block: the multi-token-prediction head that drafts the next K
// tokens on the device ("jina-ocr-v1" model page, FastMTP paragraph: drafts three
// tokens ahead for the verifier to check greedily; the head's shape is not given, so
// this is a reading: [RMSNorm(h), RMSNorm(E[t])] -> bias-free 2H -> H projection ->
// pre-norm dense SwiGLU block with a residual -> final RMSNorm -> the verifier's LM
// head, E being the LM-head matrix itself, applied K times on its own output).
// The projection and the block run on the streaming expert GEMM (k_moe_gemm) and the
// norms on the split norm kernel; this file holds the glue: the block's input rows,
// the row-block work list and the final store of the drafts.
#include "launch.h"

namespace mv {

// Input rows of draft step i for sequence b (one workgroup per sequence):
//   step 0: hidden state = hidden[b*(Kv+1) + n_b], token = committed[b][n_b]
//           (n_b = accepted_len[b], the row of the last accepted position);
//   step i > 0: hidden state = z_prev[b], token = ids_prev[b] (the previous step's
//           draft, also stored as drafts[b][i-1]).
// U[b] = [bf16(RMSNorm(h)), bf16(RMSNorm(E[token]))] in the weight element type; the
// embedding row is read from the LM head's pair layout (tile = row / 16 holds rows in
// lanes % 16; within a 256-byte K block, lane group g and sub-chunk s hold bytes
// g*64 + s*16 .. +16). Tokens outside [0, V) are clamped (the verifier never emits them).
template <typename T>
__global__ __launch_bounds__(256) void k_draft_input(const float* __restrict__ hidden,
                                                     const int32_t* __restrict__ accepted,
                                                     const int32_t* __restrict__ committed, int Kv,
                                                     const float* __restrict__ z_prev,
                                                     const int32_t* __restrict__ ids_prev,
                                                     int32_t* __restrict__ drafts, int K, int step,
                                                     const uint4* __restrict__ lm, int NKB, int H, int V,
                                                     float eps, T* __restrict__ U) {
  constexpr int EPC = 16 / (int)sizeof(T);  // elements per 16-byte chunk
  __shared__ float red[2][4];
  const int b = blockIdx.x, lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const float* h;
  int tok;
  if (step == 0) {
    const int n = min(max(accepted[b], 0), Kv);
    h = hidden + ((size_t)b * (Kv + 1) + n) * H;
    tok = committed[(size_t)b * (Kv + 1) + n];
  } else {
    h = z_prev + (size_t)b * H;
    tok = ids_prev[b];
    if (threadIdx.x == 0) drafts[(size_t)b * K + step - 1] = tok;
  }
  tok = min(max(tok, 0), V - 1);
  const int tile = tok >> 4, q = tile >> 1, t = tile & 1;
  const int n_ch = H / EPC;
  constexpr int MAXC = 4;  // chunks per thread: H <= 4096 elements
  float hv[MAXC][EPC], ev[MAXC][EPC];
  float sh = 0.f, se = 0.f;
#pragma unroll
  for (int i = 0; i < MAXC; ++i) {
    const int ch = threadIdx.x + i * 256;
    if (ch < n_ch) {
      const int o = ch * 16;  // byte offset in the embedding row
      const int kb = o >> 8, g = (o >> 6) & 3, s = (o >> 4) & 3;
      const size_t unit = ((((size_t)q * NKB + kb) * 2 + t) * 4 + s) * kWave + g * 16 + (tok & 15);
      const uint4 raw = lm[unit];
      const T* ep = reinterpret_cast<const T*>(&raw);
#pragma unroll
      for (int j = 0; j < EPC; ++j) {
        hv[i][j] = h[ch * EPC + j];
        ev[i][j] = Elem<T>::load(ep, j);
        sh += hv[i][j] * hv[i][j];
        se += ev[i][j] * ev[i][j];
      }
    }
  }
  sh = wave_sum(sh);
  se = wave_sum(se);
  if (lane == 0) {
    red[0][wave] = sh;
    red[1][wave] = se;
  }
  __syncthreads();
  const float ih = 1.0f / sqrtf((red[0][0] + red[0][1] + red[0][2] + red[0][3]) / (float)H + eps);
  const float ie = 1.0f / sqrtf((red[1][0] + red[1][1] + red[1][2] + red[1][3]) / (float)H + eps);
  T* u = U + (size_t)b * 2 * H;
#pragma unroll
  for (int i = 0; i < MAXC; ++i) {
    const int ch = threadIdx.x + i * 256;
    if (ch < n_ch) {
#pragma unroll
      for (int j = 0; j < EPC; ++j) {
        store_elem(u, (size_t)ch * EPC + j, hv[i][j] * ih);
        store_elem(u, (size_t)H + ch * EPC + j, ev[i][j] * ie);
      }
    }
  }
}

// Work list of the draft block's GEMMs: row block j of mb rows is one item of "expert" 0
// treated as an always-on expert (the GEMM's routed-expert count is 0), so its rows are
// positions j*mb .. and its outputs go to rows j*mb .. of the output buffer.
__global__ void k_draft_plan(int4* __restrict__ work, int32_t* __restrict__ n_work, int B, int mb) {
  const int n = (B + mb - 1) / mb;
  for (int j = threadIdx.x; j < n; j += blockDim.x) work[j] = make_int4(0, j * mb, min(mb, B - j * mb), j * mb);
  if (threadIdx.x == 0) *n_work = n;
}

// The last step's drafts: drafts[b][K-1] = ids[b].
__global__ void k_draft_store(const int32_t* __restrict__ ids, int32_t* __restrict__ drafts, int B, int K) {
  const int b = blockIdx.x * blockDim.x + threadIdx.x;
  if (b < B) drafts[(size_t)b * K + K - 1] = ids[b];
}

__global__ void k_fill(float* __restrict__ p, size_t n, float v) {
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (size_t)gridDim.x * blockDim.x) p[i] = v;
}

hipError_t launch_draft_input(int wdtype, const float* hidden, const int32_t* accepted, const int32_t* committed,
                              int Kv, const float* z_prev, const int32_t* ids_prev, int32_t* drafts, int K, int step,
                              const void* lm, int NKB, int H, int V, float eps, void* U, int B, hipStream_t stream) {
  if (wdtype == 1)
    k_draft_input<uint16_t><<<B, 256, 0, stream>>>(hidden, accepted, committed, Kv, z_prev, ids_prev, drafts, K, step,
                                                   static_cast<const uint4*>(lm), NKB, H, V, eps,
                                                   static_cast<uint16_t*>(U));
  else
    k_draft_input<float><<<B, 256, 0, stream>>>(hidden, accepted, committed, Kv, z_prev, ids_prev, drafts, K, step,
                                                static_cast<const uint4*>(lm), NKB, H, V, eps, static_cast<float*>(U));
  return hipGetLastError();
}

hipError_t launch_draft_plan(int4* work, int32_t* n_work, int B, int mb, hipStream_t stream) {
  k_draft_plan<<<1, 256, 0, stream>>>(work, n_work, B, mb);
  return hipGetLastError();
}

hipError_t launch_draft_store(const int32_t* ids, int32_t* drafts, int B, int K, hipStream_t stream) {
  k_draft_store<<<(B + 255) / 256, 256, 0, stream>>>(ids, drafts, B, K);
  return hipGetLastError();
}

hipError_t launch_fill(float* p, size_t n, float v, hipStream_t stream) {
  k_fill<<<256, 256, 0, stream>>>(p, n, v);
  return hipGetLastError();
}

}  // namespace mv
