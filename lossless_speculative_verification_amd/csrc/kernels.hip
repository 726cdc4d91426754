// gfx950 kernels of the greedy speculative-verification step through an MoE decoder.
//
// Method (pages: "jina-ocr-v1" model page, summary and architecture paragraphs; the
// news page's FastMTP paragraph): every position of the verifier pass runs through
// pre-norm MoE blocks (router softmax, top-6 of 64 routed experts plus 2 shared
// experts, SwiGLU experts, gate-weighted combine), then the LM head and a greedy
// argmax; acceptance keeps the longest prefix of drafts equal to the verifier's
// choices plus the verifier's next token.
//
// Kernel sequence per pass (one HIP stream, no host round trip):
//   per block l: k_norm_route_split / k_norm_route
//                               (combine of block l-1 + residual + RMSNorm + router + top-k)
//                k_plan        (expert-major stable ordering of the T*k routed slots + work
//                               list; built inside k_moe_gemm_planned on small streaming passes)
//                k_moe_gemm_planned / k_moe_gemm<UP> / k_moe_tiled<UP>
//                              (gate/up projections + SwiGLU, MFMA; tiled.hip for large passes)
//                k_moe_gemm<DOWN> / k_moe_tiled<DOWN>
//                              (down projection, one bf16 (or fp32) ybuf row per slot)
//   then         k_norm_route_split (final combine + residual + RMSNorm, no router)
//                k_lm_head / k_moe_tiled<LM>
//                              (LM-head logits tile by tile, top-1/top-2 per tile, never stored;
//                               the tiled form from 256 rows)
//                k_argmax_reduce
//   and          k_accept
#include <climits>

#include "launch.h"
#include "stream_gemm.h"

namespace mv {

// ============================================================================ repack

// Pair layout of a weight matrix set W[mat][N][K] (row-major, `row_bytes` per row).
// Output rows are grouped in tiles of 16, tiles in pairs (the two 16-column tiles one
// wavefront computes), and the contraction in blocks of 256 bytes. Destination unit u
// (16 bytes), u = ((((mat*NQ + q)*NKB + kb)*2 + t)*4 + s)*64 + lane, holds bytes
// [kb*256 + (lane/16)*64 + s*16, +16) of row 16*tile + lane%16, where tile = 2q + t, or,
// for a gate/up pair, tile q of matrix t (t = 0 gate from src0, t = 1 up from src1).
// A wavefront then reads one pair's K block as 8 fully coalesced 1 KB loads.
__global__ void k_repack_pairs(const uint8_t* __restrict__ src0, const uint8_t* __restrict__ src1,
                               uint4* __restrict__ dst, int n_mats, int N, int row_bytes, int NQ, int NKB,
                               int gate_up, size_t mat_stride) {
  const size_t total = (size_t)n_mats * NQ * NKB * kPairUnits;
  for (size_t u = (size_t)blockIdx.x * blockDim.x + threadIdx.x; u < total;
       u += (size_t)gridDim.x * blockDim.x) {
    const int lane = (int)(u % 64);
    size_t r = u / 64;
    const int s = (int)(r % 4);
    r /= 4;
    const int t = (int)(r % 2);
    r /= 2;
    const int kb = (int)(r % NKB);
    r /= NKB;
    const int q = (int)(r % NQ);
    const size_t mat = r / NQ;
    const int tile = gate_up ? q : 2 * q + t;
    const uint8_t* src = (gate_up && t) ? src1 : src0;
    const int n = tile * 16 + (lane & 15);
    uint4 v = make_uint4(0u, 0u, 0u, 0u);
    if (n < N) {
      const uint8_t* p = src + mat * mat_stride + (size_t)n * row_bytes + kb * kRowBlockBytes +
                         (lane >> 4) * 64 + s * 16;
      v = *reinterpret_cast<const uint4*>(p);
    }
    dst[u] = v;
  }
}

// Router layout: unit (l, c, e) = 16 bytes c of router row e of layer l, at index
// (l*chunks + c)*64 + e; rows e >= E are zero. Lane e of a wavefront reads its own
// expert's chunk c, and the 64 lanes together read 1 KB contiguously.
__global__ void k_repack_router(const uint8_t* __restrict__ src, uint4* __restrict__ dst, int L, int E,
                                int row_bytes) {
  const int chunks = row_bytes / 16;
  const size_t total = (size_t)L * chunks * 64;
  for (size_t u = (size_t)blockIdx.x * blockDim.x + threadIdx.x; u < total;
       u += (size_t)gridDim.x * blockDim.x) {
    const int e = (int)(u % 64);
    const size_t r = u / 64;
    const int c = (int)(r % chunks);
    const size_t l = r / chunks;
    uint4 v = make_uint4(0u, 0u, 0u, 0u);
    if (e < E) v = *reinterpret_cast<const uint4*>(src + (l * E + e) * (size_t)row_bytes + (size_t)c * 16);
    dst[u] = v;
  }
}

// ============================================================================ norm + router + top-k

// Four consecutive elements of the element type (float4 index i4) widened to float32.
__device__ __forceinline__ float4 load4(const float* p, size_t i4) { return reinterpret_cast<const float4*>(p)[i4]; }
__device__ __forceinline__ float4 load4(const uint16_t* p, size_t i4) {
  const uint2 w = reinterpret_cast<const uint2*>(p)[i4];
  return make_float4(__uint_as_float(w.x << 16), __uint_as_float(w.x & 0xFFFF0000u), __uint_as_float(w.y << 16),
                     __uint_as_float(w.y & 0xFFFF0000u));
}

// Four consecutive elements (one float4 of the residual row) stored as the element type.
__device__ __forceinline__ void store4(float* p, size_t i4, float4 u) { reinterpret_cast<float4*>(p)[i4] = u; }
__device__ __forceinline__ void store4(uint16_t* p, size_t i4, float4 u) {
  uint2 w;
  w.x = f32_to_bf16(u.x) | (f32_to_bf16(u.y) << 16);
  w.y = f32_to_bf16(u.z) | (f32_to_bf16(u.w) << 16);
  reinterpret_cast<uint2*>(p)[i4] = w;
}
// The same four elements at their place in the stage-ordered row layout (see
// stage_ordered_elem): the four stay together inside one 16-byte chunk.
__device__ __forceinline__ void store4_perm(float* p, size_t i4, float4 u) { store4(p, i4, u); }
__device__ __forceinline__ void store4_perm(uint16_t* p, size_t i4, float4 u) {
  store4(p, stage_ordered_elem((int)i4 * 4) / 4, u);
}

// One workgroup of four wavefronts handles NP consecutive positions; VM float4 per lane
// hold one residual row (H <= 256 * VM).
//  1. (wavefront per position) x = x_in + (g_0 y_0 + ... + g_{k-1} y_{k-1} + y_k + ...
//     + y_{k+S-1}): the previous block's expert outputs of the position's slots, routed
//     ones (rows slot_row[t*k + j], gates topk_w) then shared ones (gate 1), summed in
//     slot order (absent for the first block); x is
//     written back as the residual stream (and to x_copy when given). The slot rows are
//     read SB at a time with all their loads in flight together.
//  2. a = x / sqrt(mean(x^2) + eps), stored in the element type (bf16 rounding) to a_out
//     (in the stage-ordered row layout when perm_a, for the tiled expert GEMM) and, for
//     routing, to LDS.
//  3. (route) router logits for the NP positions as a small MFMA product: wavefront w
//     computes experts 16w..16w+15 against all NP rows (the 16-row MFMA tile repeats
//     row 0 in its unused rows, whose results are dropped), float32 accumulation. The
//     first half of the router weights is requested before step 1, so its latency
//     overlaps the residual reads.
//  4. (route, wavefront per position) logit of expert e in lane e plus its bias; the
//     lane's rank among the 64 (larger logit, then lower index first) is its slot when
//     below k; the gates are the softmax of the selected logits.
// Loads never sit behind a branch (the compiler would then wait for every load in
// flight at the join): indices past the end are clamped and their values masked.
template <typename T, bool ROUTE, int NP, int VM>
__global__ __launch_bounds__(256) void k_norm_route(const float* x_in, const T* __restrict__ ybuf,
                                                    const int32_t* __restrict__ slot_row,
                                                    float* x_out, float* __restrict__ x_copy,
                                                    T* __restrict__ a_out, const uint4* __restrict__ wr,
                                                    const float* __restrict__ bias,
                                                    int32_t* __restrict__ topk_id, float* __restrict__ topk_w,
                                                    int Tn, int H, int S, int E, int k, float eps, int perm_a,
                                                    int pos_major) {
  // Batches of loads in flight: slot rows read together and router K chunks (64 bytes of
  // a row each) per load batch. Small passes (NP = 4) are latency-bound: large batches,
  // the first router batch requested before anything else. Large passes (NP = 16) are
  // throughput-bound: batches small enough for three wavefronts per SIMD.
  constexpr int SB = NP < 16 ? (VM <= 5 ? 8 : 4) : (ROUTE ? 2 : 4);
  constexpr int RB = NP < 16 ? 20 : 8;
  extern __shared__ uint4 lds_raw[];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int H4 = H >> 2;
  const int row_stride = H * (int)sizeof(T) + 16;  // bytes; the pad spreads rows over banks
  char* a_lds = reinterpret_cast<char*>(lds_raw);
  float* r_lds = reinterpret_cast<float*>(a_lds + (size_t)NP * row_stride);

  const int e0 = wave * 16;
  const bool route_wave = ROUTE && e0 < E;
  const int n64 = H * (int)sizeof(T) / 64;
  const uint4* wp = wr + (size_t)(lane >> 4) * kWave + e0 + (lane & 15);
  uint4 wbuf[RB];
  if (route_wave) {
#pragma unroll
    for (int i = 0; i < RB; ++i) wbuf[i] = wp[(size_t)min(i, n64 - 1) * 4 * kWave];
  }

#pragma unroll 1
  for (int p = wave; p < NP; p += kGemmWaves) {
    const int t = blockIdx.x * NP + p;
    if (t >= Tn) continue;
    const float4* xi = reinterpret_cast<const float4*>(x_in) + (size_t)t * H4;
    float4 v[VM];
    if (ybuf) {
      const int KS = k + S;
      float4 m[VM];
#pragma unroll
      for (int j = 0; j < VM; ++j) m[j] = make_float4(0.f, 0.f, 0.f, 0.f);
      for (int s0 = 0; s0 < KS; s0 += SB) {
        float4 y[SB][VM];
        float gt[SB];
#pragma unroll
        for (int s = 0; s < SB; ++s) {
          const int sl = min(s0 + s, KS - 1);  // slot: routed j < k (its gate), then shared (gate 1)
          const int jr = min(sl, k - 1);
          const int rr = pos_major ? 0 : slot_row[(size_t)t * k + jr];
          const float gr = topk_w[(size_t)t * k + jr];
          const size_t row = pos_major ? (size_t)t * KS + sl
                                       : (sl < k ? (size_t)rr : (size_t)Tn * k + (size_t)(sl - k) * Tn + t);
          gt[s] = sl < k ? gr : 1.0f;
#pragma unroll
          for (int j = 0; j < VM; ++j) y[s][j] = load4(ybuf, row * H4 + min(lane + kWave * j, H4 - 1));
        }
#pragma unroll
        for (int s = 0; s < SB; ++s)
#pragma unroll
          for (int j = 0; j < VM; ++j) {
            const bool ok = s0 + s < KS && lane + kWave * j < H4;
            // one fused multiply-add per slot, as in k_combine (same results bit for bit)
            m[j].x = ok ? fmaf(gt[s], y[s][j].x, m[j].x) : m[j].x;
            m[j].y = ok ? fmaf(gt[s], y[s][j].y, m[j].y) : m[j].y;
            m[j].z = ok ? fmaf(gt[s], y[s][j].z, m[j].z) : m[j].z;
            m[j].w = ok ? fmaf(gt[s], y[s][j].w, m[j].w) : m[j].w;
          }
      }
#pragma unroll
      for (int j = 0; j < VM; ++j) {
        const float4 x = xi[min(lane + kWave * j, H4 - 1)];
        v[j] = make_float4(x.x + m[j].x, x.y + m[j].y, x.z + m[j].z, x.w + m[j].w);
      }
    } else {
#pragma unroll
      for (int j = 0; j < VM; ++j) v[j] = xi[min(lane + kWave * j, H4 - 1)];
    }
    float ss = 0.f;
#pragma unroll
    for (int j = 0; j < VM; ++j) {
      const int i = lane + kWave * j;
      if (i < H4) {
        if (x_out) reinterpret_cast<float4*>(x_out)[(size_t)t * H4 + i] = v[j];
        if (x_copy) reinterpret_cast<float4*>(x_copy)[(size_t)t * H4 + i] = v[j];
        ss += v[j].x * v[j].x + v[j].y * v[j].y + v[j].z * v[j].z + v[j].w * v[j].w;
      }
    }
    ss = wave_sum(ss);
    const float inv = 1.0f / sqrtf(ss / (float)H + eps);
    T* lrow = reinterpret_cast<T*>(a_lds + (size_t)p * row_stride);
#pragma unroll
    for (int j = 0; j < VM; ++j) {
      const int i = lane + kWave * j;
      if (i < H4) {
        const float4 u = make_float4(v[j].x * inv, v[j].y * inv, v[j].z * inv, v[j].w * inv);
        if (a_out) {
          if (perm_a) store4_perm(a_out + (size_t)t * H, i, u);
          else store4(a_out + (size_t)t * H, i, u);
        }
        if (ROUTE) store4(lrow, i, u);
      }
    }
  }
  if (!ROUTE) return;
  __syncthreads();

  // Router logits r[p][e] = a_p . W_r[e] for this workgroup's positions.
  if (route_wave) {
    f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
    const int row = (lane & 15) < NP ? (lane & 15) : 0;
    const uint4* arow = reinterpret_cast<const uint4*>(a_lds + (size_t)row * row_stride) + (lane >> 4);
    const uint4 zero = make_uint4(0u, 0u, 0u, 0u);
    for (int c0 = 0; c0 < n64; c0 += RB) {
      if (c0 > 0) {
#pragma unroll
        for (int i = 0; i < RB; ++i) wbuf[i] = wp[(size_t)min(c0 + i, n64 - 1) * 4 * kWave];
      }
#pragma unroll
      for (int i = 0; i < RB; ++i) {
        const bool ok = c0 + i < n64;  // a zero weight chunk adds exactly nothing
        mma_chunk(acc, arow[min(c0 + i, n64 - 1) * 4], ok ? wbuf[i] : zero, (T*)nullptr);
      }
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int p = 4 * (lane >> 4) + i;
      if (p < NP) r_lds[p * 64 + e0 + (lane & 15)] = acc[i];
    }
  }
  __syncthreads();

  const float NEG = -__builtin_huge_valf();
#pragma unroll 1
  for (int p = wave; p < NP; p += kGemmWaves) {
    const int t = blockIdx.x * NP + p;
    if (t >= Tn) continue;
    float* rl = r_lds + p * 64;
    float r = lane < E ? rl[lane] + bias[lane] : NEG;
    if (r != r) r = NEG;  // a NaN logit ranks last, so every selected id stays below E
    // Top-k by rank: lane e's rank is the number of experts ahead of it (a larger logit,
    // or an equal one at a lower index), i.e. its slot when rank < k. The position's 64
    // logits are shared through its LDS row (one wavefront per row; LDS operations of a
    // wavefront complete in order).
    __builtin_amdgcn_wave_barrier();
    rl[lane] = r;
    __builtin_amdgcn_wave_barrier();
    int rank = 0;
    float vmax = NEG;
    const float4* rl4 = reinterpret_cast<const float4*>(rl);
#pragma unroll 4
    for (int j4 = 0; j4 < 16; ++j4) {
      const float4 q = rl4[j4];
      const float qv[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const int j = 4 * j4 + c;
        rank += (qv[c] > r || (qv[c] == r && j < lane)) ? 1 : 0;
        vmax = fmaxf(vmax, qv[c]);
      }
    }
    const bool sel = rank < k;
    const float z = sel ? expf(r - vmax) : 0.f;  // the softmax over the k selected logits
    const float Z = wave_sum(z);
    if (sel) {
      topk_id[(size_t)t * k + rank] = lane;
      topk_w[(size_t)t * k + rank] = z / Z;
    }
  }

}

// Small passes: NP <= 4 positions per workgroup, so the expert-output reads of a pass
// spread over as many compute units as there are positions (one compute unit streams
// only so many bytes per microsecond). Eight wavefronts when routing, four otherwise:
//  * wavefronts 0-3 each own one quarter of the row's float4 columns (VQ per lane). For
//    each position they read the slot rows and the residual with all loads in flight
//    together and form x exactly as k_norm_route does (one fused multiply-add per slot in
//    slot order, then the residual); the sum of squares adds the four quarters' partial
//    sums in quarter order;
//  * wavefronts 4-7 (routing) request their 16 experts' router weights, NC chunks of 64
//    bytes per lane group, as the kernel starts, so those reads overlap the residual
//    reads; once the normalised rows are in LDS they form the logits with the same
//    operands as k_norm_route, chunk c accumulating into the fourth (c mod 4) of four
//    independent MFMA chains that are added at the end;
//  * wavefront p then selects position p's top-k and gates as in k_norm_route (the bias
//    is requested as the kernel starts).
// Workgroup barriers here wait for LDS traffic only: the global stores before them are
// read by later kernels, never inside this one.
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

template <typename T, bool ROUTE, int NP, int VQ, int NC>
__global__ __launch_bounds__(ROUTE ? 512 : 256) void k_norm_route_split(const float* x_in, const T* __restrict__ ybuf,
                                                          const int32_t* __restrict__ slot_row,
                                                          float* x_out, float* __restrict__ x_copy,
                                                          T* __restrict__ a_out, const uint4* __restrict__ wr,
                                                          const float* __restrict__ bias,
                                                          int32_t* __restrict__ topk_id, float* __restrict__ topk_w,
                                                          int Tn, int H, int S, int E, int k, float eps, int perm_a,
                                                    int pos_major) {
  constexpr int SB = 8;  // slot rows per load batch
  static_assert(NC % 8 == 0, "router chunks go in groups of eight");
  extern __shared__ uint4 lds_raw[];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int H4 = H >> 2, Q4 = (H4 + 3) >> 2;
  const int row_stride = H * (int)sizeof(T) + 16;  // bytes; the pad spreads rows over banks
  char* a_lds = reinterpret_cast<char*>(lds_raw);
  float* r_lds = reinterpret_cast<float*>(a_lds + (size_t)NP * row_stride);  // [NP][64] logits
  float* ss_lds = r_lds + NP * 64;                                              // [NP][4] partial sums
  const int n64 = H * (int)sizeof(T) / 64;
  const int t0 = blockIdx.x * NP;
  // the top-k wavefronts request the router bias now, not after the logits
  const float bias_l = ROUTE && wave < NP && lane < E ? bias[lane] : 0.f;

  if (ROUTE && wave >= 4) {  // router wavefronts
    const int e0 = (wave - 4) * 16;
    const bool route_wave = e0 < E;  // wavefront-uniform
    const uint4* wp = wr + (size_t)(lane >> 4) * kWave + e0 + (lane & 15);
    uint4 wbuf[NC];
#pragma unroll
    for (int i = 0; i < NC; ++i) wbuf[i] = wp[(size_t)min(i, n64 - 1) * 4 * kWave];
    lds_barrier();  // sums of squares written
    lds_barrier();  // normalised rows written
    if (route_wave) {
      // chunk c accumulates into acc4[c % 4]: four independent MFMA chains, summed at the end
      f32x4_t acc4[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) acc4[u] = f32x4_t{0.f, 0.f, 0.f, 0.f};
      const int row = (lane & 15) < NP ? (lane & 15) : 0;
      const uint4* arow = reinterpret_cast<const uint4*>(a_lds + (size_t)row * row_stride) + (lane >> 4);
      const uint4 zero = make_uint4(0u, 0u, 0u, 0u);
      // the prefetched chunks, eight LDS row chunks at a time so the row reads do not all
      // wait in registers
      static_for<NC / 8>([&](auto gc) __attribute__((always_inline)) {
        constexpr int g0 = decltype(gc)::value * 8;
        uint4 a[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) a[i] = arow[min(g0 + i, n64 - 1) * 4];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const bool ok = g0 + i < n64;  // a zero weight chunk adds exactly nothing
          mma_chunk(acc4[i % 4], a[i], ok ? wbuf[g0 + i] : zero, (T*)nullptr);
        }
        __builtin_amdgcn_sched_barrier(0);
      });
      // rows longer than NC chunks (float32 weights, wide rows): the rest eight at a time
      for (int c0 = NC; c0 < n64; c0 += 8) {
        uint4 b[8], a[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) b[i] = wp[(size_t)min(c0 + i, n64 - 1) * 4 * kWave];
#pragma unroll
        for (int i = 0; i < 8; ++i) a[i] = arow[min(c0 + i, n64 - 1) * 4];
#pragma unroll
        for (int i = 0; i < 8; ++i) mma_chunk(acc4[i % 4], a[i], c0 + i < n64 ? b[i] : zero, (T*)nullptr);
      }
      f32x4_t acc;
#pragma unroll
      for (int i = 0; i < 4; ++i) acc[i] = (acc4[0][i] + acc4[1][i]) + (acc4[2][i] + acc4[3][i]);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int p = 4 * (lane >> 4) + i;
        if (p < NP) r_lds[p * 64 + e0 + (lane & 15)] = acc[i];
      }
    }
    lds_barrier();  // logits written
  } else {
    const int q0 = wave * Q4;  // this wavefront's first float4 column
    float4 v[NP][VQ];
#pragma unroll
    for (int p = 0; p < NP; ++p) {
      const int t = t0 + p;
      float ss = 0.f;
#pragma unroll
      for (int j = 0; j < VQ; ++j) v[p][j] = make_float4(0.f, 0.f, 0.f, 0.f);
      if (t < Tn) {  // workgroup-uniform
        const float4* xi = reinterpret_cast<const float4*>(x_in) + (size_t)t * H4;
        int col[VQ];
        bool in[VQ];
#pragma unroll
        for (int j = 0; j < VQ; ++j) {
          const int c = lane + kWave * j;
          in[j] = c < Q4 && q0 + c < H4;
          col[j] = in[j] ? q0 + c : 0;
        }
        float4 x[VQ];
#pragma unroll
        for (int j = 0; j < VQ; ++j) x[j] = xi[col[j]];
        if (ybuf) {
              const int KS = k + S;
          float4 m[VQ];
#pragma unroll
          for (int j = 0; j < VQ; ++j) m[j] = make_float4(0.f, 0.f, 0.f, 0.f);
          for (int s0 = 0; s0 < KS; s0 += SB) {
            float4 y[SB][VQ];
            float gt[SB];
#pragma unroll
            for (int s = 0; s < SB; ++s) {
              const int sl = min(s0 + s, KS - 1);  // slot: routed j < k (its gate), then shared (gate 1)
              const int jr = min(sl, k - 1);
              const int rr = pos_major ? 0 : slot_row[(size_t)t * k + jr];
              const float gr = topk_w[(size_t)t * k + jr];
              const size_t row = pos_major ? (size_t)t * KS + sl
                                           : (sl < k ? (size_t)rr : (size_t)Tn * k + (size_t)(sl - k) * Tn + t);
              gt[s] = sl < k ? gr : 1.0f;
#pragma unroll
              for (int j = 0; j < VQ; ++j) y[s][j] = load4(ybuf, row * H4 + col[j]);
            }
#pragma unroll
            for (int s = 0; s < SB; ++s)
#pragma unroll
              for (int j = 0; j < VQ; ++j) {
                const bool ok = s0 + s < KS;
                m[j].x = ok ? fmaf(gt[s], y[s][j].x, m[j].x) : m[j].x;
                m[j].y = ok ? fmaf(gt[s], y[s][j].y, m[j].y) : m[j].y;
                m[j].z = ok ? fmaf(gt[s], y[s][j].z, m[j].z) : m[j].z;
                m[j].w = ok ? fmaf(gt[s], y[s][j].w, m[j].w) : m[j].w;
              }
          }
#pragma unroll
          for (int j = 0; j < VQ; ++j)
            x[j] = make_float4(x[j].x + m[j].x, x[j].y + m[j].y, x[j].z + m[j].z, x[j].w + m[j].w);
        }
#pragma unroll
        for (int j = 0; j < VQ; ++j) {
          if (in[j]) {
            v[p][j] = x[j];
            if (x_out) reinterpret_cast<float4*>(x_out)[(size_t)t * H4 + col[j]] = x[j];
            if (x_copy) reinterpret_cast<float4*>(x_copy)[(size_t)t * H4 + col[j]] = x[j];
            ss += x[j].x * x[j].x + x[j].y * x[j].y + x[j].z * x[j].z + x[j].w * x[j].w;
          }
        }
      }
      ss = wave_sum(ss);
      if (lane == 0) ss_lds[p * 4 + wave] = ss;
    }
    lds_barrier();  // sums of squares written
#pragma unroll
    for (int p = 0; p < NP; ++p) {
      const int t = t0 + p;
      if (t >= Tn) continue;
      const float ss = ((ss_lds[p * 4] + ss_lds[p * 4 + 1]) + ss_lds[p * 4 + 2]) + ss_lds[p * 4 + 3];
      const float inv = 1.0f / sqrtf(ss / (float)H + eps);
      T* lrow = reinterpret_cast<T*>(a_lds + (size_t)p * row_stride);
#pragma unroll
      for (int j = 0; j < VQ; ++j) {
        const int c = lane + kWave * j;
        if (c < Q4 && q0 + c < H4) {
          const int i = q0 + c;
          const float4 u = make_float4(v[p][j].x * inv, v[p][j].y * inv, v[p][j].z * inv, v[p][j].w * inv);
          if (a_out) {
            if (perm_a) store4_perm(a_out + (size_t)t * H, i, u);
            else store4(a_out + (size_t)t * H, i, u);
          }
          if (ROUTE) store4(lrow, i, u);
        }
      }
    }
    if (ROUTE) {
      lds_barrier();  // normalised rows written
      lds_barrier();  // logits written
    }
  }
  if (!ROUTE || wave >= NP) return;

  // wavefront p: top-k of position p, as in k_norm_route
  const int p = wave, t = t0 + p;
  if (t >= Tn) return;
  const float NEG = -__builtin_huge_valf();
  float* rl = r_lds + p * 64;
  float r = lane < E ? rl[lane] + bias_l : NEG;
  if (r != r) r = NEG;
  __builtin_amdgcn_wave_barrier();
  rl[lane] = r;
  __builtin_amdgcn_wave_barrier();
  int rank = 0;
  float vmax = NEG;
  const float4* rl4 = reinterpret_cast<const float4*>(rl);
#pragma unroll 4
  for (int j4 = 0; j4 < 16; ++j4) {
    const float4 q = rl4[j4];
    const float qv[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const int j = 4 * j4 + c;
      rank += (qv[c] > r || (qv[c] == r && j < lane)) ? 1 : 0;
      vmax = fmaxf(vmax, qv[c]);
    }
  }
  const bool sel = rank < k;
  const float z = sel ? expf(r - vmax) : 0.f;
  const float Z = wave_sum(z);
  if (sel) {
    topk_id[(size_t)t * k + rank] = lane;
    topk_w[(size_t)t * k + rank] = z / Z;
  }
}

// ============================================================================ routing plan

// The routing plan orders the T*k routed slots (slot = t*k + j) by expert, stably
// (ascending slot within an expert), and lists the GEMM work items. Routed rows occupy
// [0, T*k) of the row space in that order; shared expert s owns rows T*k + s*T + t.
// Work items (expert, first row, rows, first token) have at most pa.mb rows: each shared
// expert's position blocks first (so the blocks of one shared expert are neighbours in
// the item list), then the routed experts' row blocks in expert order.
//
// Building blocks, for a workgroup of NW wavefronts that owns slots [beg, end):
//  seg_hist:    per-wavefront expert histograms of NW contiguous sub-segments;
//  seg_cursors: exclusive scan in (expert, sub-segment) order from the per-expert write
//               base of the workgroup's range -> each sub-segment's write cursor;
//  seg_scatter: each wavefront places its sub-segment 64 slots at a time; lanes with the
//               same expert are found with six ballots over the expert id bits, and a
//               lane's rank is the count of lower lanes in its group.
// One workgroup plans a small pass alone (k_plan); a large pass is cut into chunks whose
// expert counts are taken first (k_plan_count), after which every chunk knows its write
// base and is placed by its own workgroup (k_plan_scatter).

constexpr int kPlanBatch = 8;  // slots per lane whose loads are in flight together

template <int NW>
__device__ void seg_hist(const PlanArgs& pa, int beg, int end, int (*hist)[64]) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int N = pa.Tn * pa.k;
  hist[wave][lane] = 0;
  __syncthreads();
  const int seg = (end - beg + NW - 1) / NW;
  const int b = min(end, beg + wave * seg), e = min(end, b + seg);
  for (int b0 = b; b0 < e; b0 += kPlanBatch * kWave) {
    int key[kPlanBatch];
#pragma unroll
    for (int u = 0; u < kPlanBatch; ++u) key[u] = pa.topk_id[min(b0 + u * kWave + lane, N - 1)];
#pragma unroll
    for (int u = 0; u < kPlanBatch; ++u)
      if (b0 + u * kWave + lane < e) atomicAdd(&hist[wave][min(max(key[u], 0), pa.E - 1)], 1);
  }
  __syncthreads();
}

// Wavefront 0, lane = expert: hist[w][e] becomes sub-segment w's first row for expert e.
template <int NW>
__device__ void seg_cursors(int (*hist)[64], int base) {
  int run = base;
  for (int w = 0; w < NW; ++w) {
    const int h = hist[w][threadIdx.x];
    hist[w][threadIdx.x] = run;
    run += h;
  }
}

template <int NW>
__device__ void seg_scatter(const PlanArgs& pa, int beg, int end, int (*hist)[64]) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int N = pa.Tn * pa.k, k = pa.k;
  const int seg = (end - beg + NW - 1) / NW;
  const int b = min(end, beg + wave * seg), e = min(end, b + seg);
  for (int b0 = b; b0 < e; b0 += kPlanBatch * kWave) {
    int keys[kPlanBatch];
#pragma unroll
    for (int u = 0; u < kPlanBatch; ++u) keys[u] = pa.topk_id[min(b0 + u * kWave + lane, N - 1)];
#pragma unroll
    for (int u = 0; u < kPlanBatch; ++u) {
      const int i = b0 + u * kWave + lane;
      if (b0 + u * kWave >= e) break;  // wavefront-uniform
      const bool active = i < e;
      const int key = active ? min(max(keys[u], 0), pa.E - 1) : 0;  // ids come from k_norm_route, always < E
      unsigned long long mask = __ballot(active);
#pragma unroll
      for (int bit = 0; bit < 6; ++bit) {
        const bool on = (key >> bit) & 1;
        const unsigned long long bal = __ballot(on);
        mask &= on ? bal : ~bal;
      }
      const int rank = __popcll(mask & ((1ull << lane) - 1ull));
      const int cnt = __popcll(mask);
      int pos = 0;
      if (active) pos = hist[wave][key] + rank;
      __builtin_amdgcn_wave_barrier();
      if (active) {
        const int tok = i / k, j = i - tok * k;
        pa.row_tok[pos] = tok;
        pa.slot_row[i] = pos;
        pa.row_dst[pos] = tok * (k + pa.S) + j;
        if (rank == cnt - 1) hist[wave][key] = pos + 1;
      }
      __builtin_amdgcn_wave_barrier();
    }
  }
}

// Wavefront 0, lane = expert, holding the expert's routed-row count c: first rows (off)
// and first work items (wstart) by inclusive lane scans, per-expert counts out.
__device__ void expert_offsets(const PlanArgs& pa, int c, int* off, int* wstart, bool write_counts) {
  const int lane = threadIdx.x & 63;
  const int nb = (c + pa.mb - 1) / pa.mb;
  int sc = c, sn = nb;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int oc = __shfl_up(sc, d, kWave), on = __shfl_up(sn, d, kWave);
    if (lane >= d) { sc += oc; sn += on; }
  }
  off[lane] = sc - c;
  wstart[lane] = sn - nb;
  if (write_counts && lane < pa.E) pa.counts[lane] = c;
  if (lane == 63) { off[64] = sc; wstart[64] = sn; }
}

// Work items from the expert offsets (any number of threads).
__device__ void write_work(const PlanArgs& pa, const int* off, const int* wstart, int nthreads) {
  const int tid = threadIdx.x, mb = pa.mb, Tn = pa.Tn, N = pa.Tn * pa.k;
  const int mbT = (Tn + mb - 1) / mb;
  const int nsw = pa.S * mbT;  // shared-expert items come first
  for (int idx = tid; idx < nsw; idx += nthreads) {
    const int s = idx / mbT, b = idx - s * mbT;
    pa.work[idx] = make_int4(pa.E + s, N + s * Tn + b * mb, min(mb, Tn - b * mb), b * mb);
  }
  for (int e = tid; e < pa.E; e += nthreads) {  // one thread per expert
    const int c = off[e + 1] - off[e];
    for (int b = 0; b * mb < c; ++b)
      pa.work[nsw + wstart[e] + b] = make_int4(e, off[e] + b * mb, min(mb, c - b * mb), 0);
  }
  if (tid == 0) *pa.n_work = nsw + wstart[64];
}

// Split plan (pa.hot_rows > 0): wavefront 0, lane = expert with c rows: items of a hot
// expert (c >= hot_rows) in the tiled list (first items wstart), of a cold one in the
// streaming list (first items wstart2, mb2 rows each).
__device__ void split_starts(const PlanArgs& pa, int c, int* wstart, int* wstart2) {
  const int lane = threadIdx.x & 63;
  const bool hot = c >= pa.hot_rows;
  const int nb = hot ? (c + pa.mb - 1) / pa.mb : 0, nb2 = hot ? 0 : (c + pa.mb2 - 1) / pa.mb2;
  int sn = nb, sn2 = nb2;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int o = __shfl_up(sn, d, kWave), o2 = __shfl_up(sn2, d, kWave);
    if (lane >= d) { sn += o; sn2 += o2; }
  }
  wstart[lane] = sn - nb;
  wstart2[lane] = sn2 - nb2;
  if (lane == 63) { wstart[64] = sn; wstart2[64] = sn2; }
}

__device__ void write_work_split(const PlanArgs& pa, const int* off, const int* wstart, const int* wstart2,
                                 int nthreads) {
  const int tid = threadIdx.x, mb = pa.mb, mb2 = pa.mb2, Tn = pa.Tn, N = pa.Tn * pa.k;
  const int mbT = (Tn + mb - 1) / mb;
  const int nsw = pa.S * mbT;  // shared-expert items come first
  for (int idx = tid; idx < nsw; idx += nthreads) {
    const int s = idx / mbT, b = idx - s * mbT;
    pa.work[idx] = make_int4(pa.E + s, N + s * Tn + b * mb, min(mb, Tn - b * mb), b * mb);
  }
  for (int e = tid; e < pa.E; e += nthreads) {  // one thread per expert
    const int c = off[e + 1] - off[e];
    if (c >= pa.hot_rows) {
      for (int b = 0; b * mb < c; ++b)
        pa.work[nsw + wstart[e] + b] = make_int4(e, off[e] + b * mb, min(mb, c - b * mb), 0);
    } else {
      for (int b = 0; b * mb2 < c; ++b)
        pa.work2[wstart2[e] + b] = make_int4(e, off[e] + b * mb2, min(mb2, c - b * mb2), 0);
    }
  }
  if (tid == 0) {
    *pa.n_work = nsw + wstart[64];
    *pa.n_work2 = wstart2[64];
  }
}

__global__ __launch_bounds__(1024) void k_plan(PlanArgs pa) {
  constexpr int NW = 16;
  __shared__ int hist[NW][64];
  __shared__ int off[65];
  __shared__ int wstart[65];
  __shared__ int wstart2[65];
  const int N = pa.Tn * pa.k;
  seg_hist<NW>(pa, 0, N, hist);
  if (threadIdx.x < kWave) {
    int c = 0;
    if ((int)threadIdx.x < pa.E)
      for (int w = 0; w < NW; ++w) c += hist[w][threadIdx.x];
    expert_offsets(pa, c, off, wstart, true);
    if (pa.hot_rows > 0) split_starts(pa, (int)threadIdx.x < pa.E ? c : 0, wstart, wstart2);
    seg_cursors<NW>(hist, off[threadIdx.x]);
  }
  __syncthreads();
  seg_scatter<NW>(pa, 0, N, hist);
  if (pa.hot_rows > 0) write_work_split(pa, off, wstart, wstart2, NW * kWave);
  else write_work(pa, off, wstart, NW * kWave);
}

// Large pass, step 1: chunk c's routed-slot count per expert -> chunk_cnt[c][64].
__global__ __launch_bounds__(256) void k_plan_count(PlanArgs pa) {
  constexpr int NW = 4;
  __shared__ int hist[NW][64];
  const int N = pa.Tn * pa.k;
  const int beg = min(N, (int)blockIdx.x * kPlanChunk), end = min(N, beg + kPlanChunk);
  seg_hist<NW>(pa, beg, end, hist);
  if (threadIdx.x < 64) {
    int c = 0;
    for (int w = 0; w < NW; ++w) c += hist[w][threadIdx.x];
    pa.chunk_cnt[blockIdx.x * 64 + threadIdx.x] = c;
  }
}

// Large pass, step 2: chunk c's write base per expert is the expert's first row plus the
// counts of chunks < c; workgroup 0 also writes the per-expert counts and the work list.
__global__ __launch_bounds__(256) void k_plan_scatter(PlanArgs pa) {
  constexpr int NW = 4;
  __shared__ int hist[NW][64];
  __shared__ int off[65];
  __shared__ int wstart[65];
  const int N = pa.Tn * pa.k;
  const int beg = min(N, (int)blockIdx.x * kPlanChunk), end = min(N, beg + kPlanChunk);
  seg_hist<NW>(pa, beg, end, hist);
  if (threadIdx.x < kWave) {
    const int e = threadIdx.x, G = (int)gridDim.x;
    int tot = 0, pre = 0;
    // the chunks' counts kPlanBatch at a time, all their loads in flight together
    for (int c0 = 0; c0 < G; c0 += kPlanBatch) {
      int v[kPlanBatch];
#pragma unroll
      for (int u = 0; u < kPlanBatch; ++u) v[u] = pa.chunk_cnt[min(c0 + u, G - 1) * 64 + e];
#pragma unroll
      for (int u = 0; u < kPlanBatch; ++u) {
        const int c = c0 + u;
        tot += c < G ? v[u] : 0;
        pre += c < (int)blockIdx.x ? v[u] : 0;
      }
    }
    if (e >= pa.E) tot = 0;
    expert_offsets(pa, tot, off, wstart, blockIdx.x == 0);
    seg_cursors<NW>(hist, off[e] + pre);
  }
  __syncthreads();
  seg_scatter<NW>(pa, beg, end, hist);
  if (blockIdx.x == 0) write_work(pa, off, wstart, NW * kWave);
}

// ============================================================================ grouped MFMA GEMM

// Expert GEMM over the device-built work list, PPW = g.ppw pairs per wavefront (chosen
// on the host from the position count). Exactly the workgroups that carry work come
// first (the grid is sized for the list's capacity; the rest leave at once), so all of
// them are resident together; logical workgroups are laid out XCD by XCD (xcd_logical),
// so the chunks of one item, and neighbouring items such as the row blocks of one
// shared expert, share one L2. Logical wavefront lw takes chunk c = lw % chunks (pairs
// [c*PPW, c*PPW + PPW)) of item lw / chunks.
template <typename T, int EPI, int NMT, int D, int WPG>
__global__ __launch_bounds__(kWave * WPG, MV_GEMM_WAVES_PER_SIMD) void k_moe_gemm(GemmArgs g) {
  const int chunks = (g.NQ + g.ppw - 1) / g.ppw;
  const int n_items = *g.n_work;
  const int n_wg = (n_items * chunks + WPG - 1) / WPG;
  if ((int)blockIdx.x >= n_wg) return;  // workgroup-uniform
  const int lw = xcd_logical((int)blockIdx.x, n_wg) * WPG + (threadIdx.x >> 6);
  const int item = lw / chunks, c = lw - item * chunks;
  if (item >= n_items) return;  // no barrier in this kernel
  const int4 it = g.work[item];
  const int q0 = c * g.ppw;
  const bool one_tile = NMT > 1 && it.z <= 16;
  if (g.ppw == 2) {
    if (one_tile) moe_stream<T, EPI, 1, 2, D>(g, it.x, it.y, it.z, it.w, q0);
    else moe_stream<T, EPI, NMT, 2, D>(g, it.x, it.y, it.z, it.w, q0);
  } else {
    if (one_tile) moe_stream<T, EPI, 1, 1, D + 1>(g, it.x, it.y, it.z, it.w, q0);
    else moe_stream<T, EPI, NMT, 1, D + 1>(g, it.x, it.y, it.z, it.w, q0);
  }
}

// Gate/up expert GEMM of the streaming path that builds the routing plan itself, so that
// no plan kernel runs between the norm/router kernel and this one. Every workgroup
// computes the same plan from the N = T*k routed ids (at most kSelfPlanMaxSlots):
// per-expert counts by LDS histogram, then, in wavefront 0, the items per expert
// (ceil(count / mb)) and the expert's first row, by lane scans; the item order, row space
// and row order are those of k_plan (shared experts' position blocks first, then the
// routed experts' row blocks in expert order; an expert's slots in ascending slot order).
// A wavefront then finds its item as in k_moe_gemm, compacts its expert's slots of rank
// [b*mb, b*mb + M) with ballots into LDS (tokens for the activation rows, slot ids for
// row_dst), and runs moe_stream. The item's chunk-0 wavefront writes the work item and the
// rows' position-major ybuf rows for the down GEMM; workgroup 0 writes the item count and
// the per-expert counts.
template <typename T, int NMT, int D, int WPG>
__global__ __launch_bounds__(kWave * WPG, MV_GEMM_WAVES_PER_SIMD) void k_moe_gemm_planned(GemmArgs g) {
  __shared__ int ids[kSelfPlanMaxSlots];
  __shared__ int hist[kWave];
  __shared__ int first_item[kWave + 1];  // routed expert e's items start at first_item[e]
  __shared__ int first_row[kWave];       // and its rows at first_row[e]
  __shared__ int rows[WPG][2][16 * NMT];  // per wavefront: tokens and slots of its item's rows
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int N = g.Tn * g.k, E = g.E, mb = g.mb;
  const int S = g.KS - g.k;
  const int mbT = (g.Tn + mb - 1) / mb, nsw = S * mbT;  // shared-expert items come first
  for (int i = threadIdx.x; i < kWave; i += blockDim.x) hist[i] = 0;
  __syncthreads();
  for (int i0 = 0; i0 < N; i0 += 4 * (int)blockDim.x) {
    int id[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) id[u] = g.topk_id[min(i0 + u * (int)blockDim.x + (int)threadIdx.x, N - 1)];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int i = i0 + u * (int)blockDim.x + (int)threadIdx.x;
      if (i < N) {
        const int e = min(max(id[u], 0), E - 1);  // ids come from the router, always < E
        ids[i] = e;
        atomicAdd(&hist[e], 1);
      }
    }
  }
  __syncthreads();
  if (wave == 0) {
    const int c = lane < E ? hist[lane] : 0;
    const int nb = (c + mb - 1) / mb;
    int sc = c, sn = nb;
#pragma unroll
    for (int d = 1; d < kWave; d <<= 1) {
      const int oc = __shfl_up(sc, d, kWave), on = __shfl_up(sn, d, kWave);
      if (lane >= d) { sc += oc; sn += on; }
    }
    first_row[lane] = sc - c;
    first_item[lane] = nsw + sn - nb;
    if (lane == kWave - 1) first_item[kWave] = nsw + sn;
    if (blockIdx.x == 0 && lane < E) g.plan_counts[lane] = c;
  }
  __syncthreads();
  const int n_items = first_item[kWave];
  if (blockIdx.x == 0 && threadIdx.x == 0) *g.plan_n_work = n_items;
  const int chunks = (g.NQ + g.ppw - 1) / g.ppw;
  const int n_wg = (n_items * chunks + WPG - 1) / WPG;
  if ((int)blockIdx.x >= n_wg) return;  // workgroup-uniform
  const int lw = xcd_logical((int)blockIdx.x, n_wg) * WPG + wave;
  const int item = lw / chunks, c = lw - item * chunks;
  if (item >= n_items) return;  // no barrier from here on
  int e, row0, M, tok0;
  int* tok_rows = rows[wave][0];
  int* slot_rows = rows[wave][1];
  if (item < nsw) {
    const int s = item / mbT, b = item - s * mbT;
    e = E + s; row0 = N + s * g.Tn + b * mb; M = min(mb, g.Tn - b * mb); tok0 = b * mb;
  } else {
    // the routed expert whose items contain this one: the last e with first_item[e] <= item
    const unsigned long long le = __ballot(lane < E && first_item[lane] <= item);
    e = 63 - __clzll(le);
    const int b = item - first_item[e];
    const int cnt = hist[e];
    row0 = first_row[e] + b * mb; M = min(mb, cnt - b * mb); tok0 = 0;
    // the expert's slots of rank [b*mb, b*mb + M), 64 ids at a time, in slot order
    int base = 0;
    for (int i0 = 0; i0 < N && base < b * mb + M; i0 += kWave) {  // wavefront-uniform
      const int i = i0 + lane;
      const bool hit = i < N && ids[i] == e;
      const unsigned long long m = __ballot(hit);
      const int r = base + __popcll(m & ((1ull << lane) - 1ull)) - b * mb;
      if (hit && r >= 0 && r < M) {
        tok_rows[r] = i / g.k;
        slot_rows[r] = i;
      }
      base += __popcll(m);
    }
    __builtin_amdgcn_wave_barrier();
  }
  if (c == 0) {  // the item's first chunk publishes it for the down GEMM
    if (lane == 0) g.plan_work[item] = make_int4(e, row0, M, tok0);
    if (e < E && lane < M) {
      const int i = slot_rows[lane];
      g.plan_row_dst[row0 + lane] = (i / g.k) * g.KS + (i - (i / g.k) * g.k);
    }
  }
  const int q0 = c * g.ppw;
  const bool one_tile = NMT > 1 && M <= 16;
  if (g.ppw == 2) {
    if (one_tile) moe_stream<T, EPI_UP, 1, 2, D>(g, e, row0, M, tok0, q0, tok_rows);
    else moe_stream<T, EPI_UP, NMT, 2, D>(g, e, row0, M, tok0, q0, tok_rows);
  } else {
    if (one_tile) moe_stream<T, EPI_UP, 1, 1, D + 1>(g, e, row0, M, tok0, q0, tok_rows);
    else moe_stream<T, EPI_UP, NMT, 1, D + 1>(g, e, row0, M, tok0, q0, tok_rows);
  }
}

// LM head. A workgroup of kLmWaves wavefronts (one workgroup per compute unit) covers
// kLmWaves*ppw consecutive column pairs (wavefront w: pairs w*ppw ..) for one row block of
// up to 16*NMT <= kLmRows positions, so every weight byte is read once per row block (at
// most 128 positions need one row block). The block's rows are staged once per K block for
// all the workgroup's wavefronts: eight wavefronts per compute unit in one workgroup read
// half the activation bytes that two workgroups of four would.
// The block's normalised rows are staged in LDS one 256-byte K block at a time (double
// buffered, read one K block ahead in registers) and shared by the 4 wavefronts.
// Weights stream as in moe_stream, two K blocks in flight; no load in the main loop
// depends on a branch.
// The MFMA computes the transposed tile (weights as the first operand, positions as the
// second), so lane l holds, for position 16*mt + l%16, the logits of columns
// 32q + 4*(l/16) + i and 32q + 16 + 4*(l/16) + i (i = 0..3) of pair q. Each lane folds
// them, in increasing column order, into one running (top-1 value, lowest index, top-2
// value) record per row tile; only at the end are the records merged across the four
// lane groups and then across the 4 wavefronts, and one record per position and
// workgroup goes to part.
template <typename T, int NMT>
__device__ __forceinline__ void lm_stream(const GemmArgs& g, int row0, int M, int pg, int ppw,
                                          uint4 (*As)[kLmRows][kChunksPerRow + 1],
                                          Top2 (*red)[kLmRows]) {
  constexpr int MB = NMT * 16;
  constexpr int NTH = kLmWaves * kWave;
  constexpr int RPS = NTH / kChunksPerRow;           // rows one staging pass covers
  constexpr int AL = (MB + RPS - 1) / RPS;            // 16-byte A chunks per thread per K block
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int row_units = g.K * (int)sizeof(T) / 16;
  const int NKB = row_units / kChunksPerRow;
  const int q0 = (pg * kLmWaves + wave) * ppw;
  const float NEG = -__builtin_huge_valf();
  const int F = ppw * NKB;

  // A staging: thread -> (row srow + RPS*j, chunk schunk) of the K block; AL chunks (the
  // threads past a small block's last row stage nothing).
  const int srow = threadIdx.x >> 4, schunk = threadIdx.x & 15;
  const u32x4_t* abase = reinterpret_cast<const u32x4_t*>(g.A) + schunk;
  int aoff[AL];  // 16-byte offset of each staged row (a block's rows past M repeat its first)
#pragma unroll
  for (int j = 0; j < AL; ++j) {
    const int r = srow + RPS * j;
    aoff[j] = (row0 + (r < M ? r : 0)) * row_units;
  }
  // A block f+1 waits in ra while block f is in LDS.
  u32x4_t ra[AL];
  int fa = 0, ka = 0;  // next A block: flat index (stops at the last) and K block in the row
  auto read_a = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int j = 0; j < AL; ++j) ra[j] = abase[aoff[j] + ka * kChunksPerRow];
    const bool adv = fa < F - 1;
    fa += adv ? 1 : 0;
    ka = adv ? (ka + 1 == NKB ? 0 : ka + 1) : ka;
  };
  auto write_a = [&](int buf) __attribute__((always_inline)) {
#pragma unroll
    for (int j = 0; j < AL; ++j)
      if (srow + RPS * j < MB) *reinterpret_cast<u32x4_t*>(&As[buf][srow + RPS * j][schunk]) = ra[j];
  };

  // Pairs past the vocabulary's last pair stream a copy of it; their columns are masked.
  const uint4* Bw = g.B + (size_t)min(q0, g.NQ - 1) * NKB * kPairUnits + lane;
  const int nq_real = max(0, min(ppw, g.NQ - q0));
  const int FB = max(1, nq_real) * NKB;  // K blocks with distinct weights for this wavefront
  uint4 rb[2][8];
  int fl = 0;
  auto load_b = [&](uint4(&b)[8]) __attribute__((always_inline)) {
#pragma unroll
    for (int u = 0; u < 8; ++u) b[u] = load_stream(Bw + (size_t)fl * kPairUnits + u * kWave);
    fl += fl < FB - 1 ? 1 : 0;
  };

  f32x4_t acc[NMT][2];
  Top2 best[NMT];  // running record of position 16*mt + lane%16 over this lane's columns
#pragma unroll
  for (int mt = 0; mt < NMT; ++mt) acc[mt][0] = acc[mt][1] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int mt = 0; mt < NMT; ++mt) best[mt] = Top2{NEG, INT_MAX, NEG};
  auto compute = [&](int buf, const uint4(&b)[8]) __attribute__((always_inline)) {
#pragma unroll
    for (int s = 0; s < 4; ++s)
#pragma unroll
      for (int mt = 0; mt < NMT; ++mt) {
        const uint4 a = As[buf][mt * 16 + (lane & 15)][(lane >> 4) * 4 + s];
        mma_chunk(acc[mt][0], b[s], a, (T*)nullptr);
        mma_chunk(acc[mt][1], b[4 + s], a, (T*)nullptr);
      }
  };
  auto fold = [&](int q) __attribute__((always_inline)) {  // fold the finished pair q into the running records
    const int cb = 2 * q * 16 + 4 * (lane >> 4);
    const bool full = (2 * q + 2) * 16 <= g.n_valid;  // every column of the pair is a word
#pragma unroll
    for (int mt = 0; mt < NMT; ++mt) {
      Top2 b = best[mt];
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int i = 0; i < 4; ++i) {  // columns in increasing order: a later equal value never wins
          const int c = cb + 16 * t + i;
          top2_push(b, (full | ((q < g.NQ) & (c < g.n_valid))) ? acc[mt][t][i] : NEG, c);
        }
      best[mt] = b;
    }
#pragma unroll
    for (int mt = 0; mt < NMT; ++mt) acc[mt][0] = acc[mt][1] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  };

  // prologue: A block 0 into LDS, block 1 into registers; B blocks 0 and 1. In every
  // step the activation read goes out before the weight loads: waits are in issue
  // order, so waiting for the activations then never waits for the newest weights.
  read_a();
  write_a(0);
  read_a();
  load_b(rb[0]);
  load_b(rb[1]);
  __syncthreads();
  // Pair by pair, two K blocks per step (NKB is even, so LDS buffer and B register set
  // of block kb are both kb & 1). Every load in the steps is in range: the last two
  // blocks of the last pair are done apart, loading no weights. Activation reads past
  // the last block repeat it (they are L2 hits and feed nothing).
  for (int qi = 0; qi < ppw; ++qi) {
    const bool last = qi == ppw - 1;
    const int kend = last ? NKB - 2 : NKB;
    for (int kb0 = 0; kb0 < kend; kb0 += 2) {
      static_for<2>([&](auto sc) __attribute__((always_inline)) {
        constexpr int s = decltype(sc)::value;
        compute(s, rb[s]);
        write_a(s ^ 1);
        read_a();
        load_b(rb[s]);
        __syncthreads();
      });
    }
    if (last) {
      static_for<2>([&](auto sc) __attribute__((always_inline)) {
        constexpr int s = decltype(sc)::value;
        compute(s, rb[s]);
        if (s == 0) write_a(1);
        __syncthreads();
      });
    }
    fold(q0 + qi);
  }

  // merge the four lane groups' records of each position; lanes 0-15 then hold them
#pragma unroll
  for (int mt = 0; mt < NMT; ++mt) {
    Top2 b = best[mt];
    b = top2_merge(b, top2_shfl_xor(b, 16));
    b = top2_merge(b, top2_shfl_xor(b, 32));
    if (lane < 16) red[wave][mt * 16 + lane] = b;
  }
  __syncthreads();
  if ((int)threadIdx.x < M) {
    const int r = threadIdx.x;
    Top2 rec = red[0][r];
#pragma unroll
    for (int w = 1; w < kLmWaves; ++w) rec = top2_merge(rec, red[w][r]);
    g.part[(size_t)(row0 + r) * g.n_pg + pg] = rec;
  }
}

template <typename T>
__global__ __launch_bounds__(kLmWaves * kWave, 1) void k_lm_head(GemmArgs g) {
  __shared__ uint4 As[2][kLmRows][kChunksPerRow + 1];
  __shared__ Top2 red[kLmWaves][kLmRows];
  const int n_items = (g.Tn + kLmRows - 1) / kLmRows;
  const int n = n_items * g.n_pg;
  if ((int)blockIdx.x >= n) return;  // workgroup-uniform
  // column-group major: the row blocks of one column group are logical neighbours, so
  // they run side by side on one XCD and share its weight stream through L2
  const int L = xcd_logical((int)blockIdx.x, n);
  const int pg = L / n_items, item = L - pg * n_items;
  const int row0 = item * kLmRows, M = min(kLmRows, g.Tn - row0);
  const int ppw = g.lm_ppw;
  if (M <= 16) lm_stream<T, 1>(g, row0, M, pg, ppw, As, red);
  else if (M <= 32) lm_stream<T, 2>(g, row0, M, pg, ppw, As, red);
  else if (M <= 64) lm_stream<T, 4>(g, row0, M, pg, ppw, As, red);
  else lm_stream<T, 8>(g, row0, M, pg, ppw, As, red);
}

// ============================================================================ argmax, accept, combine

// One wavefront per position merges the per-workgroup records (exact max operations,
// so the merge order does not matter) into the greedy id and the top-1/top-2 margin.
__global__ __launch_bounds__(256) void k_argmax_reduce(const Top2* __restrict__ part, int n_pg, int Tn,
                                                       int32_t* __restrict__ argmax, float* __restrict__ margin) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + wave;
  if (t >= Tn) return;
  const float NEG = -__builtin_huge_valf();
  constexpr int RB = 8;  // records per lane requested together
  Top2 rec{NEG, INT_MAX, NEG};
  const Top2* row = part + (size_t)t * n_pg;
  for (int p0 = 0; p0 < n_pg; p0 += RB * kWave) {
    Top2 r[RB];
#pragma unroll
    for (int u = 0; u < RB; ++u) r[u] = row[min(p0 + u * kWave + lane, n_pg - 1)];
#pragma unroll
    for (int u = 0; u < RB; ++u)  // past the end: the loaded record would count twice, so it is skipped
      if (p0 + u * kWave + lane < n_pg) rec = top2_merge(rec, r[u]);
  }
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) rec = top2_merge(rec, top2_shfl_xor(rec, m));
  if (lane == 0) {
    argmax[t] = rec.i1;
    if (margin) margin[t] = rec.v1 - rec.v2;
  }
}

// Greedy acceptance, one thread per sequence: count leading drafts equal to the
// verifier's choice at the same position; commit the verifier's choices 0..n.
__global__ void k_accept(const int32_t* __restrict__ drafts, const int32_t* __restrict__ argmax, int B, int K,
                         int32_t* __restrict__ accepted, int32_t* __restrict__ committed) {
  const int b = blockIdx.x * blockDim.x + threadIdx.x;
  if (b >= B) return;
  const int32_t* y = argmax + (size_t)b * (K + 1);
  int n = 0;
  while (n < K && drafts[(size_t)b * K + n] == y[n]) ++n;
  accepted[b] = n;
  for (int i = 0; i <= K; ++i) committed[(size_t)b * (K + 1) + i] = i <= n ? y[i] : -1;
}

// m[t] = sum_j gate_j * y(t, j) in slot order (the block output before the residual add).
template <typename T>
__global__ void k_combine(const T* __restrict__ ybuf, const int32_t* __restrict__ slot_row,
                          const float* __restrict__ gate, int Tn, int H, int k, int S, int pos_major,
                          float* __restrict__ m) {
  const int H4 = H >> 2;
  const size_t total = (size_t)Tn * H4;
  for (size_t u = (size_t)blockIdx.x * blockDim.x + threadIdx.x; u < total; u += (size_t)gridDim.x * blockDim.x) {
    const size_t t = u / H4, i = u % H4;
    float4 s = make_float4(0.f, 0.f, 0.f, 0.f);
    for (int j = 0; j < k + S; ++j) {
      const size_t row = pos_major ? t * (size_t)(k + S) + j
                                   : (j < k ? (size_t)slot_row[t * k + j] : (size_t)Tn * k + (size_t)(j - k) * Tn + t);
      const float gt = j < k ? gate[t * k + j] : 1.0f;
      const float4 y = load4(ybuf, row * H4 + i);
      s.x = fmaf(gt, y.x, s.x);
      s.y = fmaf(gt, y.y, s.y);
      s.z = fmaf(gt, y.z, s.z);
      s.w = fmaf(gt, y.w, s.w);
    }
    reinterpret_cast<float4*>(m)[u] = s;
  }
}

// Routed slot of each expert-major row, from the row's position-major expert-output row.
__global__ void k_row_slot(const int32_t* __restrict__ row_dst, int n, int k, int KS, int32_t* __restrict__ out) {
  const int r = blockIdx.x * blockDim.x + threadIdx.x;
  if (r >= n) return;
  const int d = row_dst[r];
  out[r] = (d / KS) * k + d % KS;
}

// ============================================================================ launchers

static unsigned grid_for(size_t n, unsigned block, unsigned cap = 65535u * 8u) {
  size_t g = (n + block - 1) / block;
  if (g < 1) g = 1;
  return (unsigned)(g > cap ? cap : g);
}

hipError_t launch_repack_pairs(const void* src0, const void* src1, void* dst, int n_mats, int N, int row_bytes,
                               int NQ, int NKB, int gate_up, size_t mat_stride, hipStream_t stream) {
  const size_t total = (size_t)n_mats * NQ * NKB * kPairUnits;
  k_repack_pairs<<<grid_for(total, 256), 256, 0, stream>>>(
      static_cast<const uint8_t*>(src0), static_cast<const uint8_t*>(src1), static_cast<uint4*>(dst), n_mats, N,
      row_bytes, NQ, NKB, gate_up, mat_stride);
  return hipGetLastError();
}

hipError_t launch_repack_router(const void* src, void* dst, int L, int E, int row_bytes, hipStream_t stream) {
  const size_t total = (size_t)L * (row_bytes / 16) * 64;
  k_repack_router<<<grid_for(total, 256), 256, 0, stream>>>(static_cast<const uint8_t*>(src),
                                                             static_cast<uint4*>(dst), L, E, row_bytes);
  return hipGetLastError();
}

// Positions per workgroup of the routing norm kernel: one up to 256 positions (every
// position on its own compute unit), then two (each workgroup reads the 164 KB of router
// weights once for two positions: 19.8 -> 14.9 us per block at 512 positions; four there
// took 20.9 us, half the compute units idle) and four from 1025.
int norm_split_positions(int Tn) { return Tn <= 256 ? 1 : (Tn <= 1024 ? 2 : 4); }

size_t norm_lds_bytes(int wdtype, int H, int np) {
  return (size_t)np * (H * (wdtype == 1 ? 2 : 4) + 16) + (size_t)np * 64 * sizeof(float) +
         (size_t)np * 4 * sizeof(float);
}

template <typename T, int NP, int VM>
static void norm_route_t(bool route, const float* x_in, const T* ybuf, const int32_t* slot_row, float* x_out,
                         float* x_copy, void* a_out, const uint4* w, const float* bias, int32_t* topk_id,
                         float* topk_w, int Tn, int H, int S, int E, int k, float eps, int perm_a, int pos_major,
                         hipStream_t stream) {
  const dim3 grid((Tn + NP - 1) / NP), block(256);
  const int wdtype = sizeof(T) == 2 ? 1 : 0;
  if (route)
    k_norm_route<T, true, NP, VM><<<grid, block, norm_lds_bytes(wdtype, H, NP), stream>>>(
        x_in, ybuf, slot_row, x_out, x_copy, static_cast<T*>(a_out), w, bias, topk_id, topk_w, Tn, H, S, E, k, eps,
        perm_a, pos_major);
  else
    k_norm_route<T, false, NP, VM><<<grid, block, 0, stream>>>(x_in, ybuf, slot_row, x_out, x_copy,
                                                               static_cast<T*>(a_out), w, bias, topk_id, topk_w, Tn,
                                                               H, S, E, k, eps, perm_a, pos_major);
}

template <typename T, int NP, int VQ>
static void norm_split_t(bool route, const float* x_in, const T* ybuf, const int32_t* slot_row, float* x_out,
                         float* x_copy, void* a_out, const uint4* w, const float* bias, int32_t* topk_id,
                         float* topk_w, int Tn, int H, int S, int E, int k, float eps, int perm_a, int pos_major,
                         hipStream_t stream) {
  constexpr int NC = 40;  // router chunks requested at the start: a 1280-wide bf16 row
  const dim3 grid((Tn + NP - 1) / NP);
  const int wdtype = sizeof(T) == 2 ? 1 : 0;
  const size_t lds = norm_lds_bytes(wdtype, H, NP);
  if (route)
    k_norm_route_split<T, true, NP, VQ, NC><<<grid, dim3(512), lds, stream>>>(
        x_in, ybuf, slot_row, x_out, x_copy, static_cast<T*>(a_out), w, bias, topk_id, topk_w, Tn, H, S, E, k, eps,
        perm_a, pos_major);
  else
    k_norm_route_split<T, false, NP, VQ, NC><<<grid, dim3(256), lds, stream>>>(
        x_in, ybuf, slot_row, x_out, x_copy, static_cast<T*>(a_out), w, bias, topk_id, topk_w, Tn, H, S, E, k, eps,
        perm_a, pos_major);
}

template <typename T, int NP>
static void norm_split_np(bool route, const float* x_in, const T* ybuf, const int32_t* slot_row, float* x_out,
                          float* x_copy, void* a_out, const uint4* w, const float* bias, int32_t* topk_id,
                          float* topk_w, int Tn, int H, int S, int E, int k, float eps, int perm_a, int pos_major,
                          hipStream_t stream) {
  const int q4 = (H / 4 + 3) / 4;            // float4 columns per quarter row
  const int vq = (q4 + kWave - 1) / kWave;  // float4 per lane of one quarter
  if (vq <= 1) norm_split_t<T, NP, 1>(route, x_in, ybuf, slot_row, x_out, x_copy, a_out, w, bias, topk_id, topk_w, Tn, H, S, E, k, eps, perm_a, pos_major, stream);
  else if (vq == 2) norm_split_t<T, NP, 2>(route, x_in, ybuf, slot_row, x_out, x_copy, a_out, w, bias, topk_id, topk_w, Tn, H, S, E, k, eps, perm_a, pos_major, stream);
  else norm_split_t<T, NP, 4>(route, x_in, ybuf, slot_row, x_out, x_copy, a_out, w, bias, topk_id, topk_w, Tn, H, S, E, k, eps, perm_a, pos_major, stream);
}

template <typename T>
static void norm_split(bool route, const float* x_in, const T* ybuf, const int32_t* slot_row, float* x_out,
                       float* x_copy, void* a_out, const uint4* w, const float* bias, int32_t* topk_id,
                       float* topk_w, int Tn, int H, int S, int E, int k, float eps, int perm_a, int pos_major,
                       hipStream_t stream) {
  const int np = route ? norm_split_positions(Tn) : 1;  // no router weights to share: one position per workgroup
  if (np == 1) norm_split_np<T, 1>(route, x_in, ybuf, slot_row, x_out, x_copy, a_out, w, bias, topk_id, topk_w, Tn, H, S, E, k, eps, perm_a, pos_major, stream);
  else if (np == 2) norm_split_np<T, 2>(route, x_in, ybuf, slot_row, x_out, x_copy, a_out, w, bias, topk_id, topk_w, Tn, H, S, E, k, eps, perm_a, pos_major, stream);
  else norm_split_np<T, 4>(route, x_in, ybuf, slot_row, x_out, x_copy, a_out, w, bias, topk_id, topk_w, Tn, H, S, E, k, eps, perm_a, pos_major, stream);
}

template <typename T, int NP>
static void norm_route_np(bool route, const float* x_in, const T* ybuf, const int32_t* slot_row, float* x_out,
                          float* x_copy, void* a_out, const uint4* w, const float* bias, int32_t* topk_id,
                          float* topk_w, int Tn, int H, int S, int E, int k, float eps, int perm_a, int pos_major,
                          hipStream_t stream) {
  const int vm = (H / 4 + kWave - 1) / kWave;  // float4 per lane of one row
  if (vm <= 2) norm_route_t<T, NP, 2>(route, x_in, ybuf, slot_row, x_out, x_copy, a_out, w, bias, topk_id, topk_w, Tn, H, S, E, k, eps, perm_a, pos_major, stream);
  else if (vm == 5) norm_route_t<T, NP, 5>(route, x_in, ybuf, slot_row, x_out, x_copy, a_out, w, bias, topk_id, topk_w, Tn, H, S, E, k, eps, perm_a, pos_major, stream);
  else if (vm <= 8) norm_route_t<T, NP, 8>(route, x_in, ybuf, slot_row, x_out, x_copy, a_out, w, bias, topk_id, topk_w, Tn, H, S, E, k, eps, perm_a, pos_major, stream);
  else norm_route_t<T, NP, 16>(route, x_in, ybuf, slot_row, x_out, x_copy, a_out, w, bias, topk_id, topk_w, Tn, H, S, E, k, eps, perm_a, pos_major, stream);
}

hipError_t launch_norm_route(int wdtype, bool route, const float* x_in, const void* ybuf,
                             const int32_t* slot_row, float* x_out, float* x_copy, void* a_out, const void* wr,
                             const float* bias, int32_t* topk_id, float* topk_w, int Tn, int H, int S, int E,
                             int k, float eps, bool perm_a, bool pos_major, hipStream_t stream) {
  const uint4* w = static_cast<const uint4*>(wr);
  // the no-router combine (the final norm) runs split at every size
  const bool big = route && Tn >= kNormSplitMaxPositions;
  if (wdtype == 1) {
    if (big) norm_route_np<uint16_t, 16>(route, x_in, static_cast<const uint16_t*>(ybuf), slot_row, x_out, x_copy, a_out, w, bias, topk_id, topk_w, Tn, H, S, E, k, eps, perm_a, pos_major, stream);
    else norm_split<uint16_t>(route, x_in, static_cast<const uint16_t*>(ybuf), slot_row, x_out, x_copy, a_out, w, bias, topk_id, topk_w, Tn, H, S, E, k, eps, perm_a, pos_major, stream);
  } else {
    if (big) norm_route_np<float, 16>(route, x_in, static_cast<const float*>(ybuf), slot_row, x_out, x_copy, a_out, w, bias, topk_id, topk_w, Tn, H, S, E, k, eps, perm_a, pos_major, stream);
    else norm_split<float>(route, x_in, static_cast<const float*>(ybuf), slot_row, x_out, x_copy, a_out, w, bias, topk_id, topk_w, Tn, H, S, E, k, eps, perm_a, pos_major, stream);
  }
  return hipGetLastError();
}

int plan_chunks(int Tn, int k) { return (Tn * k + kPlanChunk - 1) / kPlanChunk; }

hipError_t launch_plan(const PlanArgs& pa, hipStream_t stream) {
  const int n = plan_chunks(pa.Tn, pa.k);
  if (pa.hot_rows > 0 && n > kPlanSingleMaxChunks) return hipErrorInvalidValue;  // split plan: one workgroup only
  if (n <= kPlanSingleMaxChunks || !pa.chunk_cnt) {
    k_plan<<<1, 1024, 0, stream>>>(pa);
  } else {
    k_plan_count<<<n, 256, 0, stream>>>(pa);
    k_plan_scatter<<<n, 256, 0, stream>>>(pa);
  }
  return hipGetLastError();
}

template <typename T>
static void gemm_t(int epi, const GemmArgs& args, unsigned n_wg, hipStream_t stream) {
  const dim3 grid(n_wg);
  if (epi == EPI_UP)
    k_moe_gemm<T, EPI_UP, MV_GEMM_NMT, MV_GEMM_D, kStreamWavesUp><<<grid, dim3(kWave * kStreamWavesUp), 0, stream>>>(args);
  else if (epi == EPI_DOWN)
    k_moe_gemm<T, EPI_DOWN, MV_GEMM_NMT, MV_GEMM_D, kStreamWavesDown><<<grid, dim3(kWave * kStreamWavesDown), 0, stream>>>(args);
  else k_lm_head<T><<<grid, dim3(kLmWaves * kWave), 0, stream>>>(args);
}

hipError_t launch_gemm_planned(int wdtype, const GemmArgs& args, unsigned n_wg, hipStream_t stream) {
  const dim3 grid(n_wg), block(kWave * kStreamWavesUp);
  if (wdtype == 1)
    k_moe_gemm_planned<uint16_t, MV_GEMM_NMT, MV_GEMM_D, kStreamWavesUp><<<grid, block, 0, stream>>>(args);
  else
    k_moe_gemm_planned<float, MV_GEMM_NMT, MV_GEMM_D, kStreamWavesUp><<<grid, block, 0, stream>>>(args);
  return hipGetLastError();
}

hipError_t launch_gemm(int wdtype, int epi, const GemmArgs& args, unsigned n_wg, hipStream_t stream) {
  if (wdtype == 1) gemm_t<uint16_t>(epi, args, n_wg, stream);
  else gemm_t<float>(epi, args, n_wg, stream);
  return hipGetLastError();
}

hipError_t launch_argmax_reduce(const Top2* part, int n_pg, int Tn, int32_t* argmax, float* margin,
                                hipStream_t stream) {
  k_argmax_reduce<<<(Tn + 3) / 4, 256, 0, stream>>>(part, n_pg, Tn, argmax, margin);
  return hipGetLastError();
}

hipError_t launch_accept(const int32_t* drafts, const int32_t* argmax, int B, int K, int32_t* accepted,
                         int32_t* committed, hipStream_t stream) {
  k_accept<<<(B + 255) / 256, 256, 0, stream>>>(drafts, argmax, B, K, accepted, committed);
  return hipGetLastError();
}

hipError_t launch_row_slot(const int32_t* row_dst, int n, int k, int KS, int32_t* row_slot, hipStream_t stream) {
  k_row_slot<<<(n + 255) / 256, 256, 0, stream>>>(row_dst, n, k, KS, row_slot);
  return hipGetLastError();
}

hipError_t launch_combine(int wdtype, const void* ybuf, const int32_t* slot_row, const float* gate, int Tn, int H,
                          int k, int S, bool pos_major, float* m, hipStream_t stream) {
  const unsigned grid = grid_for((size_t)Tn * (H / 4), 256);
  if (wdtype == 1)
    k_combine<<<grid, 256, 0, stream>>>(static_cast<const uint16_t*>(ybuf), slot_row, gate, Tn, H, k, S,
                                        pos_major ? 1 : 0, m);
  else
    k_combine<<<grid, 256, 0, stream>>>(static_cast<const float*>(ybuf), slot_row, gate, Tn, H, k, S,
                                        pos_major ? 1 : 0, m);
  return hipGetLastError();
}

}  // namespace mv
