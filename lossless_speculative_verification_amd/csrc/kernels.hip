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
//   per block l: k_norm_route  (combine of block l-1 + residual + RMSNorm + router + top-k)
//                k_plan        (expert-major stable ordering of the T*k routed slots + work list)
//                k_gemm<UP>    (gate/up projections + SwiGLU, MFMA, weights streamed once)
//                k_gemm<DOWN>  (down projection, gate scaling, one ybuf row per slot)
//   then         k_norm_route  (final combine + residual + RMSNorm, no router)
//                k_gemm<LM>    (LM-head logits tile by tile, top-1/top-2 per tile, never stored)
//                k_argmax_reduce
//   and          k_accept
#include <climits>

#include "launch.h"

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

// One wavefront per position, four per workgroup.
//  1. x = x_in + sum_j ybuf[j] (j = 0..KS-1 in order; absent for the first block);
//     x is written back as the residual stream (and to x_copy when given).
//  2. a = x / sqrt(mean(x^2) + eps), stored in the element type (bf16 rounding).
//  3. (route) logits r_e = a . W_r[e] + bias_e, lane e = expert e (E <= 64), float32.
//  4. (route) k rounds of a wavefront argmax (larger logit, then lower index) give the
//     selected experts in slot order; gates = softmax of the selected logits.
template <typename T, bool ROUTE>
__global__ __launch_bounds__(256) void k_norm_route(const float* x_in, const float* __restrict__ ybuf,
                                                    float* x_out, float* __restrict__ x_copy,
                                                    T* __restrict__ a_out, const uint4* __restrict__ wr,
                                                    const float* __restrict__ bias,
                                                    int32_t* __restrict__ topk_id, float* __restrict__ topk_w,
                                                    int Tn, int H, int KS, int E, int k, float eps) {
  extern __shared__ uint4 a_lds_raw[];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + wave;
  const bool valid = t < Tn;  // every wavefront stays to the workgroup barrier below
  const int H4 = H >> 2;
  const size_t t0 = valid ? (size_t)t : 0;
  const float4* xi = reinterpret_cast<const float4*>(x_in) + t0 * H4;
  float4* xo = x_out ? reinterpret_cast<float4*>(x_out) + t0 * H4 : nullptr;
  float4* xc = x_copy ? reinterpret_cast<float4*>(x_copy) + t0 * H4 : nullptr;
  const float4* yb0 = ybuf ? reinterpret_cast<const float4*>(ybuf) + t0 * KS * H4 : nullptr;

  // x = x_in + (y_0 + y_1 + ... + y_{KS-1}), the block output summed in slot order.
  auto residual = [&](int i) {
    float4 v = xi[i];
    if (yb0) {
      float4 m = yb0[i];
      for (int j = 1; j < KS; ++j) {
        const float4 y = yb0[(size_t)j * H4 + i];
        m.x += y.x; m.y += y.y; m.z += y.z; m.w += y.w;
      }
      v.x += m.x; v.y += m.y; v.z += m.z; v.w += m.w;
    }
    return v;
  };

  float ss = 0.f;
  if (valid) {
    for (int i = lane; i < H4; i += kWave) {
      const float4 v = residual(i);
      if (xo) xo[i] = v;
      if (xc) xc[i] = v;
      ss += v.x * v.x + v.y * v.y + v.z * v.z + v.w * v.w;
    }
  }
  ss = wave_sum(ss);
  const float inv = 1.0f / sqrtf(ss / (float)H + eps);

  // Normalise. x is re-read from what this lane itself wrote (x_out), or recomputed
  // the same way when there is no x_out; each lane touches only its own elements.
  T* a_lds = reinterpret_cast<T*>(a_lds_raw) + (size_t)wave * H;
  T* arow = a_out + t0 * H;
  if (valid) {
    for (int i = lane; i < H4; i += kWave) {
      const float4 v = xo ? xo[i] : residual(i);
      const float u[4] = {v.x * inv, v.y * inv, v.z * inv, v.w * inv};
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        store_elem(arow, (size_t)4 * i + c, u[c]);
        if (ROUTE) store_elem(a_lds, (size_t)4 * i + c, u[c]);
      }
    }
  }
  if (!ROUTE) return;
  __syncthreads();
  if (!valid) return;

  // Router logits: lane e accumulates a . W_r[e] over the row in order.
  constexpr int P = Elem<T>::per16;
  const int chunks = H / P;
  const uint4* al = reinterpret_cast<const uint4*>(a_lds);
  float acc = 0.f;
#pragma unroll 8
  for (int c = 0; c < chunks; ++c) {
    const uint4 w = wr[(size_t)c * 64 + lane];
    const uint4 av = al[c];
    const T* wp = reinterpret_cast<const T*>(&w);
    const T* ap = reinterpret_cast<const T*>(&av);
#pragma unroll
    for (int i = 0; i < P; ++i) acc += Elem<T>::load(ap, i) * Elem<T>::load(wp, i);
  }
  const float NEG = -__builtin_huge_valf();
  float r = lane < E ? acc + bias[lane] : NEG;
  if (r != r) r = NEG;  // a NaN logit ranks last, so every selected id stays below E

  // Top-k by repeated wavefront argmax; lane j keeps the j-th selection.
  bool taken = false;
  float my_v = NEG, v0 = 0.f;
  int my_e = 0;
  for (int j = 0; j < k; ++j) {
    float bv = taken ? NEG : r;
    int bi = taken ? INT_MAX : lane;
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) {
      const float ov = __shfl_xor(bv, m, kWave);
      const int oi = __shfl_xor(bi, m, kWave);
      if (ov > bv || (ov == bv && oi < bi)) { bv = ov; bi = oi; }
    }
    if (lane == bi) taken = true;
    if (lane == j) { my_v = bv; my_e = bi; }
    if (j == 0) v0 = bv;
  }
  const float z = lane < k ? expf(my_v - v0) : 0.f;
  const float Z = wave_sum(z);
  if (lane < k) {
    topk_id[(size_t)t * k + lane] = my_e;
    topk_w[(size_t)t * k + lane] = z / Z;
  }
}

// ============================================================================ routing plan

// One workgroup of 16 wavefronts orders the T*k routed slots (slot = t*k + j) by
// expert, stably (ascending slot within an expert), and lists the GEMM work items.
//  phase 1: per-wavefront expert histograms of 16 contiguous slot segments;
//  phase 2: exclusive scan in (expert, segment) order -> each segment's write base;
//  phase 3: each wavefront places its segment 64 slots at a time; lanes with the same
//           expert are found with six ballots over the expert id bits, and a lane's
//           rank is the count of lower lanes in its group;
//  phase 4: work items of at most kGemmMB rows: routed experts first (expert order),
//           then each shared expert's position blocks.
// Routed rows occupy [0, T*k) of the row space; shared expert s owns rows
// T*k + s*T + t.
__global__ __launch_bounds__(1024) void k_plan(const int32_t* __restrict__ topk_id,
                                               const float* __restrict__ topk_w, int Tn, int k, int E, int S,
                                               int32_t* __restrict__ row_tok, int32_t* __restrict__ row_dst,
                                               float* __restrict__ row_gate, int4* __restrict__ work,
                                               int32_t* __restrict__ n_work, int32_t* __restrict__ counts) {
  __shared__ int hist[16][64];
  __shared__ int off[65];
  __shared__ int wstart[65];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int N = Tn * k, KS = k + S;
  hist[wave][lane] = 0;
  __syncthreads();

  const int seg = (N + 15) / 16;
  const int beg = min(N, wave * seg), end = min(N, beg + seg);
  for (int i = beg + lane; i < end; i += kWave) atomicAdd(&hist[wave][min(max(topk_id[i], 0), E - 1)], 1);
  __syncthreads();

  if (wave == 0) {
    int c = 0;
    if (lane < E)
      for (int w = 0; w < 16; ++w) c += hist[w][lane];
    const int nb = (c + kGemmMB - 1) / kGemmMB;
    // inclusive scans over lanes of c and nb
    int sc = c, sn = nb;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
      const int oc = __shfl_up(sc, d, kWave), on = __shfl_up(sn, d, kWave);
      if (lane >= d) { sc += oc; sn += on; }
    }
    off[lane] = sc - c;
    wstart[lane] = sn - nb;
    if (lane < E) counts[lane] = c;
    if (lane == 63) { off[64] = sc; wstart[64] = sn; }
    int run = sc - c;
    for (int w = 0; w < 16; ++w) {
      const int h = hist[w][lane];
      hist[w][lane] = run;  // becomes the segment's write cursor for this expert
      run += h;
    }
  }
  __syncthreads();

  for (int b0 = beg; b0 < end; b0 += kWave) {
    const int i = b0 + lane;
    const bool active = i < end;
    const int key = active ? min(max(topk_id[i], 0), E - 1) : 0;  // ids come from k_norm_route, always < E
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
      row_tok[pos] = tok;
      row_dst[pos] = tok * KS + j;
      row_gate[pos] = topk_w[i];
      if (rank == cnt - 1) hist[wave][key] = pos + 1;
    }
    __builtin_amdgcn_wave_barrier();
  }

  if (tid < E) {
    const int c = off[tid + 1] - off[tid];
    for (int b = 0; b * kGemmMB < c; ++b)
      work[wstart[tid] + b] = make_int4(tid, off[tid] + b * kGemmMB, min(kGemmMB, c - b * kGemmMB), 0);
  }
  const int nrw = wstart[64];
  const int mbT = (Tn + kGemmMB - 1) / kGemmMB;
  for (int idx = tid; idx < S * mbT; idx += 1024) {
    const int s = idx / mbT, b = idx - s * mbT;
    work[nrw + idx] = make_int4(E + s, N + s * Tn + b * kGemmMB, min(kGemmMB, Tn - b * kGemmMB), b * kGemmMB);
  }
  if (tid == 0) *n_work = nrw + S * mbT;
}

// ============================================================================ grouped MFMA GEMM

// One workgroup = 4 wavefronts = 4 column pairs (2 x 16 output columns each) of one
// expert, for up to kGemmMB rows of that expert (one work item). Weights stream from
// HBM once, straight into registers, in the pair layout (8 coalesced 1 KB loads per
// wavefront per 256-byte K block, two K blocks in flight). The work item's activation
// rows are staged in LDS one K block at a time (double-buffered, one 16-byte pad per
// row so the 16 rows an MFMA reads hit distinct banks) and read as MFMA A operands.
// Products accumulate in float32 MFMA (16x16x32 bf16 or 16x16x4 f32).
//   UP:   tile t = 0 is the gate projection, t = 1 the up projection of the same 16
//         intermediate columns; the epilogue forms silu(gate) * up and stores it.
//   DOWN: the epilogue scales by the row's gate (1 for shared experts) and writes the
//         row's own ybuf slot; no two workgroups write the same element.
//   LM:   the epilogue reduces each row's 32 logits per wavefront to (top-1 value,
//         lowest index, top-2 value), then across the 4 wavefronts; one record per row
//         and workgroup goes to `part`.
template <typename T, int EPI>
__global__ __launch_bounds__(256) void k_gemm(GemmArgs g) {
  constexpr int MT = kGemmMB / 16;
  __shared__ uint4 As[2][kGemmMB][kChunksPerRow + 1];
  __shared__ Top2 red[EPI == EPI_LM ? kGemmWaves : 1][EPI == EPI_LM ? kGemmMB : 1];

  const int pg = blockIdx.x;
  int e, row0, M, tok0;
  if (EPI == EPI_LM) {
    e = 0;
    row0 = blockIdx.y * kGemmMB;
    M = min(kGemmMB, g.Tn - row0);
    tok0 = row0;
    if (M <= 0) return;
  } else {
    if ((int)blockIdx.y >= *g.n_work) return;
    const int4 it = g.work[blockIdx.y];
    e = it.x; row0 = it.y; M = it.z; tok0 = it.w;
  }
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int q = pg * kGemmWaves + wave;
  const bool qok = q < g.NQ;
  const int row_units = g.K * (int)sizeof(T) / 16;
  const int NKB = row_units / kChunksPerRow;
  const uint4* Bq = g.B + ((size_t)e * g.NQ + (qok ? q : 0)) * (size_t)NKB * kPairUnits + lane;

  // Activation staging: thread -> row srow + 16*it, 16-byte chunk schunk of the K block.
  const int srow = threadIdx.x >> 4, schunk = threadIdx.x & 15;
  const uint4* arow[MT];
#pragma unroll
  for (int it = 0; it < MT; ++it) {
    const int r = srow + 16 * it;
    arow[it] = nullptr;
    if (r < M) {
      int src;
      if (EPI == EPI_UP) src = (e < g.E) ? g.row_tok[row0 + r] : tok0 + r;
      else if (EPI == EPI_DOWN) src = row0 + r;
      else src = tok0 + r;
      arow[it] = reinterpret_cast<const uint4*>(g.A) + (size_t)src * row_units + schunk;
    }
  }
  uint4 ra[MT], rb0[8], rb1[8];
  auto load_a = [&](int kb) {
#pragma unroll
    for (int it = 0; it < MT; ++it) ra[it] = arow[it] ? arow[it][kb * kChunksPerRow] : make_uint4(0u, 0u, 0u, 0u);
  };
  auto store_a = [&](int buf) {
#pragma unroll
    for (int it = 0; it < MT; ++it) As[buf][srow + 16 * it][schunk] = ra[it];
  };
  auto load_b = [&](int kb, uint4(&rb)[8]) {
    if (!qok) return;
#pragma unroll
    for (int u = 0; u < 8; ++u) rb[u] = load_stream(Bq + (size_t)kb * kPairUnits + u * kWave);
  };

  f32x4_t acc[MT][2];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) acc[mt][0] = acc[mt][1] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  const int n_mt = (M + 15) >> 4;
  auto compute = [&](int buf, const uint4(&rb)[8]) {
    if (!qok) return;
#pragma unroll
    for (int s = 0; s < 4; ++s) {
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        if (mt < n_mt) {
          const uint4 a = As[buf][mt * 16 + (lane & 15)][(lane >> 4) * 4 + s];
          mma_chunk(acc[mt][0], a, rb[s], (T*)nullptr);
          mma_chunk(acc[mt][1], a, rb[4 + s], (T*)nullptr);
        }
      }
    }
  };

  load_a(0);
  store_a(0);
  load_b(0, rb0);
  if (NKB > 1) load_b(1, rb1);
  __syncthreads();
  for (int kb = 0; kb < NKB; kb += 2) {
    if (kb + 1 < NKB) load_a(kb + 1);
    compute(0, rb0);
    if (kb + 2 < NKB) load_b(kb + 2, rb0);
    if (kb + 1 < NKB) store_a(1);
    __syncthreads();
    if (kb + 1 >= NKB) break;
    if (kb + 2 < NKB) load_a(kb + 2);
    compute(1, rb1);
    if (kb + 3 < NKB) load_b(kb + 3, rb1);
    if (kb + 2 < NKB) store_a(0);
    __syncthreads();
  }

  const int col = lane & 15, rg = (lane >> 4) * 4;
  if (EPI == EPI_UP) {
    if (!qok) return;
    T* h = reinterpret_cast<T*>(g.h);
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      if (mt >= n_mt) break;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = mt * 16 + rg + i;
        if (r < M) {
          const float gv = acc[mt][0][i], uv = acc[mt][1][i];
          const float hv = gv / (1.0f + expf(-gv)) * uv;
          store_elem(h, (size_t)(row0 + r) * g.I + q * 16 + col, hv);
        }
      }
    }
  } else if (EPI == EPI_DOWN) {
    if (!qok) return;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      if (mt >= n_mt) break;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = mt * 16 + rg + i;
        if (r < M) {
          int dst;
          float gate;
          if (e < g.E) {
            dst = g.row_dst[row0 + r];
            gate = g.row_gate[row0 + r];
          } else {
            dst = (tok0 + r) * g.KS + g.k + (e - g.E);
            gate = 1.0f;
          }
          float* yrow = g.ybuf + (size_t)dst * g.H + (2 * q) * 16 + col;
          yrow[0] = acc[mt][0][i] * gate;
          yrow[16] = acc[mt][1][i] * gate;
        }
      }
    }
  } else {  // EPI_LM
    const float NEG = -__builtin_huge_valf();
    const int c0 = 2 * q * 16 + col, c1 = c0 + 16;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      if (mt >= n_mt) break;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float v0 = (qok && c0 < g.n_valid) ? acc[mt][0][i] : NEG;
        const float v1 = (qok && c1 < g.n_valid) ? acc[mt][1][i] : NEG;
        Top2 rec;
        if (v0 >= v1) { rec.v1 = v0; rec.i1 = c0; rec.v2 = v1; }
        else { rec.v1 = v1; rec.i1 = c1; rec.v2 = v0; }
#pragma unroll
        for (int m = 1; m < 16; m <<= 1) rec = top2_merge(rec, top2_shfl_xor(rec, m));
        if (col == 0) red[wave][mt * 16 + rg + i] = rec;
      }
    }
    __syncthreads();
    if ((int)threadIdx.x < M) {
      const int r = threadIdx.x;
      Top2 rec = red[0][r];
#pragma unroll
      for (int w = 1; w < kGemmWaves; ++w) rec = top2_merge(rec, red[w][r]);
      g.part[(size_t)(row0 + r) * g.n_pg + pg] = rec;
    }
  }
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
  Top2 rec{NEG, INT_MAX, NEG};
  for (int p = lane; p < n_pg; p += kWave) rec = top2_merge(rec, part[(size_t)t * n_pg + p]);
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

// m[t] = sum_j ybuf[t][j] in slot order (the block output before the residual add).
__global__ void k_combine(const float* __restrict__ ybuf, int Tn, int H, int KS, float* __restrict__ m) {
  const int H4 = H >> 2;
  const size_t total = (size_t)Tn * H4;
  for (size_t u = (size_t)blockIdx.x * blockDim.x + threadIdx.x; u < total; u += (size_t)gridDim.x * blockDim.x) {
    const size_t t = u / H4, i = u % H4;
    const float4* yb = reinterpret_cast<const float4*>(ybuf) + t * KS * H4 + i;
    float4 s = yb[0];
    for (int j = 1; j < KS; ++j) {
      const float4 y = yb[(size_t)j * H4];
      s.x += y.x; s.y += y.y; s.z += y.z; s.w += y.w;
    }
    reinterpret_cast<float4*>(m)[u] = s;
  }
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

hipError_t launch_norm_route(int wdtype, bool route, const float* x_in, const float* ybuf, float* x_out,
                             float* x_copy, void* a_out, const void* wr, const float* bias, int32_t* topk_id,
                             float* topk_w, int Tn, int H, int KS, int E, int k, float eps, hipStream_t stream) {
  const dim3 grid((Tn + 3) / 4), block(256);
  const uint4* w = static_cast<const uint4*>(wr);
  if (wdtype == 1) {
    const size_t lds = route ? (size_t)4 * H * sizeof(uint16_t) : 0;
    if (route)
      k_norm_route<uint16_t, true><<<grid, block, lds, stream>>>(x_in, ybuf, x_out, x_copy,
                                                                 static_cast<uint16_t*>(a_out), w, bias, topk_id,
                                                                 topk_w, Tn, H, KS, E, k, eps);
    else
      k_norm_route<uint16_t, false><<<grid, block, 0, stream>>>(x_in, ybuf, x_out, x_copy,
                                                                static_cast<uint16_t*>(a_out), w, bias, topk_id,
                                                                topk_w, Tn, H, KS, E, k, eps);
  } else {
    const size_t lds = route ? (size_t)4 * H * sizeof(float) : 0;
    if (route)
      k_norm_route<float, true><<<grid, block, lds, stream>>>(x_in, ybuf, x_out, x_copy, static_cast<float*>(a_out),
                                                              w, bias, topk_id, topk_w, Tn, H, KS, E, k, eps);
    else
      k_norm_route<float, false><<<grid, block, 0, stream>>>(x_in, ybuf, x_out, x_copy, static_cast<float*>(a_out),
                                                             w, bias, topk_id, topk_w, Tn, H, KS, E, k, eps);
  }
  return hipGetLastError();
}

hipError_t launch_plan(const int32_t* topk_id, const float* topk_w, int Tn, int k, int E, int S, int32_t* row_tok,
                       int32_t* row_dst, float* row_gate, int4* work, int32_t* n_work, int32_t* counts,
                       hipStream_t stream) {
  k_plan<<<1, 1024, 0, stream>>>(topk_id, topk_w, Tn, k, E, S, row_tok, row_dst, row_gate, work, n_work, counts);
  return hipGetLastError();
}

hipError_t launch_gemm(int wdtype, int epi, const GemmArgs& args, dim3 grid, hipStream_t stream) {
  const dim3 block(256);
  if (wdtype == 1) {
    if (epi == EPI_UP) k_gemm<uint16_t, EPI_UP><<<grid, block, 0, stream>>>(args);
    else if (epi == EPI_DOWN) k_gemm<uint16_t, EPI_DOWN><<<grid, block, 0, stream>>>(args);
    else k_gemm<uint16_t, EPI_LM><<<grid, block, 0, stream>>>(args);
  } else {
    if (epi == EPI_UP) k_gemm<float, EPI_UP><<<grid, block, 0, stream>>>(args);
    else if (epi == EPI_DOWN) k_gemm<float, EPI_DOWN><<<grid, block, 0, stream>>>(args);
    else k_gemm<float, EPI_LM><<<grid, block, 0, stream>>>(args);
  }
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

hipError_t launch_combine(const float* ybuf, int Tn, int H, int KS, float* m, hipStream_t stream) {
  k_combine<<<grid_for((size_t)Tn * (H / 4), 256), 256, 0, stream>>>(ybuf, Tn, H, KS, m);
  return hipGetLastError();
}

}  // namespace mv
