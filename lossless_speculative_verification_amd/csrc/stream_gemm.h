// The streaming expert-GEMM unit: one wavefront, one work item of up to 16*NMT rows,
// PPW column pairs, the whole contraction (used by k_moe_gemm, k_moe_gemm_planned and
// the tiled kernel's streaming items).
#pragma once

#include "launch.h"

namespace mv {

// One wavefront computes PPW consecutive column pairs (2 x 16 output columns each) of one
// expert work item (up to 16*NMT rows) over the whole contraction, the pairs side by
// side so that one loop serves them all:
//  * weights stream from HBM once, in the pair layout: per 256-byte K block and pair,
//    8 fully coalesced 1 KB non-temporal loads; D K blocks in flight;
//  * the item's activation rows are read straight from global memory (small and
//    L2-resident), once per K block for all PPW pairs: lane l reads row 16*mt + l%16
//    of each row tile, the 64 bytes of the K block that its lane group l/16 contracts;
//    rows past the item's end repeat row 0 and their results are dropped;
//  * products accumulate in float32 MFMA (16x16x32 bf16, or 16x16x4 f32).
// The main loop holds only loads and MFMAs, and no load in it depends on a branch: a
// store, a spill or a conditional load there would make the compiler wait for every
// load in flight. The epilogue follows the loop:
//   UP:   tile t = 0 is the gate projection, t = 1 the up projection of the same 16
//         intermediate columns; the epilogue forms silu(gate) * up and stores it.
//   DOWN: the epilogue writes the row's expert output to its slot's position-major row
//         of ybuf, t*(k+S) + j (the gate is applied where the slots are summed); no two
//         wavefronts write the same element.
// There is no LDS and no barrier: wavefronts run free.
// STAGED: the layout of the tiled kernel's passes (activation rows and h in the stage
// order of the tiled GEMM, one ybuf row per routed or shared row, row0 + r), for the
// streaming work items that kernel runs beside its tiles.
template <typename T, int EPI, int NMT, int PPW, int D, bool STAGED = false>
__device__ __forceinline__ void moe_stream(const GemmArgs& g, int e, int row0, int M, int tok0, int q0,
                                           const int* tok_lds = nullptr) {
  const int lane = threadIdx.x & 63;
  const int row_units = g.K * (int)sizeof(T) / 16;
  const int NKB = row_units / kChunksPerRow;
  const int col = lane & 15, rg = (lane >> 4) * 4;
  const uint4* Bw[PPW];
#pragma unroll
  for (int p = 0; p < PPW; ++p) {
    const int q = min(q0 + p, g.NQ - 1);  // a pair past the end repeats the last one; not stored
    Bw[p] = g.B + ((size_t)e * g.NQ + q) * (size_t)NKB * kPairUnits + lane;
  }
  uint4 ra[D][NMT][4], rb[D][PPW][8];
  f32x4_t acc[PPW][NMT][2];
#pragma unroll
  for (int p = 0; p < PPW; ++p)
#pragma unroll
    for (int mt = 0; mt < NMT; ++mt) acc[p][mt][0] = acc[p][mt][1] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  int kl = 0;  // next K block to load (stays at the last one once reached, when NKB < D)
  auto load_w = [&](uint4(&b)[PPW][8]) __attribute__((always_inline)) {
#pragma unroll
    for (int p = 0; p < PPW; ++p)
#pragma unroll
      for (int u = 0; u < 8; ++u) b[p][u] = load_stream(Bw[p] + (size_t)kl * kPairUnits + u * kWave);
  };
  // The first weight blocks go out before anything that needs the item's row indices.
  static_for<D>([&](auto sc) __attribute__((always_inline)) {
    load_w(rb[decltype(sc)::value]);
    kl += kl < NKB - 1 ? 1 : 0;
  });

  const uint4* ap[NMT];
#pragma unroll
  for (int mt = 0; mt < NMT; ++mt) {
    const int r = mt * 16 + (lane & 15);
    const int rr = r < M ? r : 0;
    int src;
    if constexpr (EPI == EPI_UP) src = (e < g.E) ? (tok_lds ? tok_lds[rr] : g.row_tok[row0 + rr]) : tok0 + rr;
    else src = row0 + rr;
    ap[mt] = reinterpret_cast<const uint4*>(g.A) + (size_t)src * row_units + (STAGED ? (lane >> 4) : (lane >> 4) * 4);
  }
  // DOWN: lane l holds the position-major ybuf row of item row l % (16*NMT); routed rows
  // from the plan, shared expert s's row of position t is t*KS + k + s
  int dst_row = 0;
  if constexpr (EPI == EPI_DOWN) {
    const int r = lane & (16 * NMT - 1);
    const int rr = r < M ? r : 0;
    if constexpr (STAGED) dst_row = row0 + rr;
    else dst_row = e < g.E ? g.row_dst[row0 + rr] : (tok0 + rr) * g.KS + g.k + (e - g.E);
  }
  int ka = 0;  // next K block of activations to load
  auto load_a = [&](uint4(&a)[NMT][4]) __attribute__((always_inline)) {
#pragma unroll
    for (int mt = 0; mt < NMT; ++mt)
#pragma unroll
      for (int s = 0; s < 4; ++s) a[mt][s] = ap[mt][ka * kChunksPerRow + (STAGED ? 4 * s : s)];
    ka += ka < NKB - 1 ? 1 : 0;
  };
  static_for<D>([&](auto sc) __attribute__((always_inline)) { load_a(ra[decltype(sc)::value]); });
  // In the loop a stage's activations go out before its weights.
  auto load = [&](uint4(&a)[NMT][4], uint4(&b)[PPW][8]) __attribute__((always_inline)) {
    load_a(a);
    load_w(b);
    kl += kl < NKB - 1 ? 1 : 0;
  };
  auto compute = [&](const uint4(&a)[NMT][4], const uint4(&b)[PPW][8]) __attribute__((always_inline)) {
#pragma unroll
    for (int s = 0; s < 4; ++s)
#pragma unroll
      for (int p = 0; p < PPW; ++p)
#pragma unroll
        for (int mt = 0; mt < NMT; ++mt) {
          mma_chunk(acc[p][mt][0], a[mt][s], b[p][s], (T*)nullptr);
          mma_chunk(acc[p][mt][1], a[mt][s], b[p][4 + s], (T*)nullptr);
        }
  };

  // Main loop: every load in it is in range (K block k0 + D + s < NKB). The tail then
  // computes the last D..2D-1 blocks, loading the r = NKB - k0 - D not yet requested.
  int k0 = 0;
  for (; k0 + 2 * D <= NKB; k0 += D) {
    static_for<D>([&](auto sc) __attribute__((always_inline)) {
      constexpr int s = decltype(sc)::value;
      compute(ra[s], rb[s]);
      load(ra[s], rb[s]);
      __builtin_amdgcn_sched_barrier(0);  // keep the loads here, D blocks ahead of their use
    });
  }
  const int r = NKB - k0 - D;
  static_for<D>([&](auto sc) __attribute__((always_inline)) {
    constexpr int s = decltype(sc)::value;
    if (k0 + s < NKB) compute(ra[s], rb[s]);
    if (s < r) load(ra[s], rb[s]);
  });
  static_for<D - 1>([&](auto sc) __attribute__((always_inline)) {
    constexpr int s = decltype(sc)::value;
    if (s < r) compute(ra[s], rb[s]);
  });

#pragma unroll
  for (int p = 0; p < PPW; ++p) {
    const int q = q0 + p;
    if (q >= g.NQ) break;
    if constexpr (EPI == EPI_UP) {
      T* h = reinterpret_cast<T*>(g.h);
#pragma unroll
      for (int mt = 0; mt < NMT; ++mt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int r = mt * 16 + rg + i;
          if (r < M) {
            const float gv = acc[p][mt][0][i], uv = acc[p][mt][1][i];
            const int ce = STAGED ? stage_ordered_elem(q * 16 + col) : q * 16 + col;
            store_elem(h, (size_t)(row0 + r) * g.I + ce, swiglu(gv, uv));
          }
        }
    } else {
#pragma unroll
      for (int mt = 0; mt < NMT; ++mt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int r = mt * 16 + rg + i;
          const int dr = __shfl(dst_row, r, kWave);
          if (r < M) {
            T* yrow = reinterpret_cast<T*>(g.ybuf) + (size_t)dr * g.H + (2 * q) * 16 + col;
            store_elem(yrow, 0, acc[p][mt][0][i]);
            store_elem(yrow, 16, acc[p][mt][1][i]);
          }
        }
    }
  }
}

}  // namespace mv
