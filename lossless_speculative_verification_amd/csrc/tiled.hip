// Expert GEMMs for passes with many positions per expert (prefill-sized passes):
// an LDS-tiled grouped MFMA GEMM over work items of up to kTileM rows of one expert.
//
// The products are those of the verify step's MoE block (pages: "jina-ocr-v1" model page,
// architecture paragraph: 64 routed + 2 shared SwiGLU experts, top-6 routing):
//   UP:   h = bf16(silu(A W_gate^T) * (A W_up^T)) for the expert's rows of A
//   DOWN: y = bf16(h W_down^T), written to the same row of ybuf as the row of h
// with the same row space, work list, outputs and float32 accumulation as the
// streaming kernels (k_moe_gemm), so either path can run any block. The same kernel also
// runs the LM head of large passes (pages: model page, summary paragraph: greedy choice
// over a 129,280-word vocabulary):
//   LM:   per 256-row item and 256-column tile, the top-1/top-2 record of every row of
//         A W_lm^T (float32 logits, never stored), merged later by k_argmax_reduce.
// With a split plan (cold experts in a second work list of 32-row items) the kernel also
// runs those items with the streaming unit, on compute units without tiles first.
#include <type_traits>

#include "launch.h"
#include "stream_gemm.h"

namespace mv {

// Tile: kTileM rows x kTilePairs column pairs (256 output columns; for UP the pairs are
// (gate tile q, up tile q), i.e. 128 intermediate columns). 8 wavefronts (two per SIMD)
// in a 2 x 4 grid: wavefront (wm, wn) owns rows 128*wm.. and the pairs 2*wn, 2*wn + 1,
// i.e. 8 x 4 MFMA tiles of 16x16 (128 accumulator registers).
//
// The contraction advances one MFMA step (32 elements) per stage: stage st is step
// s = st % 4 of the 256-byte K block kb = st / 4 of the pair layout, in which lane group
// g = l / 16 contracts the 16-byte chunk g*4 + s of the block. LDS holds a stage as
// 16-byte units in exactly the order the MFMA reads them:
//   A unit (mt, l):   row 16*mt + l % 16 of the item, chunk (l/16)*4 + s of block kb
//   B unit (p, t, l): pair-layout unit (t, s, l) of block kb of pair p of the tile
// so every LDS read of a wavefront is 1 KB contiguous (no bank conflicts), and every
// 1 KB run is filled by one wavefront-wide direct global-to-LDS load (lane l's 16 bytes
// land at unit l of the run): wavefront w fills A row tiles w and w + 8 and the B runs
// (p, t) = ((w + 8r) / 2, w % 2), r = 0, 1 — four loads per wavefront per stage.
//
// The MFMA takes the weights as its first operand and the activations as its second, so
// lane l of a 16x16 result holds position 16*i + l % 16 and the four consecutive output
// columns 4*(l/16)..+3; the epilogue pairs two such results with one lane swap and stores
// 16 bytes per lane, no LDS round trip.
//
// Pipeline: kTileStages = 4 LDS stages in a ring. Step st multiplies stage st from
// registers while stage st + 1's operands are read from LDS and stages st + 2 .. st + 4
// are in flight to LDS: after waiting for this wavefront's loads of stage st + 1 and its
// LDS reads of stage st, a barrier makes stage st + 1 visible and frees the slot of
// stage st, into which stage st + 4 is requested. The loads write LDS without passing
// through registers, so the registers hold only the accumulators and two steps'
// operands. The waits are explicit (the compiler does not count these loads), and the
// barrier is a plain s_barrier that is also a compiler memory barrier: no load or LDS
// access moves across it, and it does not wait for the loads in flight.
constexpr int kTilePairs = 8;
constexpr int kTileThreads = 512;
constexpr int kTileStages = 4;
constexpr int kRunUnits = kWave;       // 16-byte units per 1 KB run
constexpr int kStageRuns = 16;         // runs per operand per stage
constexpr int kLoadsPerStage = 4;      // direct loads per wavefront per stage
constexpr int kUpStores = 8;           // epilogue stores per wavefront: UP 8 row tiles
constexpr int kDownStores = 16;        //   DOWN 8 row tiles x 2 pairs
constexpr int kLmStores = 1;           //   LM one merged record per lane

// s_waitcnt for at most N vector-memory operations of this wavefront still in flight and
// none of its LDS operations (expcnt left unconstrained).
template <int N>
__device__ __forceinline__ void wait_vmem_lds() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (0 << 8) | ((N >> 4) << 14));
}
__device__ __forceinline__ void block_barrier() { asm volatile("s_barrier" ::: "memory"); }
// Direct global-to-LDS loads (lane l's 16 or 4 bytes land at lds + 16*l or 4*l; lds is
// wavefront-uniform and goes to M0). Written as assembly so that the compiler does not
// track them: it would otherwise drain every such load in flight before any LDS read it
// cannot prove disjoint from them. Their completion is covered by the explicit waits
// above; M0 is used by nothing else in these kernels.
__device__ __forceinline__ void lds_load16(const void* gptr, const void* lds) {
  const uint32_t m0 = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)lds);
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, off" ::"s"(m0), "v"(gptr) : "memory", "m0");
}
__device__ __forceinline__ void lds_load4(const void* gptr, const void* lds) {
  const uint32_t m0 = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)lds);
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dword %1, off" ::"s"(m0), "v"(gptr) : "memory", "m0");
}
// Two float32 values to a packed pair of bf16 (round to nearest even, one instruction).
typedef float f32x2_cv_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2_cv_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2_cv_t){a, b}, bf16x2_cv_t));
}
__device__ __forceinline__ void sched_fence() { __builtin_amdgcn_sched_barrier(0); }

template <int EPI>
__global__ __launch_bounds__(kTileThreads, 1) void k_moe_tiled(GemmArgs g) {
  constexpr int NST = EPI == EPI_UP ? kUpStores : (EPI == EPI_DOWN ? kDownStores : kLmStores);
  constexpr int STAGE2 = 2 * kLoadsPerStage;  // loads of two stages
  constexpr int WAVES = kTileThreads / kWave;
  __shared__ u32x4_t lds[kTileStages][2][kStageRuns * kRunUnits];
  // A source rows of this wavefront's two runs (lanes 0..15 run w, 16..31 run w + 8), for
  // the tiles of even and odd index
  __shared__ int rows_lds[2][WAVES][kWave];
  // LM: the four column wavefronts' records of each row of the tile
  __shared__ Top2 lm_red[EPI == EPI_LM ? 4 : 1][EPI == EPI_LM ? kTileM : 1];
  const int NT = (g.NQ + kTilePairs - 1) / kTilePairs;
  // LM: no work list, the items are the consecutive 256-row blocks of the Tn rows
  const int n_items = EPI == EPI_LM ? (g.Tn + kTileM - 1) / kTileM : *g.n_work;
  // Down GEMM whose tiles, twice over, and streaming items still fit one round of the
  // device (small skewed passes): every item is run as two 128-row halves, so twice the
  // compute units share it; in a half tile the wavefronts of rows 128..255 hold only
  // padding and skip their products. Such a launch gives every workgroup at most one tile.
  bool half = false;
  if constexpr (EPI == EPI_DOWN) {
    const int units = g.n_work2 ? *g.n_work2 * g.NQ : 0;
    half = 2 * n_items * NT + (units + 7) / 8 <= (int)gridDim.x;
  }
  const int n_tiles = n_items * NT * (half ? 2 : 1);
  // This workgroup's tiles: XCD x (hardware workgroups are dealt to the 8 XCDs in turn)
  // owns the x-th contiguous range of logical tiles, and its nbx workgroups take every
  // nbx-th tile of it, so at any time one XCD works on neighbouring tiles (the row
  // blocks and column groups of one expert) that share its L2.
  const int x = blockIdx.x & 7, jx = blockIdx.x >> 3;
  const int nbx = ((int)gridDim.x - x + 7) >> 3;
  int start = 0;
  for (int y = 0; y < x; ++y) start += (n_tiles - y + 7) >> 3;
  const int cnt = (n_tiles - x + 7) >> 3;
  const int n_my = jx < cnt ? (cnt - jx + nbx - 1) / nbx : 0;
  do {  // the tiles of this workgroup (none: straight to the streaming items)
  if (n_my == 0) break;  // workgroup-uniform

  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int row_units = g.K * 2 / 16;  // 16-byte units per activation row
  const int NKB = row_units / kChunksPerRow;
  const int nst = 4 * NKB;             // stages (steps) per tile, a multiple of 4, >= 8
  const int total = n_my * nst;        // steps of this workgroup
  const char* Ab = reinterpret_cast<const char*>(g.A);
  const char* Bb = reinterpret_cast<const char*>(g.B);
  const uint32_t row_bytes = (uint32_t)row_units * 16u;

  // Tile m of this workgroup: expert, first row, rows, first token, column tile (all
  // wavefront-uniform).
  struct TileInfo {
    int e, row0, M, tok0, nt;
  };
  auto info = [&](int m) __attribute__((always_inline)) {
    const int lt = start + jx + m * nbx;
    if constexpr (EPI == EPI_LM) {
      // column-tile major: the row items of one column tile are neighbours on one XCD and
      // share its weight tile through L2
      const int nt = __builtin_amdgcn_readfirstlane(lt / n_items), item = lt - nt * n_items;
      return TileInfo{0, item * kTileM, min(kTileM, g.Tn - item * kTileM), item * kTileM, nt};
    } else {
      // half: item-major, the two halves' column tiles after each other
      const int per = half ? 2 * NT : NT;
      const int item = __builtin_amdgcn_readfirstlane(lt / per);
      const int nt = lt - item * per, hf = nt >= NT ? 1 : 0;
      // the work list is not written while the kernel runs: read it as constant memory
      // (a scalar load, which the waits for the direct loads do not count)
      typedef int i32x4_t __attribute__((ext_vector_type(4)));
      typedef const __attribute__((address_space(4))) i32x4_t* const_work_ptr;
      const i32x4_t it = ((const_work_ptr)(uintptr_t)g.work)[item];
      if (!half) return TileInfo{it[0], it[1], it[2], it[3], nt};
      const int h0 = (kTileM / 2) * hf;  // a second half of no rows has M <= 0
      return TileInfo{it[0], it[1] + h0, min(kTileM / 2, it[2] - h0), it[3] + h0, nt - hf * NT};
    }
  };
  // The A source rows of tile t into rows_lds[buf][w]: lane l < 32 holds the row of row
  // (w + 8*(l/16))*16 + l%16 of the item (rows past its end repeat its last row; their
  // results go to the sink row). Routed gate/up rows come from row_tok through one 4-byte
  // direct load (lanes 32..63 repeat lanes 0..31); other rows are consecutive.
  auto set_rows = [&](const TileInfo& t, int buf) __attribute__((always_inline)) {
    const int rr = min((w + 8 * ((lane >> 4) & 1)) * 16 + (lane & 15), t.M - 1);
    if (EPI == EPI_UP && t.e < g.E) {
      lds_load4(g.row_tok + t.row0 + rr, &rows_lds[buf][w][0]);
    } else {
      rows_lds[buf][w][lane] = (EPI == EPI_UP ? t.tok0 : t.row0) + rr;
    }
  };
  // Stage st of tile t (rows src0/src1 of its two A runs): B from the tile's pairs (pairs
  // past the last repeat it; not stored). Wavefront-uniform base plus a 32-bit per-lane
  // offset (every operand buffer is below 4 GiB).
  auto issue_a = [&](int src0, int src1, int stage) __attribute__((always_inline)) {
    const int kb = stage >> 2, s = stage & 3, slot = stage & (kTileStages - 1);
    const uint32_t ka = (uint32_t)(((lane >> 4) + kb * kChunksPerRow + 4 * s) * 16);
    lds_load16(Ab + ((uint32_t)src0 * row_bytes + ka), &lds[slot][0][w * kRunUnits]);
    lds_load16(Ab + ((uint32_t)src1 * row_bytes + ka), &lds[slot][0][(w + 8) * kRunUnits]);
  };
  auto issue_b = [&](const TileInfo& t, int stage) __attribute__((always_inline)) {
    const int kb = stage >> 2, s = stage & 3, slot = stage & (kTileStages - 1);
    const int q0 = min(t.nt * kTilePairs + (w >> 1), g.NQ - 1);
    const int q1 = min(t.nt * kTilePairs + ((w + 8) >> 1), g.NQ - 1);
    const size_t bk = (size_t)kb * kPairUnits + s * kWave + (w & 1) * 4 * kWave;
    const size_t b0 = ((size_t)t.e * g.NQ + q0) * (size_t)NKB * kPairUnits + bk;
    const size_t b1 = ((size_t)t.e * g.NQ + q1) * (size_t)NKB * kPairUnits + bk;
    const uint32_t lo = (uint32_t)lane * 16u;
    lds_load16(Bb + b0 * 16 + lo, &lds[slot][1][w * kRunUnits]);
    lds_load16(Bb + b1 * 16 + lo, &lds[slot][1][(w + 8) * kRunUnits]);
  };
  auto issue = [&](const TileInfo& t, int src0, int src1, int stage) __attribute__((always_inline)) {
    issue_a(src0, src1, stage);
    issue_b(t, stage);
  };

  const int wm = w >> 2, wn = w & 3;
  f32x4_t acc[8][2][2];
  auto clear = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
      for (int pp = 0; pp < 2; ++pp) acc[i][pp][0] = acc[i][pp][1] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  };
  // operands of one step (A row tiles 8*wm + i, B tiles (2*wn + pp, t)), two sets
  u32x4_t fa[2][8], fb[2][2][2];
  auto read = [&](u32x4_t(&a)[8], u32x4_t(&b)[2][2], int stage) __attribute__((always_inline)) {
    const int slot = stage & (kTileStages - 1);
#pragma unroll
    for (int pp = 0; pp < 2; ++pp)
#pragma unroll
      for (int t = 0; t < 2; ++t) b[pp][t] = lds[slot][1][((2 * wn + pp) * 2 + t) * kRunUnits + lane];
#pragma unroll
    for (int i = 0; i < 8; ++i) a[i] = lds[slot][0][(8 * wm + i) * kRunUnits + lane];
  };
  // the 8 products of row tiles i0 and i0 + 1
  auto mma_rows = [&](const u32x4_t(&a)[8], const u32x4_t(&b)[2][2], int i0) __attribute__((always_inline)) {
#pragma unroll
    for (int i = i0; i < i0 + 2; ++i)
#pragma unroll
      for (int pp = 0; pp < 2; ++pp)
#pragma unroll
        for (int t = 0; t < 2; ++t)
          acc[i][pp][t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, b[pp][t]),
                                                                  __builtin_bit_cast(bf16x8_t, a[i]),
                                                                  acc[i][pp][t], 0, 0, 0);
  };
  // Every lane issues exactly NST 16-byte stores (rows past the item's end and columns past
  // the last go to the sink row), so the in-flight counts the waits rely on are exact. Lane
  // group gq = l / 16 of a 16x16 result holds columns 4*gq..+3 of position l % 16; one
  // permlane16 swap between two such results (gate/up: the wavefront's two pairs; down: the
  // two 16-column tiles of a pair) leaves each lane 8 consecutive columns, so a store
  // instruction writes 16 positions x 64 contiguous bytes instead of 16 x 32 bytes twice.
  auto epilogue = [&](const TileInfo& t) __attribute__((always_inline)) {
    const int gq = lane >> 4;
    if constexpr (EPI == EPI_LM) {
      // Each lane folds its 16 logits of a row in increasing column order (a later equal
      // value never wins), the four lane groups and then the four column wavefronts are
      // merged (lowest index on equal values), and lane l < 32 of wavefront w stores row
      // 32 w + l's record of this column tile. Every lane stores exactly once: lanes with
      // no row of the item write the record slot past the last one.
      const float NEG = -__builtin_huge_valf();
      // columns past the vocabulary (only in the last column tile) never enter a record
      // A lane's 16 values of a row: the largest and second largest of the multiset by
      // running max / median-of-three (order-free), then the lowest column holding the
      // largest, by a scan from the highest column down. The same record as folding the
      // values one by one in column order (top2_push), in about half the instructions.
      auto fold = [&](auto checked) __attribute__((always_inline)) {
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          float v[16];
          bool ok[16];
#pragma unroll
          for (int u = 0; u < 16; ++u) {  // u = 8 pp + 4 tt + j: increasing columns
            const int pp = u >> 3, tt = (u >> 2) & 1, j = u & 3;
            const int q = t.nt * kTilePairs + 2 * wn + pp, c = (2 * q + tt) * 16 + 4 * gq + j;
            ok[u] = !decltype(checked)::value || ((q < g.NQ) & (c < g.n_valid));
            v[u] = ok[u] ? acc[i][pp][tt][j] : NEG;
          }
          float v1 = NEG, v2 = NEG;
#pragma unroll
          for (int u = 0; u < 16; ++u) {
            v2 = __builtin_amdgcn_fmed3f(v1, v2, v[u]);
            v1 = __builtin_amdgcn_fmed3f(v1, v[u], __builtin_huge_valf());
          }
          int i1 = INT_MAX;
#pragma unroll
          for (int u = 15; u >= 0; --u) {
            const int pp = u >> 3, tt = (u >> 2) & 1, j = u & 3;
            const int c = (2 * (t.nt * kTilePairs + 2 * wn + pp) + tt) * 16 + 4 * gq + j;
            i1 = (ok[u] & (v[u] == v1)) ? c : i1;
          }
          Top2 b{v1, v1 > NEG ? i1 : INT_MAX, v2};  // no value above -inf: no column, as one by one
          b = top2_merge(b, top2_shfl_xor(b, 16));
          b = top2_merge(b, top2_shfl_xor(b, 32));
          if (lane < 16) lm_red[wn][128 * wm + 16 * i + lane] = b;
        }
      };
      if ((t.nt + 1) * kTilePairs * 32 <= g.n_valid) fold(std::false_type{});  // workgroup-uniform
      else fold(std::true_type{});
      wait_vmem_lds<63>();  // this wavefront's LDS writes done (loads in flight stay)
      block_barrier();
      const int r = 32 * w + (lane & 31);
      Top2 rec = lm_red[0][r];
#pragma unroll
      for (int v = 1; v < 4; ++v) rec = top2_merge(rec, lm_red[v][r]);
      const size_t slot = lane < 32 && r < t.M ? (size_t)(t.row0 + r) * g.n_pg + t.nt : (size_t)g.Tn * g.n_pg;
      g.part[slot] = rec;
    } else {
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int r = 128 * wm + 16 * i + (lane & 15);
        const bool row_ok = r < t.M;
        if constexpr (EPI == EPI_UP) {
          uint32_t lo[2], hi[2];  // bf16 pairs of columns 4*gq, 4*gq+1 and 4*gq+2, 4*gq+3 of pair pp
#pragma unroll
          for (int pp = 0; pp < 2; ++pp) {
            float sv[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) sv[j] = swiglu(acc[i][pp][0][j], acc[i][pp][1][j]);
            lo[pp] = pack_bf16x2(sv[0], sv[1]);
            hi[pp] = pack_bf16x2(sv[2], sv[3]);
          }
          // lane group gq now holds columns 8*(gq/2)..+7 of pair 2*wn + gq%2
          const auto xl = __builtin_amdgcn_permlane16_swap(lo[0], lo[1], false, false);
          const auto xh = __builtin_amdgcn_permlane16_swap(hi[0], hi[1], false, false);
          const int q = t.nt * kTilePairs + 2 * wn + (gq & 1);
          const int e = q * 16 + 8 * (gq >> 1);
          const size_t off = row_ok && q < g.NQ ? (size_t)(t.row0 + r) * g.I + stage_ordered_elem(e)
                                                : (size_t)g.sink_row * g.I;
          *reinterpret_cast<uint4*>(reinterpret_cast<uint16_t*>(g.h) + off) =
              make_uint4((uint32_t)xl[0], (uint32_t)xh[0], (uint32_t)xl[1], (uint32_t)xh[1]);
        } else {
#pragma unroll
          for (int pp = 0; pp < 2; ++pp) {
            const int q = t.nt * kTilePairs + 2 * wn + pp;
            const uint32_t d0 = pack_bf16x2(acc[i][pp][0][0], acc[i][pp][0][1]);
            const uint32_t d1 = pack_bf16x2(acc[i][pp][0][2], acc[i][pp][0][3]);
            const uint32_t e0 = pack_bf16x2(acc[i][pp][1][0], acc[i][pp][1][1]);
            const uint32_t e1 = pack_bf16x2(acc[i][pp][1][2], acc[i][pp][1][3]);
            // lane group gq now holds columns 8*(gq/2)..+7 of the pair's tile gq%2
            const auto x0 = __builtin_amdgcn_permlane16_swap(d0, e0, false, false);
            const auto x1 = __builtin_amdgcn_permlane16_swap(d1, e1, false, false);
            const int col = (2 * q + (gq & 1)) * 16 + 8 * (gq >> 1);
            const size_t off = row_ok && q < g.NQ && col < g.H ? (size_t)(t.row0 + r) * g.H + col
                                                               : (size_t)g.sink_row * g.H;
            *reinterpret_cast<uint4*>(reinterpret_cast<uint16_t*>(g.ybuf) + off) =
                make_uint4((uint32_t)x0[0], (uint32_t)x1[0], (uint32_t)x0[1], (uint32_t)x1[1]);
          }
        }
      }
    }
  };

  // prologue: tile 0's rows requested, then the weights of stages 0..2 (they need no row
  // index, so they are in flight while the rows arrive); once the rows are in, the
  // activations of stages 0..2; once stage 0 is in, stage 3 too, and stage 0 read; then
  // the wait for stage 1 that the first step expects (its count assumes whole stages
  // issued in order, which the prologue's split order is not)
  TileInfo cur = info(0), nxt = cur;
  if (half && cur.M <= 0) break;  // the empty second half of a short item (its only tile)
  if (n_my > 1) nxt = info(1);
  set_rows(cur, 0);
  issue_b(cur, 0);
  issue_b(cur, 1);
  issue_b(cur, 2);
  wait_vmem_lds<6>();  // the rows' load (before the six weight loads) is in
  int src0 = rows_lds[0][w][lane & 15], src1 = rows_lds[0][w][16 + (lane & 15)];
  clear();
  issue_a(src0, src1, 0);
  issue_a(src0, src1, 1);
  issue_a(src0, src1, 2);
  wait_vmem_lds<4>();  // stage 0 in: its activations, and everything issued before them
  block_barrier();
  issue(cur, src0, src1, 3);
  read(fa[0], fb[0], 0);
  wait_vmem_lds<6>();  // stage 1 in: after its activations only stage 2's (2) and stage 3 (4)

  // Step gs (tile m, step st of it): wait for this wavefront's loads of stage gs + 1 (the
  // loads issued after them may stay in flight: two stages, plus the previous tile's
  // stores in the first three steps of a tile) and for its LDS reads, barrier, then
  // multiply stage gs while reading stage gs + 1's operands and the A rows of the stage to
  // request, and request stage gs + 4 into the slot stage gs freed. The scheduling fences
  // keep that order (the compiler would otherwise pull each read next to its first use,
  // and move the requests). At step 0
  // of tile m the rows of tile m + 1 are set (in by step 3, before its first request);
  // the last step of a tile ends with its epilogue.
  int m = 0, st = 0;
  for (int gs = 0; gs < total; gs += 2) {
    static_for<2>([&](auto sc) __attribute__((always_inline)) {
      constexpr int u = decltype(sc)::value;
      const int gcur = gs + u;
      const bool request = gcur + 4 < total;  // workgroup-uniform
      const bool own = st + 4 < nst;  // the stage to request is this tile's, else the next's
      // (the last step reads a stage it does not use: every read stays inside LDS)
      const int left = total - 2 - gcur;  // stages issued after stage gcur + 1, at most 2
      if (m > 0 && st < 3) {
        if constexpr (STAGE2 + NST < 63) wait_vmem_lds<STAGE2 + NST>();
        else wait_vmem_lds<63>();
      } else if (left >= 2) {
        wait_vmem_lds<STAGE2>();
      } else if (left == 1) {
        wait_vmem_lds<kLoadsPerStage>();
      } else {
        wait_vmem_lds<0>();
      }
      block_barrier();
      const int buf = (m + (own ? 0 : 1)) & 1;
      const int r0 = rows_lds[buf][w][lane & 15], r1 = rows_lds[buf][w][16 + (lane & 15)];
      const int slot1 = (st + 1) & (kTileStages - 1);
      // (down: a wavefront whose 128 rows are all padding skips its products; its operand
      // reads and requests stay, as every wavefront's loads fill the shared stage)
      // Stage gs + 1's 12 operand reads interleaved with stage gs's 32 products (about one
      // read per two products, so the reads and the address arithmetic fill the matrix
      // pipe's busy cycles), and the requests of stage gs + 4 placed between the products:
      // the activation runs after 8 of them, the weight runs after 16. Requested after all
      // 32 (when every wavefront of the compute unit sends its four loads at once) the
      // steps ran 1-3 % slower.
#pragma unroll
      for (int pp = 0; pp < 2; ++pp)
#pragma unroll
        for (int t = 0; t < 2; ++t) fb[u ^ 1][pp][t] = lds[slot1][1][((2 * wn + pp) * 2 + t) * kRunUnits + lane];
      if (EPI != EPI_DOWN || 128 * wm < cur.M) mma_rows(fa[u], fb[u], 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);  // the two row-index reads
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);  // two MFMA
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // one LDS read
      }
      sched_fence();
      if (request) issue_a(r0, r1, own ? st + 4 : st + 4 - nst);
      sched_fence();
#pragma unroll
      for (int i = 0; i < 4; ++i) fa[u ^ 1][i] = lds[slot1][0][(8 * wm + i) * kRunUnits + lane];
      if (EPI != EPI_DOWN || 128 * wm < cur.M) mma_rows(fa[u], fb[u], 2);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      }
      sched_fence();
      if (request) {
        if (own) issue_b(cur, st + 4);
        else issue_b(nxt, st + 4 - nst);
      }
      sched_fence();
#pragma unroll
      for (int i = 4; i < 8; ++i) fa[u ^ 1][i] = lds[slot1][0][(8 * wm + i) * kRunUnits + lane];
      if (EPI != EPI_DOWN || 128 * wm < cur.M) mma_rows(fa[u], fb[u], 4);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      }
      sched_fence();
      if (EPI != EPI_DOWN || 128 * wm < cur.M) mma_rows(fa[u], fb[u], 6);
      sched_fence();
      if (st == 0 && m + 1 < n_my) set_rows(nxt, (m + 1) & 1);
      if (++st == nst) {  // workgroup-uniform: tile m done
        epilogue(cur);
        clear();
        st = 0;
        ++m;
        cur = nxt;
        if (m + 1 < n_my) nxt = info(m + 1);
      }
    });
  }
  } while (0);

  // Streaming work items of a split plan (cold experts, items of up to 32 rows): one
  // wavefront per (item, column pair) unit, no LDS and no barrier. Workgroups
  // without tiles take the first round of units, then every workgroup takes units in
  // turn (those without tiles first), so the units fill the compute units the tiles
  // leave idle before they wait behind tiles.
  if constexpr (EPI != EPI_LM) {
    if (g.n_work2 != nullptr) {
      const int units = *g.n_work2 * g.NQ;  // one column pair per unit
      const int wv = __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6);
      // workgroups without tiles (n_free; this one's index among them f, else its index
      // among those with tiles t_idx), from the same per-XCD dealing as the tiles
      int n_free = 0, f = -1, t_idx = 0;
      for (int y = 0; y < 8; ++y) {
        const int nb_y = ((int)gridDim.x - y + 7) >> 3, c_y = (n_tiles - y + 7) >> 3;
        if (y == x) {
          if (jx >= c_y) f = n_free + (jx - c_y);
          else t_idx += jx;
        }
        if (y < x) t_idx += min(nb_y, c_y);
        n_free += max(0, nb_y - c_y);
      }
      // this wavefront's units: u0 (tile-free workgroups' round 0), then u1, u1 + G8, ...
      const int G8 = (int)gridDim.x * 8;
      int u0, u1;
      if (n_free == 0) {
        u0 = units;
        u1 = (int)blockIdx.x * 8 + wv;
      } else {
        // place in the order of all wavefronts, tile-free workgroups first
        const int slot = f >= 0 ? f * 8 + wv : (n_free + t_idx) * 8 + wv;
        u0 = f >= 0 ? slot : units;
        u1 = n_free * 8 + slot;
      }
      for (int u = u0 < units ? u0 : u1; u < units; u = (u == u0 ? u1 : u + G8)) {
        const int item = u / g.NQ, q = u - item * g.NQ;
        const int4 it = g.work2[item];
        moe_stream<uint16_t, EPI, 2, 1, MV_GEMM_D + 1, true>(g, it.x, it.y, it.z, it.w, q);
      }
    }
  }
}

int tiled_tiles_per_item(int NQ) { return (NQ + kTilePairs - 1) / kTilePairs; }

// n_wg: one workgroup per compute unit (each holds 128 KB of LDS); the workgroups walk
// the tile list themselves.
hipError_t launch_gemm_tiled(int epi, const GemmArgs& args, unsigned n_wg, hipStream_t stream) {
  const dim3 grid(n_wg), block(kTileThreads);
  if (epi == EPI_UP) k_moe_tiled<EPI_UP><<<grid, block, 0, stream>>>(args);
  else if (epi == EPI_DOWN) k_moe_tiled<EPI_DOWN><<<grid, block, 0, stream>>>(args);
  else k_moe_tiled<EPI_LM><<<grid, block, 0, stream>>>(args);
  return hipGetLastError();
}

}  // namespace mv
