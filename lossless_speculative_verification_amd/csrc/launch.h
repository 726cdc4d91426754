// Internal launch interface between the C-ABI host code and the gfx950 kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "device_common.h"

namespace mv {

enum Epilogue { EPI_UP = 0, EPI_DOWN = 1, EPI_LM = 2 };

// Arguments of the routing plan (see plan_body in kernels.hip).
struct PlanArgs {
  const int32_t* topk_id;
  const float* topk_w;
  int Tn, k, E, S;
  int32_t* row_tok;   // out: token of each routed row
  int32_t* slot_row;  // out: routed row of each slot t*k + j
  int32_t* row_dst;   // out: position-major ybuf row t*(k+S) + j of each routed row
  int4* work;
  int32_t* n_work;
  int32_t* counts;
  int mb;              // rows per work item
  int32_t* chunk_cnt;  // [chunks][64] scratch of the large-pass plan, or NULL (one workgroup)
  // Split plan (one-workgroup plan only; hot_rows > 0): routed experts with fewer than
  // hot_rows rows get work items of mb2 rows in a second list (work2 / n_work2) for the
  // streaming unit of the tiled kernel; the others and the shared experts stay in work.
  int hot_rows;
  int mb2;
  int4* work2;
  int32_t* n_work2;
};

// Arguments of the expert GEMMs and the LM head (see k_moe_gemm, k_lm_head in kernels.hip).
struct GemmArgs {
  const int4* work;        // work items (expert, first row, rows, first token); NULL for the LM head
  const int32_t* n_work;   // number of valid work items (device)
  const void* A;           // activation rows: UP a[T][H] (gathered), DOWN h[rows][I], LM a[T][H]
  const int32_t* row_tok;  // UP: token of each routed row
  const int32_t* row_dst;  // streaming DOWN: position-major ybuf row of each routed row
  const uint4* B;          // packed weights of this layer (pair layout)
  int K;                   // contraction length in elements
  int NQ;                  // column pairs (2 x 16 columns) per expert
  int n_valid;             // LM: vocabulary size (columns beyond it are padding)
  int Tn;                  // positions in this pass
  int k, E, KS, H, I;      // top-k, routed experts, k + shared, hidden, intermediate
  void* h;                 // UP out: h[rows][I]
  void* ybuf;              // DOWN out: ybuf[rows][H] in the weight element type, one row per slot
  Top2* part;              // LM out: part[T][n_pg]
  int n_pg;                // LM: workgroups along the vocabulary (each 4 * lm_ppw pairs)
  int lm_ppw;              // LM: column pairs per wavefront
  int ppw;                 // expert GEMMs: column pairs per wavefront (1 or 2)
  int max_items;           // expert GEMMs: capacity of the work list (grid covers max_items x chunks)
  int sink_row;            // tiled expert GEMMs: row of h / ybuf that takes the stores of padding rows
  // Streaming gate/up that builds the routing plan itself (launch_gemm_planned): it reads
  // topk_id and writes the work list, item count, per-expert counts and row_dst that the
  // plan kernel would have written (for the down GEMM and the bench), with items of mb rows.
  const int32_t* topk_id;
  // Tiled kernel: streaming work items (split plan) run beside the tiles, or n_work2 NULL
  const int4* work2;
  const int32_t* n_work2;
  int4* plan_work;
  int32_t* plan_n_work;
  int32_t* plan_counts;
  int32_t* plan_row_dst;
  int mb;
};

hipError_t launch_repack_pairs(const void* src0, const void* src1, void* dst, int n_mats, int N,
                               int row_bytes, int NQ, int NKB, int gate_up, size_t mat_stride_bytes,
                               hipStream_t stream);
hipError_t launch_repack_router(const void* src, void* dst, int L, int E, int row_bytes,
                                hipStream_t stream);
// Combine of the previous block (gates from topk_w; ybuf rows position-major, t*(k+S) + j,
// when pos_major, else gathered through slot_row) + residual + RMSNorm (+ router and
// top-k when route, overwriting topk_id/topk_w); a_out in the stage-ordered row layout
// when perm_a (bf16 only).
hipError_t launch_norm_route(int wdtype, bool route, const float* x_in, const void* ybuf,
                             const int32_t* slot_row, float* x_out, float* x_copy, void* a_out, const void* wr,
                             const float* bias, int32_t* topk_id, float* topk_w, int Tn, int H, int S, int E,
                             int k, float eps, bool perm_a, bool pos_major, hipStream_t stream);
// Routing plan: one workgroup for up to kPlanSingleMaxChunks chunks of kPlanChunk slots
// (or when chunk_cnt is NULL), else a count pass and a scatter pass of one workgroup
// per chunk.
hipError_t launch_plan(const PlanArgs& pa, hipStream_t stream);
int plan_chunks(int Tn, int k);
// One-dimensional grid of n_wg workgroups (item x column-pair group, see k_moe_gemm; LM head: k_lm_head).
hipError_t launch_gemm(int wdtype, int epi, const GemmArgs& args, unsigned n_wg, hipStream_t stream);
// Gate/up of the streaming path with the plan built in its prologue (no launch_plan), for
// passes of at most kSelfPlanMaxSlots routed slots; same grid as launch_gemm(EPI_UP).
hipError_t launch_gemm_planned(int wdtype, const GemmArgs& args, unsigned n_wg, hipStream_t stream);
// LDS-tiled expert GEMM (bf16) over work items of up to kTileM rows and
// tiled_tiles_per_item(NQ) column tiles each; n_wg persistent workgroups (one per compute
// unit) share the tiles. Needs K >= 256 elements.
hipError_t launch_gemm_tiled(int epi, const GemmArgs& args, unsigned n_wg, hipStream_t stream);
int tiled_tiles_per_item(int NQ);
// Positions per workgroup of the split norm/router kernel (passes below
// kNormSplitMaxPositions) and the norm kernels' dynamic LDS bytes.
int norm_split_positions(int Tn);
size_t norm_lds_bytes(int wdtype, int H, int np);
hipError_t launch_argmax_reduce(const Top2* part, int n_pg, int Tn, int32_t* argmax, float* margin,
                                hipStream_t stream);
hipError_t launch_accept(const int32_t* drafts, const int32_t* argmax, int B, int K, int32_t* accepted,
                         int32_t* committed, hipStream_t stream);
// m[t] = sum_j gate[t][j] * y(t, j) + sum_s y(t, k + s), with y(t, j) = ybuf[t*(k+S) + j]
// when pos_major, else ybuf[slot_row[t*k + j]] (j < k) and ybuf[T*k + s*T + t] (shared);
// ybuf holds the weight element type (bf16 when wdtype is 1).
hipError_t launch_combine(int wdtype, const void* ybuf, const int32_t* slot_row, const float* gate, int Tn, int H,
                          int k, int S, bool pos_major, float* m, hipStream_t stream);

// Test hook: row_slot[r] = slot t*k + j of routed row r, from its position-major
// expert-output row row_dst[r] = t*KS + j (n = T*k rows).
hipError_t launch_row_slot(const int32_t* row_dst, int n, int k, int KS, int32_t* row_slot, hipStream_t stream);

// Draft block (draft.hip). Input rows of draft step `step` for B sequences (one
// workgroup each): U[b] = [RMSNorm(h_b), RMSNorm(E[t_b])] in the weight type, with h_b, t_b
// the verifier pass's last accepted row (step 0) or the previous step's output hidden
// state and draft (step > 0, which also stores drafts[b][step-1]); E = the LM head in its
// pair layout (NKB K blocks per pair). H <= 4096.
hipError_t launch_draft_input(int wdtype, const float* hidden, const int32_t* accepted, const int32_t* committed,
                              int Kv, const float* z_prev, const int32_t* ids_prev, int32_t* drafts, int K, int step,
                              const void* lm, int NKB, int H, int V, float eps, void* U, int B, hipStream_t stream);
// Work list of ceil(B / mb) row blocks of one always-on expert (expert index 0).
hipError_t launch_draft_plan(int4* work, int32_t* n_work, int B, int mb, hipStream_t stream);
// drafts[b][K-1] = ids[b].
hipError_t launch_draft_store(const int32_t* ids, int32_t* drafts, int B, int K, hipStream_t stream);
// p[0..n) = v.
hipError_t launch_fill(float* p, size_t n, float v, hipStream_t stream);

}  // namespace mv
