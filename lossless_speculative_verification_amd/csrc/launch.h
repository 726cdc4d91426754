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
  int32_t* row_tok;
  int32_t* row_dst;
  float* row_gate;
  int4* work;
  int32_t* n_work;
  int32_t* counts;
};

// Arguments of the expert GEMMs and the LM head (see k_moe_gemm, k_lm_head in kernels.hip).
struct GemmArgs {
  const int4* work;        // work items (expert, first row, rows, first token); NULL for the LM head
  const int32_t* n_work;   // number of valid work items (device)
  const void* A;           // activation rows: UP a[T][H] (gathered), DOWN h[rows][I], LM a[T][H]
  const int32_t* row_tok;  // UP: token of each routed row
  const uint4* B;          // packed weights of this layer (pair layout)
  int K;                   // contraction length in elements
  int NQ;                  // column pairs (2 x 16 columns) per expert
  int n_valid;             // LM: vocabulary size (columns beyond it are padding)
  int Tn;                  // positions in this pass
  int k, E, KS, H, I;      // top-k, routed experts, k + shared, hidden, intermediate
  void* h;                 // UP out: h[rows][I]
  const int32_t* row_dst;  // DOWN: ybuf row of each routed row
  const float* row_gate;   // DOWN: gate of each routed row
  float* ybuf;             // DOWN out: ybuf[T][KS][H]
  Top2* part;              // LM out: part[T][n_pg]
  int n_pg;                // LM: workgroups along the vocabulary (each 4 * lm_ppw pairs)
  int lm_ppw;              // LM: column pairs per wavefront
  int ppw;                 // expert GEMMs: column pairs per wavefront (1 or 2)
  int max_items;           // expert GEMMs: capacity of the work list (grid covers max_items x chunks)
};

hipError_t launch_repack_pairs(const void* src0, const void* src1, void* dst, int n_mats, int N,
                               int row_bytes, int NQ, int NKB, int gate_up, size_t mat_stride_bytes,
                               hipStream_t stream);
hipError_t launch_repack_router(const void* src, void* dst, int L, int E, int row_bytes,
                                hipStream_t stream);
// Combine + residual + RMSNorm (+ router and top-k when route).
hipError_t launch_norm_route(int wdtype, bool route, const float* x_in, const float* ybuf, float* x_out,
                             float* x_copy, void* a_out, const void* wr, const float* bias,
                             int32_t* topk_id, float* topk_w, int Tn, int H, int KS, int E, int k,
                             float eps, hipStream_t stream);
hipError_t launch_plan(const PlanArgs& pa, hipStream_t stream);
// One-dimensional grid of n_wg workgroups (item x column-pair group, see k_gemm).
hipError_t launch_gemm(int wdtype, int epi, const GemmArgs& args, unsigned n_wg, hipStream_t stream);
// Positions per workgroup of the norm/router kernel and its dynamic LDS bytes.
int norm_positions_per_wg(int Tn);
size_t norm_lds_bytes(int wdtype, int H, int np);
hipError_t launch_argmax_reduce(const Top2* part, int n_pg, int Tn, int32_t* argmax, float* margin,
                                hipStream_t stream);
hipError_t launch_accept(const int32_t* drafts, const int32_t* argmax, int B, int K, int32_t* accepted,
                         int32_t* committed, hipStream_t stream);
hipError_t launch_combine(const float* ybuf, int Tn, int H, int KS, float* m, hipStream_t stream);

}  // namespace mv
