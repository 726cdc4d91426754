// Host side of the C ABI declared in include/moe_verify.h.
//
// Every entry point checks its arguments on the host before any HIP call, reports
// failures as status codes plus a thread-local message, and only enqueues work on the
// caller's stream during a step (no allocation, synchronisation or host copy there).
#include <cstdarg>
#include <cstdio>
#include <algorithm>
#include <cstring>
#include <mutex>
#include <string>
#include <type_traits>
#include <vector>

#include "launch.h"
#include "moe_verify.h"

#define MV_API extern "C" __attribute__((visibility("default")))

namespace {

thread_local std::string g_last_error;

int fail(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return code;
}

int ok() {
  g_last_error.clear();
  return MOE_OK;
}

int elem_bytes(int32_t wdtype) { return wdtype == MOE_BF16 ? 2 : 4; }

// Elements per 256-byte K block: the contraction granule of the packed GEMM layout.
int kblock_elems(int32_t wdtype) { return mv::kRowBlockBytes / elem_bytes(wdtype); }

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Upper bound on GEMM work items of at most mb rows for T positions (each routed
// expert's rows split in blocks of mb, plus at most one partial block per expert, plus
// the shared blocks).
int64_t max_work_items(const moe_verify_config& c, int64_t T, int64_t mb = mv::kGemmMB) {
  return (T * c.top_k + mb - 1) / mb + c.n_routed + (int64_t)c.n_shared * ((T + mb - 1) / mb);
}

// Split plan of tiled passes planned by one workgroup: routed experts with fewer than
// kSplitHotRows rows go to the tiled kernel's streaming unit in items of kSplitRows rows
// (a mostly empty 256 x 256 tile costs a compute unit as long as a full one, and the
// streaming unit reads the expert's weights once per 32 rows instead). At most
// ceil((kSplitHotRows - 1) / kSplitRows) items per routed expert.
constexpr int kSplitHotRows = 64;
constexpr int kSplitRows = 32;
int64_t max_split_items(const moe_verify_config& c) {
  return (int64_t)c.n_routed * ((kSplitHotRows - 1 + kSplitRows - 1) / kSplitRows);
}

// Passes of at least this many positions run the expert GEMMs on the LDS-tiled kernel
// (bf16 weights, contractions of at least 256 elements): work items of up to kTileM rows
// then keep the matrix cores busy, while smaller passes are bound by the weight stream
// and use the streaming kernel.
#ifndef MV_TILED_MIN_POSITIONS
#define MV_TILED_MIN_POSITIONS 256
#endif
bool use_tiled(const moe_verify_config& c, int Tn) {
  return c.wdtype == MOE_BF16 && Tn >= MV_TILED_MIN_POSITIONS && c.hidden >= 256 && c.inter >= 256;
}
// The LM head runs on the tiled GEMM (k_moe_tiled<EPI_LM>, 256-row items) from 256 rows on,
// except between 257 and 384 rows (a second item at most half full): beyond two 128-row
// blocks the streaming LM head is bound by LDS reads rather than by the weight stream, while
// a tiled round costs the same for a half-empty item. Measured (one MI355X, full vocabulary,
// tiled vs streaming): 256 rows 99 vs 117 us, 384: 168 vs 164, 448: 167 vs 220, 512: 169 vs
// 215, 640: 238 vs 256, 768: 242 vs 299.
bool use_tiled_lm(const moe_verify_config& c, int Tv) {
  const int r = Tv % mv::kTileM;
  const bool half_empty_second = Tv < 2 * mv::kTileM && r > 0 && 2 * r <= mv::kTileM;
  return c.wdtype == MOE_BF16 && c.vocab > 0 && c.hidden >= 256 && Tv >= mv::kTileM && !half_empty_second;
}

int check_config(const moe_verify_config* c) {
  if (!c) return fail(MOE_EINVAL, "config is NULL");
  if (c->wdtype != MOE_F32 && c->wdtype != MOE_BF16) return fail(MOE_EINVAL, "wdtype %d is not MOE_F32 or MOE_BF16", c->wdtype);
  if (c->hidden <= 0 || c->inter <= 0 || c->n_layers <= 0 || c->n_routed <= 0 || c->top_k <= 0 ||
      c->n_shared < 0 || c->vocab < 0 || c->max_positions <= 0)
    return fail(MOE_EINVAL, "config has a non-positive size (hidden %d inter %d layers %d routed %d top_k %d "
                "shared %d vocab %d max_positions %d)", c->hidden, c->inter, c->n_layers, c->n_routed, c->top_k,
                c->n_shared, c->vocab, c->max_positions);
  if (!(c->rms_eps >= 0.0f)) return fail(MOE_EINVAL, "rms_eps must be >= 0");
  if (c->n_routed > 64) return fail(MOE_EUNSUPPORTED, "n_routed %d > 64 (one wavefront lane per routed expert)", c->n_routed);
  if (c->top_k > c->n_routed) return fail(MOE_EUNSUPPORTED, "top_k %d > n_routed %d", c->top_k, c->n_routed);
  if (c->n_shared > 8) return fail(MOE_EUNSUPPORTED, "n_shared %d > 8", c->n_shared);
  const int kb = kblock_elems(c->wdtype);
  if (c->hidden % kb || c->inter % kb)
    return fail(MOE_EUNSUPPORTED, "hidden %d and inter %d must be multiples of %d for this dtype", c->hidden,
                c->inter, kb);
  // the LM head pipelines the contraction two 256-byte blocks at a time
  if (c->vocab > 0 && c->hidden % (2 * kb))
    return fail(MOE_EUNSUPPORTED, "with an LM head, hidden %d must be a multiple of %d for this dtype", c->hidden,
                2 * kb);
  // hidden: one residual row is held in 16 float4 per lane; the router's LDS rows fit 64 KB
  if (c->hidden > (c->wdtype == MOE_BF16 ? 4096 : 2048) || c->inter > 16384)
    return fail(MOE_EUNSUPPORTED, "hidden %d (max %d for this dtype) or inter %d (max 16384) too large", c->hidden,
                c->wdtype == MOE_BF16 ? 4096 : 2048, c->inter);
  if (max_work_items(*c, c->max_positions) > 65535 || (int64_t)c->max_positions * c->top_k > (1ll << 30))
    return fail(MOE_EUNSUPPORTED, "max_positions %d too large", c->max_positions);
  // The tiled GEMM forms each lane's activation offset in 32 bits: its operand buffers
  // (the normalised rows a [P][H], read by the tiled expert GEMM and the tiled LM head, and
  // the SwiGLU rows h [P*(k+S)+1][I]) must stay below 4 GiB whenever a pass can take that
  // path.
  if (c->wdtype == MOE_BF16 && c->hidden >= 256 && c->max_positions >= MV_TILED_MIN_POSITIONS) {
    const int64_t P = c->max_positions, KS = c->top_k + c->n_shared;
    const bool expert_tiles = c->inter >= 256, lm_tiles = c->vocab > 0 && c->max_positions >= mv::kTileM;
    const int64_t a_bytes = (expert_tiles || lm_tiles) ? P * c->hidden * 2 : 0;
    const int64_t h_bytes = expert_tiles ? (P * KS + 1) * c->inter * 2 : 0;
    if (a_bytes >= (1ll << 32) || h_bytes >= (1ll << 32))
      return fail(MOE_EUNSUPPORTED, "max_positions %d: the tiled GEMM operands (%lld and %lld bytes) must stay below 4 GiB",
                  c->max_positions, (long long)a_bytes, (long long)h_bytes);
  }
  return MOE_OK;
}

int check_step(const moe_verify_config* c, int32_t B, int32_t K, int has_in, int has_argmax, int has_hout) {
  if (B < 1) return fail(MOE_EINVAL, "B = %d, need B >= 1", B);
  if (K < 0) return fail(MOE_EINVAL, "K = %d, need K >= 0", K);
  const int64_t T = (int64_t)B * ((int64_t)K + 1);
  if (T > c->max_positions) return fail(MOE_EINVAL, "B*(K+1) = %lld exceeds max_positions %d", (long long)T, c->max_positions);
  if (!has_in) return fail(MOE_EINVAL, "hidden_in is NULL");
  if (c->vocab > 0 && !has_argmax) return fail(MOE_EINVAL, "argmax_out is required when vocab > 0");
  if (c->vocab == 0 && has_argmax) return fail(MOE_EINVAL, "argmax_out given but the config has no LM head");
  if (c->vocab == 0 && !has_hout) return fail(MOE_EINVAL, "hidden_out is required when vocab == 0");
  return MOE_OK;
}

// Makes the context's device current for the scope of a call, restoring the caller's.
struct DeviceGuard {
  int prev = -1;
  bool changed = false;
  hipError_t err = hipSuccess;
  explicit DeviceGuard(int dev) {
    err = hipGetDevice(&prev);
    if (err == hipSuccess && prev != dev) {
      err = hipSetDevice(dev);
      changed = err == hipSuccess;
    }
  }
  ~DeviceGuard() {
    if (changed) (void)hipSetDevice(prev);
  }
};

// Per-pass buffers of the verify step for up to P positions (device memory).
struct Workspace {
  int P = 0;                     // capacity in positions
  float* x_ws = nullptr;         // [P][H] residual stream
  void* a = nullptr;             // [P][H] normalised rows, in the weight type
  int32_t* topk_id = nullptr;    // [P][k]
  float* topk_w = nullptr;       // [P][k]
  int32_t* row_tok = nullptr;    // [P*k] token of each routed row
  int32_t* slot_row = nullptr;   // [P*k] routed row of each slot (inverse of the expert-major order)
  int32_t* row_dst = nullptr;    // [P*k] position-major ybuf row of each routed row (streaming path)
  int4* work = nullptr;          // GEMM work list
  int32_t* n_work = nullptr;     // its length
  int4* work2 = nullptr;         // split plan: streaming work items of the tiled passes
  int32_t* n_work2 = nullptr;    // their number
  int32_t* chunk_cnt = nullptr;  // [chunks][64] expert counts per slot chunk (large-pass plan)
  void* h = nullptr;             // [P*(k+S)+1][I] SwiGLU rows (+ a sink row for padding stores)
  void* ybuf = nullptr;          // [P*(k+S)+1][H] expert outputs, one row per slot, weight type
  mv::Top2* part = nullptr;      // [P][n_pg] LM-head partial records (vocab > 0)
  int32_t* counts = nullptr;     // [L][E] routed-slot count per expert of the last pass
};

// Places a workspace for P positions at base, each piece on a 256-byte boundary, and returns
// its size in bytes; with base == nullptr only the size is computed.
size_t layout_workspace(const moe_verify_config& g, int n_pg_lm, int P, char* base, Workspace* w) {
  const size_t es = elem_bytes(g.wdtype), Pz = (size_t)P;
  const size_t k = g.top_k, KS = g.top_k + g.n_shared, H = g.hidden, I = g.inter;
  size_t off = 0;
  auto take = [&](auto** ptr, size_t bytes) {
    if (base) *ptr = reinterpret_cast<std::remove_pointer_t<std::remove_reference_t<decltype(ptr)>>>(base + off);
    off += (bytes + 255) / 256 * 256;
  };
  Workspace tmp;
  Workspace& o = w ? *w : tmp;
  o.P = P;
  take(&o.x_ws, Pz * H * sizeof(float));
  take(&o.a, Pz * H * es);
  take(&o.topk_id, Pz * k * sizeof(int32_t));
  take(&o.topk_w, Pz * k * sizeof(float));
  take(&o.row_tok, Pz * k * sizeof(int32_t));
  take(&o.slot_row, Pz * k * sizeof(int32_t));
  take(&o.row_dst, Pz * k * sizeof(int32_t));
  take(&o.work, (size_t)max_work_items(g, P) * sizeof(int4));
  take(&o.n_work, sizeof(int32_t));
  take(&o.work2, (size_t)max_split_items(g) * sizeof(int4));
  take(&o.n_work2, sizeof(int32_t));
  take(&o.chunk_cnt, (size_t)mv::plan_chunks(P, g.top_k) * 64 * sizeof(int32_t));
  take(&o.h, (Pz * KS + 1) * I * es);
  take(&o.ybuf, (Pz * KS + 1) * H * es);
  // (+1: the tiled LM head's lanes without a row store into the slot past the last)
  if (g.vocab > 0) take(&o.part, (Pz * n_pg_lm + 1) * sizeof(mv::Top2));
  take(&o.counts, (size_t)g.n_layers * g.n_routed * sizeof(int32_t));
  return off;
}

}  // namespace

struct moe_verify_ctx {
  moe_verify_config cfg{};
  int device = 0;
  int n_cu = 256;  // compute units of the device (sizes the streaming GEMM grids)
  int es = 2;
  int NQ_up = 0, NQ_dn = 0, NQ_lm = 0, n_pg_lm = 0, NKB_H = 0, NKB_I = 0;
  size_t router_units_per_layer = 0, up_units_per_layer = 0, down_units_per_layer = 0;
  // packed weights
  uint4* router_p = nullptr;
  float* bias_p = nullptr;  // [L][64]
  uint4* up_p = nullptr;
  uint4* down_p = nullptr;
  uint4* lm_p = nullptr;
  Workspace ws;  // the context's per-pass buffers, for max_positions positions
  int last_T = 0, last_layer = 0;  // positions and block of the last MoE block run (debug_plan)
  // draft block (moe_draft_init): packed weights and its own buffers; the projection and
  // block outputs use ybuf, the normalised rows a, the LM partials part, the GEMM work list
  // work / n_work
  int draft_inter = 0;
  uint4* draft_proj_p = nullptr;  // H x 2H, pair layout
  uint4* draft_up_p = nullptr;    // gate/up pairs, I_d x H
  uint4* draft_down_p = nullptr;  // H x I_d
  void* draft_u = nullptr;        // [P][2H] block input rows
  float* draft_z = nullptr;       // [P][H] block residual stream (the next step's hidden state)
  float* draft_zero = nullptr;    // [P][H] zeros (residual before the projection)
  float* draft_ones = nullptr;    // [P] unit gates
  void* draft_h = nullptr;        // [P][I_d] SwiGLU rows
  int32_t* draft_ids = nullptr;   // [P] drafts of the current step
  std::vector<void*> allocs;
  // profiling: one event pair per launch of the last step, and running totals
  bool prof = false;
  std::vector<hipEvent_t> ev;
  std::vector<int> ev_kind;
  int n_pairs = 0;
  double prof_ms[MOE_PROF_KINDS] = {};
  int64_t prof_n[MOE_PROF_KINDS] = {};

  ~moe_verify_ctx() {
    for (hipEvent_t e : ev) (void)hipEventDestroy(e);
    for (void* p : allocs) (void)hipFree(p);
  }
  // Record the start event of a launch of class `kind` (no-op unless profiling).
  void prof_begin(int kind, hipStream_t st) {
    if (!prof || 2 * n_pairs + 1 >= (int)ev.size()) return;
    ev_kind[n_pairs] = kind;
    (void)hipEventRecord(ev[2 * n_pairs], st);
  }
  void prof_end(hipStream_t st) {
    if (!prof || 2 * n_pairs + 1 >= (int)ev.size()) return;
    (void)hipEventRecord(ev[2 * n_pairs + 1], st);
    ++n_pairs;
  }
  // Free one allocation made by alloc() (waits for the device first) and clear the pointer.
  template <typename P>
  void release(P** p) {
    if (!*p) return;
    for (size_t i = 0; i < allocs.size(); ++i)
      if (allocs[i] == static_cast<void*>(*p)) {
        (void)hipFree(allocs[i]);
        allocs.erase(allocs.begin() + i);
        break;
      }
    *p = nullptr;
  }
  template <typename P>
  hipError_t alloc(P** out, size_t bytes) {
    void* p = nullptr;
    hipError_t e = hipMalloc(&p, bytes < 256 ? 256 : bytes);
    if (e != hipSuccess) return e;
    allocs.push_back(p);
    *out = static_cast<P*>(p);
    return hipSuccess;
  }
};

// ---- per-pass buffers without allocation ------------------------------------------------
// moe_verify_step_static takes every per-pass buffer from this device array (one copy per GPU,
// held until the process ends). Host code never hands the array's name to a kernel: the
// device address of each GPU's copy comes from hipGetSymbolAddress, resolved once per device
// with that device current, and only that address is used.
static __device__ __align__(256) char scratch[MOE_VERIFY_STATIC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// Device address of the current device's copy of `scratch` (dev must be current).
hipError_t scratch_address(int dev, void** out) {
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return hipSuccess;
}

}  // namespace

namespace {

#define MV_CHECK(call)                                                                          \
  do {                                                                                          \
    hipError_t e_ = (call);                                                                     \
    if (e_ != hipSuccess) return fail(MOE_EDEVICE, "%s: %s", #call, hipGetErrorString(e_));     \
  } while (0)

// Launch the MoE block `l` over Tn positions whose residual input is x_in (plus the
// previous block's ybuf when given; that sum is stored to x_out when given, which may be
// x_in itself). Leaves the block's per-slot outputs in ybuf.
int run_block(moe_verify_ctx* c, const Workspace& w, int l, const float* x_in, const void* ybuf_prev, float* x_out, int Tn,
              hipStream_t st) {
  const moe_verify_config& g = c->cfg;
  const int E = g.n_routed, S = g.n_shared, k = g.top_k, KS = k + S, H = g.hidden, I = g.inter;
  const bool tiled = use_tiled(g, Tn);
  const int mb = tiled ? mv::kTileM : mv::kGemmMB;
  const int wmax = (int)max_work_items(g, Tn, mb);
  mv::PlanArgs pa{};
  pa.topk_id = w.topk_id;
  pa.topk_w = w.topk_w;
  pa.Tn = Tn; pa.k = k; pa.E = E; pa.S = S;
  pa.row_tok = w.row_tok;
  pa.slot_row = w.slot_row;
  pa.row_dst = w.row_dst;
  pa.work = w.work;
  pa.n_work = w.n_work;
  pa.counts = w.counts + (size_t)l * E;
  pa.mb = mb;
  pa.chunk_cnt = w.chunk_cnt;
  // tiled passes that one plan workgroup handles split off their cold experts
  const bool split = tiled && mv::plan_chunks(Tn, k) <= mv::kPlanSingleMaxChunks;
  if (split) {
    pa.hot_rows = kSplitHotRows;
    pa.mb2 = kSplitRows;
    pa.work2 = w.work2;
    pa.n_work2 = w.n_work2;
  }
  c->prof_begin(MOE_PROF_NORM_ROUTE, st);
  MV_CHECK(mv::launch_norm_route(g.wdtype, true, x_in, ybuf_prev, w.slot_row, x_out, nullptr, w.a,
                                 c->router_p + l * c->router_units_per_layer, c->bias_p + (size_t)l * 64, w.topk_id,
                                 w.topk_w, Tn, H, S, E, k, g.rms_eps, tiled, !tiled, st));
  c->prof_end(st);
  // small streaming passes: the gate/up GEMM builds the plan in its prologue
  const bool self_plan = !tiled && Tn * k <= mv::kSelfPlanMaxSlots;
  if (!self_plan) {
    c->prof_begin(MOE_PROF_PLAN, st);
    MV_CHECK(mv::launch_plan(pa, st));
    c->prof_end(st);
  }
  mv::GemmArgs a{};
  a.work = w.work;
  a.n_work = w.n_work;
  a.Tn = Tn;
  a.k = k; a.E = E; a.KS = KS; a.H = H; a.I = I;
  a.row_tok = w.row_tok;
  a.row_dst = w.row_dst;
  a.max_items = wmax;
  a.sink_row = w.P * KS;  // the extra row past every real row of h and ybuf
  a.topk_id = w.topk_id;
  a.plan_work = w.work;
  a.plan_n_work = w.n_work;
  a.plan_counts = pa.counts;
  a.plan_row_dst = w.row_dst;
  a.mb = mb;
  if (split) {
    a.work2 = w.work2;
    a.n_work2 = w.n_work2;
  }
  // Streaming kernel: two pairs per wavefront when the expected items x pairs fill at
  // least one round of resident wavefronts (routed items: one per touched expert while
  // positions are few).
  const int wave_target = c->n_cu * mv::kGemmWaves * MV_GEMM_WAVES_PER_SIMD;
  const int est_items = std::min(E, Tn * k) + S * ((Tn + mb - 1) / mb);
  auto grid_for = [&](int NQ, int wpg, int* ppw) -> unsigned {
    if (tiled) return (unsigned)c->n_cu;  // persistent: one workgroup per compute unit
    *ppw = est_items * NQ >= wave_target ? 2 : 1;
    const int chunks = (NQ + *ppw - 1) / *ppw;
    return (unsigned)((wmax * chunks + wpg - 1) / wpg);
  };
  auto launch = [&](int epi, unsigned n_wg) {
    return tiled ? mv::launch_gemm_tiled(epi, a, n_wg, st) : mv::launch_gemm(g.wdtype, epi, a, n_wg, st);
  };
  // gate/up + SwiGLU
  a.A = w.a;
  a.B = c->up_p + l * c->up_units_per_layer;
  a.K = H;
  a.NQ = c->NQ_up;
  a.h = w.h;
  c->prof_begin(MOE_PROF_GEMM_UP, st);
  unsigned n_wg = grid_for(c->NQ_up, mv::kStreamWavesUp, &a.ppw);
  if (self_plan) MV_CHECK(mv::launch_gemm_planned(g.wdtype, a, n_wg, st));
  else MV_CHECK(launch(mv::EPI_UP, n_wg));
  c->prof_end(st);
  // down + gate scale
  a.A = w.h;
  a.B = c->down_p + l * c->down_units_per_layer;
  a.K = I;
  a.NQ = c->NQ_dn;
  a.ybuf = w.ybuf;
  c->prof_begin(MOE_PROF_GEMM_DOWN, st);
  n_wg = grid_for(c->NQ_dn, mv::kStreamWavesDown, &a.ppw);
  MV_CHECK(launch(mv::EPI_DOWN, n_wg));
  c->prof_end(st);
  return MOE_OK;
}

}  // namespace

MV_API int moe_verify_check_config(const moe_verify_config* cfg) {
  const int rc = check_config(cfg);
  return rc ? rc : ok();
}

MV_API int moe_verify_check_step(const moe_verify_config* cfg, int32_t B, int32_t K, int has_hidden_in,
                                 int has_argmax, int has_hidden_out) {
  int rc = check_config(cfg);
  if (rc) return rc;
  rc = check_step(cfg, B, K, has_hidden_in, has_argmax, has_hidden_out);
  return rc ? rc : ok();
}

MV_API const char* moe_verify_last_error(void) { return g_last_error.c_str(); }

MV_API int moe_verify_init(const moe_verify_config* cfg, const moe_verify_weights* w, void* stream,
                           moe_verify_ctx** out) {
  if (!out) return fail(MOE_EINVAL, "out is NULL");
  *out = nullptr;
  int rc = check_config(cfg);
  if (rc) return rc;
  if (!w) return fail(MOE_EINVAL, "weights is NULL");
  if (!w->router_w || !w->w_gate || !w->w_up || !w->w_down) return fail(MOE_EINVAL, "a required weight pointer is NULL");
  if ((cfg->vocab > 0) != (w->lm_head != nullptr)) return fail(MOE_EINVAL, "lm_head must be non-NULL iff vocab > 0");
  if (!aligned16(w->router_w) || !aligned16(w->w_gate) || !aligned16(w->w_up) || !aligned16(w->w_down) ||
      (w->lm_head && !aligned16(w->lm_head)))
    return fail(MOE_EINVAL, "weight pointers must be 16-byte aligned");

  const moe_verify_config& g = *cfg;
  hipStream_t st = static_cast<hipStream_t>(stream);
  moe_verify_ctx* c = new (std::nothrow) moe_verify_ctx();
  if (!c) return fail(MOE_ENOMEM, "host allocation failed");
  c->cfg = g;
  c->es = elem_bytes(g.wdtype);
  hipError_t he = hipGetDevice(&c->device);
  if (he == hipSuccess) he = hipDeviceGetAttribute(&c->n_cu, hipDeviceAttributeMultiprocessorCount, c->device);
  if (he != hipSuccess) {
    delete c;
    return fail(MOE_EDEVICE, "device query: %s", hipGetErrorString(he));
  }
  if (c->n_cu < 1) c->n_cu = 1;
  const int E = g.n_routed, S = g.n_shared, H = g.hidden, I = g.inter, L = g.n_layers;
  const size_t es = c->es, P = (size_t)g.max_positions;
  c->NKB_H = (int)(H * es / mv::kRowBlockBytes);
  c->NKB_I = (int)(I * es / mv::kRowBlockBytes);
  c->NQ_up = I / 16;
  c->NQ_dn = (H + 31) / 32;
  c->NQ_lm = (g.vocab + 31) / 32;
  // partial records per row: the streaming head's column groups (at least one pair per
  // wavefront) or the tiled head's column tiles, whichever is more
  c->n_pg_lm = std::max((c->NQ_lm + mv::kLmWaves - 1) / mv::kLmWaves, mv::tiled_tiles_per_item(c->NQ_lm));
  c->router_units_per_layer = (size_t)(H * es / 16) * 64;
  c->up_units_per_layer = (size_t)(E + S) * c->NQ_up * c->NKB_H * mv::kPairUnits;
  c->down_units_per_layer = (size_t)(E + S) * c->NQ_dn * c->NKB_I * mv::kPairUnits;
  const size_t lm_units = (size_t)c->NQ_lm * c->NKB_H * mv::kPairUnits;

  hipError_t ae = hipSuccess;
  auto A = [&](auto** p, size_t bytes) {
    if (ae == hipSuccess) ae = c->alloc(p, bytes);
  };
  A(&c->router_p, c->router_units_per_layer * L * 16);
  A(&c->bias_p, (size_t)L * 64 * sizeof(float));
  A(&c->up_p, c->up_units_per_layer * L * 16);
  A(&c->down_p, c->down_units_per_layer * L * 16);
  if (g.vocab > 0) A(&c->lm_p, lm_units * 16);
  // the per-pass workspace: one allocation laid out by layout_workspace
  char* ws_base = nullptr;
  A(&ws_base, layout_workspace(g, c->n_pg_lm, (int)P, nullptr, nullptr));
  if (ae == hipSuccess) layout_workspace(g, c->n_pg_lm, (int)P, ws_base, &c->ws);
  if (ae != hipSuccess) {
    delete c;
    (void)hipGetLastError();
    return fail(MOE_ENOMEM, "device allocation failed: %s", hipGetErrorString(ae));
  }

  auto bail = [&](hipError_t e, const char* what) {
    delete c;
    return fail(MOE_EDEVICE, "%s: %s", what, hipGetErrorString(e));
  };
  const size_t row_h = H * es, row_i = I * es;
  if ((he = mv::launch_repack_router(w->router_w, c->router_p, L, E, (int)row_h, st)) != hipSuccess)
    return bail(he, "router repack");
  if ((he = hipMemsetAsync(c->bias_p, 0, (size_t)L * 64 * sizeof(float), st)) != hipSuccess) return bail(he, "bias clear");
  // a work list that no plan has written yet holds no items
  if ((he = hipMemsetAsync(c->ws.n_work, 0, sizeof(int32_t), st)) != hipSuccess) return bail(he, "work count clear");
  if (w->router_bias &&
      (he = hipMemcpy2DAsync(c->bias_p, 64 * sizeof(float), w->router_bias, E * sizeof(float), E * sizeof(float), L,
                             hipMemcpyDeviceToDevice, st)) != hipSuccess)
    return bail(he, "bias copy");
  // gate/up: pair q = (gate tile q, up tile q); matrices are the L*(E+S) experts
  if ((he = mv::launch_repack_pairs(w->w_gate, w->w_up, c->up_p, L * (E + S), I, (int)row_h, c->NQ_up, c->NKB_H, 1,
                                    (size_t)I * row_h, st)) != hipSuccess)
    return bail(he, "gate/up repack");
  if ((he = mv::launch_repack_pairs(w->w_down, w->w_down, c->down_p, L * (E + S), H, (int)row_i, c->NQ_dn, c->NKB_I, 0,
                                    (size_t)H * row_i, st)) != hipSuccess)
    return bail(he, "down repack");
  if (g.vocab > 0 &&
      (he = mv::launch_repack_pairs(w->lm_head, w->lm_head, c->lm_p, 1, g.vocab, (int)row_h, c->NQ_lm, c->NKB_H, 0,
                                    (size_t)g.vocab * row_h, st)) != hipSuccess)
    return bail(he, "lm_head repack");
  if ((he = hipStreamSynchronize(st)) != hipSuccess) return bail(he, "repack");
  // this device's static scratch (moe_verify_step_static): resolved here, while the device is
  // current; a failure is reported by that call, which retries
  void* scratch_dev = nullptr;
  if (scratch_address(c->device, &scratch_dev) != hipSuccess) (void)hipGetLastError();
  *out = c;
  return ok();
}

namespace {

// LM head and argmax over the normalised rows row0 .. row0 + Tn - 1 of w.a, which are in
// the stage-ordered layout of the tiled GEMM when tiled (use_tiled_lm), else in row order.
int run_lm_head(moe_verify_ctx* c, const Workspace& w, int row0, int Tn, int32_t* argmax_out, float* margin_out,
                bool tiled, hipStream_t st) {
  const moe_verify_config& g = c->cfg;
  if (tiled) {
    // 256-row items x 256-column tiles, one record per row and column tile
    const int NT = mv::tiled_tiles_per_item(c->NQ_lm);
    const int n_tiles = (Tn + mv::kTileM - 1) / mv::kTileM * NT;
    mv::GemmArgs a{};
    a.A = static_cast<const char*>(w.a) + (size_t)row0 * g.hidden * c->es;
    a.B = c->lm_p;
    a.K = g.hidden;
    a.NQ = c->NQ_lm;
    a.n_valid = g.vocab;
    a.Tn = Tn;
    a.part = w.part;
    a.n_pg = NT;
    c->prof_begin(MOE_PROF_LM_HEAD, st);
    MV_CHECK(mv::launch_gemm_tiled(mv::EPI_LM, a, (unsigned)std::min(c->n_cu, n_tiles), st));
    c->prof_end(st);
    c->prof_begin(MOE_PROF_ARGMAX, st);
    MV_CHECK(mv::launch_argmax_reduce(w.part, NT, Tn, argmax_out, margin_out, st));
    c->prof_end(st);
    return MOE_OK;
  }
  // Workgroups (kLmWaves wavefronts, one per CU) cover one row block of up to kLmRows
  // positions; pairs per wavefront so that the workgroups of one row block make about
  // one round on the device (further row blocks share the weight stream through L2).
  const int n_items = (Tn + mv::kLmRows - 1) / mv::kLmRows;
  const int target = c->n_cu * mv::kLmWaves;  // pair streams per round
  const int ppw = std::max(1, (c->NQ_lm + target - 1) / target);
  const int n_pg = (c->NQ_lm + mv::kLmWaves * ppw - 1) / (mv::kLmWaves * ppw);
  mv::GemmArgs a{};
  a.A = static_cast<const char*>(w.a) + (size_t)row0 * g.hidden * c->es;
  a.B = c->lm_p;
  a.K = g.hidden;
  a.NQ = c->NQ_lm;
  a.n_valid = g.vocab;
  a.Tn = Tn;
  a.part = w.part;
  a.n_pg = n_pg;
  a.lm_ppw = ppw;
  c->prof_begin(MOE_PROF_LM_HEAD, st);
  MV_CHECK(mv::launch_gemm(g.wdtype, mv::EPI_LM, a, (unsigned)(n_items * n_pg), st));
  c->prof_end(st);
  c->prof_begin(MOE_PROF_ARGMAX, st);
  MV_CHECK(mv::launch_argmax_reduce(w.part, n_pg, Tn, argmax_out, margin_out, st));
  c->prof_end(st);
  return MOE_OK;
}

}  // namespace

namespace {

// The MoE blocks over Tn = n_prefill + Tv positions, the final norm, and the LM head and
// argmax over the last Tv of them.
int run_pass(moe_verify_ctx* c, const Workspace& w, const float* hidden_in, int n_prefill, int Tv, int32_t* argmax_out, float* margin_out,
             float* hidden_out, hipStream_t st) {
  const moe_verify_config& g = c->cfg;
  const int Tn = n_prefill + Tv;
  int rc;
  DeviceGuard dg(c->device);
  if (dg.err != hipSuccess) return fail(MOE_EDEVICE, "device select: %s", hipGetErrorString(dg.err));
  c->n_pairs = 0;
  for (int l = 0; l < g.n_layers; ++l) {
    // block 0's residual is hidden_in itself: block 1 reads it there, so it is not copied
    rc = run_block(c, w, l, l <= 1 ? hidden_in : w.x_ws, l == 0 ? nullptr : w.ybuf, l == 0 ? nullptr : w.x_ws, Tn, st);
    if (rc) return rc;
  }
  const bool lm_tiled = use_tiled_lm(g, Tv);
  c->prof_begin(MOE_PROF_NORM_ROUTE, st);
  MV_CHECK(mv::launch_norm_route(g.wdtype, false, g.n_layers == 1 ? hidden_in : w.x_ws, w.ybuf, w.slot_row, nullptr, hidden_out,
                                 g.vocab > 0 ? w.a : nullptr, nullptr, nullptr, nullptr, w.topk_w, Tn, g.hidden,
                                 g.n_shared, g.n_routed, g.top_k, g.rms_eps, lm_tiled, !use_tiled(g, Tn), st));
  c->prof_end(st);
  if (g.vocab > 0) {
    rc = run_lm_head(c, w, n_prefill, Tv, argmax_out, margin_out, lm_tiled, st);
    if (rc) return rc;
  }
  return MOE_OK;
}

}  // namespace

MV_API int moe_verify_step(moe_verify_ctx* c, const float* hidden_in, int32_t B, int32_t K, int32_t* argmax_out,
                           float* margin_out, float* hidden_out, void* stream) {
  if (!c) return fail(MOE_EINVAL, "context is NULL");
  const int rc = check_step(&c->cfg, B, K, hidden_in != nullptr, argmax_out != nullptr, hidden_out != nullptr);
  if (rc) return rc;
  const int rp = run_pass(c, c->ws, hidden_in, 0, B * (K + 1), argmax_out, margin_out, hidden_out,
                          static_cast<hipStream_t>(stream));
  if (rp) return rp;
  c->last_T = B * (K + 1);
  c->last_layer = c->cfg.n_layers - 1;
  return ok();
}

MV_API int moe_verify_step_mixed(moe_verify_ctx* c, const float* hidden_in, int32_t n_prefill, int32_t B, int32_t K,
                                 int32_t* argmax_out, float* margin_out, float* hidden_out, void* stream) {
  if (!c) return fail(MOE_EINVAL, "context is NULL");
  if (n_prefill < 0) return fail(MOE_EINVAL, "n_prefill = %d, need n_prefill >= 0", n_prefill);
  const moe_verify_config& g = c->cfg;
  int rc = check_step(&g, B, K, hidden_in != nullptr, argmax_out != nullptr, hidden_out != nullptr);
  if (rc) return rc;
  if ((int64_t)n_prefill + (int64_t)B * ((int64_t)K + 1) > g.max_positions)
    return fail(MOE_EINVAL, "n_prefill + B*(K+1) = %lld exceeds max_positions %d",
                (long long)n_prefill + (long long)B * ((long long)K + 1), g.max_positions);
  rc = run_pass(c, c->ws, hidden_in, n_prefill, B * (K + 1), argmax_out, margin_out, hidden_out,
                static_cast<hipStream_t>(stream));
  if (rc) return rc;
  c->last_T = n_prefill + B * (K + 1);
  c->last_layer = g.n_layers - 1;
  return ok();
}

MV_API int moe_verify_step_static(moe_verify_ctx* c, const float* hidden_in, int32_t B, int32_t K,
                                  int32_t* argmax_out, float* margin_out, float* hidden_out, void* stream) {
  if (!c) return fail(MOE_EINVAL, "context is NULL");
  const moe_verify_config& g = c->cfg;
  const int rc = check_step(&g, B, K, hidden_in != nullptr, argmax_out != nullptr, hidden_out != nullptr);
  if (rc) return rc;
  const int T = B * (K + 1);
  const size_t need = layout_workspace(g, c->n_pg_lm, T, nullptr, nullptr);
  if (need > (size_t)MOE_VERIFY_STATIC_SCRATCH_BYTES)
    return fail(MOE_EUNSUPPORTED, "a pass of %d positions needs %zu bytes of per-pass buffers; the static scratch holds %zu",
                T, need, (size_t)MOE_VERIFY_STATIC_SCRATCH_BYTES);
  DeviceGuard dg(c->device);
  if (dg.err != hipSuccess) return fail(MOE_EDEVICE, "device select: %s", hipGetErrorString(dg.err));
  void* base = nullptr;
  const hipError_t e = scratch_address(c->device, &base);
  if (e != hipSuccess) return fail(MOE_EDEVICE, "hipGetSymbolAddress(scratch): %s", hipGetErrorString(e));
  // every buffer of the pass is written before it is read, so nothing needs clearing
  Workspace w;
  layout_workspace(g, c->n_pg_lm, T, static_cast<char*>(base), &w);
  const int rp = run_pass(c, w, hidden_in, 0, T, argmax_out, margin_out, hidden_out, static_cast<hipStream_t>(stream));
  return rp ? rp : ok();
}

MV_API int accept_greedy(const int32_t* draft_ids, const int32_t* argmax_ids, int32_t B, int32_t K,
                         int32_t* accepted_len, int32_t* committed, void* stream) {
  if (B < 1) return fail(MOE_EINVAL, "B = %d, need B >= 1", B);
  if (K < 0) return fail(MOE_EINVAL, "K = %d, need K >= 0", K);
  if ((K > 0 && !draft_ids) || !argmax_ids || !accepted_len || !committed)
    return fail(MOE_EINVAL, "a required pointer is NULL");
  MV_CHECK(mv::launch_accept(draft_ids, argmax_ids, B, K, accepted_len, committed, static_cast<hipStream_t>(stream)));
  return ok();
}

MV_API int moe_verify_debug_layer(moe_verify_ctx* c, int32_t layer, const float* x_in, int32_t T, float* moe_out,
                                  int32_t* topk_id, float* topk_w, void* stream) {
  if (!c) return fail(MOE_EINVAL, "context is NULL");
  const moe_verify_config& g = c->cfg;
  if (layer < 0 || layer >= g.n_layers) return fail(MOE_EINVAL, "layer %d out of range [0, %d)", layer, g.n_layers);
  if (T < 1 || T > g.max_positions) return fail(MOE_EINVAL, "T = %d out of range [1, %d]", T, g.max_positions);
  if (!x_in) return fail(MOE_EINVAL, "x_in is NULL");
  hipStream_t st = static_cast<hipStream_t>(stream);
  DeviceGuard dg(c->device);
  if (dg.err != hipSuccess) return fail(MOE_EDEVICE, "device select: %s", hipGetErrorString(dg.err));
  int rc = run_block(c, c->ws, layer, x_in, nullptr, nullptr, T, st);
  if (rc) return rc;
  c->last_T = T;
  c->last_layer = layer;
  if (moe_out)
    MV_CHECK(mv::launch_combine(g.wdtype, c->ws.ybuf, c->ws.slot_row, c->ws.topk_w, T, g.hidden, g.top_k, g.n_shared, !use_tiled(g, T),
                                moe_out, st));
  const size_t kb = (size_t)T * g.top_k * 4;
  if (topk_id) MV_CHECK(hipMemcpyAsync(topk_id, c->ws.topk_id, kb, hipMemcpyDeviceToDevice, st));
  if (topk_w) MV_CHECK(hipMemcpyAsync(topk_w, c->ws.topk_w, kb, hipMemcpyDeviceToDevice, st));
  return ok();
}

MV_API int moe_verify_debug_head(moe_verify_ctx* c, const float* x_in, int32_t T, int32_t* argmax_out,
                                 float* margin_out, void* stream) {
  if (!c) return fail(MOE_EINVAL, "context is NULL");
  const moe_verify_config& g = c->cfg;
  if (g.vocab <= 0) return fail(MOE_EINVAL, "the context has no LM head (vocab == 0)");
  if (T < 1 || T > g.max_positions) return fail(MOE_EINVAL, "T = %d out of range [1, %d]", T, g.max_positions);
  if (!x_in || !argmax_out) return fail(MOE_EINVAL, "x_in and argmax_out are required");
  hipStream_t st = static_cast<hipStream_t>(stream);
  DeviceGuard dg(c->device);
  if (dg.err != hipSuccess) return fail(MOE_EDEVICE, "device select: %s", hipGetErrorString(dg.err));
  // the final norm with no expert outputs to add: a = RMSNorm(x_in) in the weight type
  const bool lm_tiled = use_tiled_lm(g, T);
  c->prof_begin(MOE_PROF_NORM_ROUTE, st);
  MV_CHECK(mv::launch_norm_route(g.wdtype, false, x_in, nullptr, nullptr, nullptr, nullptr, c->ws.a, nullptr, nullptr,
                                 nullptr, nullptr, T, g.hidden, g.n_shared, g.n_routed, g.top_k, g.rms_eps, lm_tiled,
                                 true, st));
  c->prof_end(st);
  const int rc = run_lm_head(c, c->ws, 0, T, argmax_out, margin_out, lm_tiled, st);
  return rc ? rc : ok();
}

MV_API int moe_verify_debug_plan(moe_verify_ctx* c, int32_t* row_slot, int32_t* counts, void* stream) {
  if (!c) return fail(MOE_EINVAL, "context is NULL");
  if (!row_slot) return fail(MOE_EINVAL, "row_slot is NULL");
  if (c->last_T < 1) return fail(MOE_EINVAL, "no MoE block has run on this context");
  const moe_verify_config& g = c->cfg;
  hipStream_t st = static_cast<hipStream_t>(stream);
  DeviceGuard dg(c->device);
  if (dg.err != hipSuccess) return fail(MOE_EDEVICE, "device select: %s", hipGetErrorString(dg.err));
  MV_CHECK(mv::launch_row_slot(c->ws.row_dst, c->last_T * g.top_k, g.top_k, g.top_k + g.n_shared, row_slot, st));
  if (counts)
    MV_CHECK(hipMemcpyAsync(counts, c->ws.counts + (size_t)c->last_layer * g.n_routed, (size_t)g.n_routed * sizeof(int32_t),
                            hipMemcpyDeviceToDevice, st));
  return ok();
}

MV_API int moe_draft_init(moe_verify_ctx* c, const moe_draft_weights* w, void* stream) {
  if (!c) return fail(MOE_EINVAL, "context is NULL");
  if (!w) return fail(MOE_EINVAL, "weights is NULL");
  const moe_verify_config& g = c->cfg;
  if (g.vocab <= 0) return fail(MOE_EINVAL, "the draft block needs a context with an LM head (vocab > 0)");
  if (!w->proj || !w->w_gate || !w->w_up || !w->w_down) return fail(MOE_EINVAL, "a required weight pointer is NULL");
  if (!aligned16(w->proj) || !aligned16(w->w_gate) || !aligned16(w->w_up) || !aligned16(w->w_down))
    return fail(MOE_EINVAL, "weight pointers must be 16-byte aligned");
  const int H = g.hidden, Id = w->inter, es = c->es;
  if (Id < 16 || Id > 16384 || Id % 16 != 0 || (Id * es) % mv::kRowBlockBytes != 0)
    return fail(MOE_EUNSUPPORTED, "draft inter %d: need a multiple of %d in [16, 16384]", Id, mv::kRowBlockBytes / es);
  hipStream_t st = static_cast<hipStream_t>(stream);
  DeviceGuard dg(c->device);
  if (dg.err != hipSuccess) return fail(MOE_EDEVICE, "device select: %s", hipGetErrorString(dg.err));
  // detached until the new weights are in place: a failure below leaves no draft block.
  // A previous call's buffers are freed first (hipFree waits for work still using them).
  c->draft_inter = 0;
  MV_CHECK(hipStreamSynchronize(st));
  c->release(&c->draft_proj_p);
  c->release(&c->draft_up_p);
  c->release(&c->draft_down_p);
  c->release(&c->draft_u);
  c->release(&c->draft_z);
  c->release(&c->draft_zero);
  c->release(&c->draft_ones);
  c->release(&c->draft_h);
  c->release(&c->draft_ids);
  const size_t P = (size_t)g.max_positions;
  const int NQ_h = (H + 31) / 32, NKB_2H = 2 * H * es / mv::kRowBlockBytes, NKB_I = Id * es / mv::kRowBlockBytes;
  hipError_t ae = hipSuccess;
  auto A = [&](auto** p, size_t bytes) {
    if (ae == hipSuccess) ae = c->alloc(p, bytes);
  };
  A(&c->draft_proj_p, (size_t)NQ_h * NKB_2H * mv::kPairUnits * 16);
  A(&c->draft_up_p, (size_t)(Id / 16) * c->NKB_H * mv::kPairUnits * 16);
  A(&c->draft_down_p, (size_t)NQ_h * NKB_I * mv::kPairUnits * 16);
  A(&c->draft_u, P * 2 * H * es);
  A(&c->draft_z, P * H * sizeof(float));
  A(&c->draft_zero, P * H * sizeof(float));
  A(&c->draft_ones, P * sizeof(float));
  A(&c->draft_h, (P + 1) * Id * es);
  A(&c->draft_ids, P * sizeof(int32_t));
  if (ae != hipSuccess) {
    (void)hipGetLastError();
    return fail(MOE_ENOMEM, "device allocation failed: %s", hipGetErrorString(ae));
  }
  const int row_h = H * es;
  MV_CHECK(mv::launch_repack_pairs(w->proj, w->proj, c->draft_proj_p, 1, H, 2 * row_h, NQ_h, NKB_2H, 0,
                                   (size_t)H * 2 * row_h, st));
  MV_CHECK(mv::launch_repack_pairs(w->w_gate, w->w_up, c->draft_up_p, 1, Id, row_h, Id / 16, c->NKB_H, 1,
                                   (size_t)Id * row_h, st));
  MV_CHECK(mv::launch_repack_pairs(w->w_down, w->w_down, c->draft_down_p, 1, H, Id * es, NQ_h, NKB_I, 0,
                                   (size_t)H * Id * es, st));
  MV_CHECK(hipMemsetAsync(c->draft_zero, 0, P * H * sizeof(float), st));
  MV_CHECK(mv::launch_fill(c->draft_ones, P, 1.0f, st));
  MV_CHECK(hipStreamSynchronize(st));
  c->draft_inter = Id;
  return ok();
}

MV_API int moe_draft_step(moe_verify_ctx* c, const float* hidden, const int32_t* accepted_len,
                          const int32_t* committed, int32_t B, int32_t Kv, int32_t K, int32_t* drafts, void* stream) {
  if (!c) return fail(MOE_EINVAL, "context is NULL");
  if (c->draft_inter == 0) return fail(MOE_EINVAL, "no draft weights: call moe_draft_init first");
  const moe_verify_config& g = c->cfg;
  if (B < 1) return fail(MOE_EINVAL, "B = %d, need B >= 1", B);
  if (Kv < 0) return fail(MOE_EINVAL, "Kv = %d, need Kv >= 0", Kv);
  if (K < 1) return fail(MOE_EINVAL, "K = %d, need K >= 1", K);
  if ((int64_t)B * ((int64_t)Kv + 1) > g.max_positions)
    return fail(MOE_EINVAL, "B*(Kv+1) = %lld exceeds max_positions %d", (long long)B * ((long long)Kv + 1), g.max_positions);
  if (!hidden || !accepted_len || !committed || !drafts) return fail(MOE_EINVAL, "a required pointer is NULL");
  hipStream_t st = static_cast<hipStream_t>(stream);
  DeviceGuard dg(c->device);
  if (dg.err != hipSuccess) return fail(MOE_EDEVICE, "device select: %s", hipGetErrorString(dg.err));
  const int H = g.hidden, Id = c->draft_inter, mb = mv::kGemmMB;
  const int max_items = (g.max_positions + mb - 1) / mb;
  // The GEMMs see one always-on expert (routed count 0) whose work items are row blocks.
  mv::GemmArgs a{};
  a.work = c->ws.work;
  a.n_work = c->ws.n_work;
  a.Tn = B;
  a.k = 0; a.E = 0; a.KS = 1; a.H = H; a.I = Id;
  a.max_items = max_items;
  const int wave_target = c->n_cu * mv::kGemmWaves * MV_GEMM_WAVES_PER_SIMD;
  const int items = (B + mb - 1) / mb;
  auto grid = [&](int NQ, int wpg, int* ppw) {
    *ppw = items * NQ >= wave_target ? 2 : 1;
    return (unsigned)((max_items * ((NQ + *ppw - 1) / *ppw) + wpg - 1) / wpg);
  };
  MV_CHECK(mv::launch_draft_plan(c->ws.work, c->ws.n_work, B, mb, st));
  for (int i = 0; i < K; ++i) {
    MV_CHECK(mv::launch_draft_input(g.wdtype, hidden, accepted_len, committed, Kv, c->draft_z, c->draft_ids, drafts, K,
                                    i, c->lm_p, c->NKB_H, H, g.vocab, g.rms_eps, c->draft_u, B, st));
    // projection 2H -> H (an output-side GEMM like the experts' down projection)
    mv::GemmArgs p = a;
    p.A = c->draft_u; p.B = c->draft_proj_p; p.K = 2 * H; p.NQ = (H + 31) / 32; p.ybuf = c->ws.ybuf;
    unsigned n_wg = grid(p.NQ, mv::kStreamWavesDown, &p.ppw);
    MV_CHECK(mv::launch_gemm(g.wdtype, mv::EPI_DOWN, p, n_wg, st));
    // residual stream z = projection output; a = bf16(RMSNorm(z)) (one unit-gate slot per row)
    MV_CHECK(mv::launch_norm_route(g.wdtype, false, c->draft_zero, c->ws.ybuf, nullptr, c->draft_z, nullptr, c->ws.a, nullptr,
                                   nullptr, nullptr, c->draft_ones, B, H, 0, 0, 1, g.rms_eps, false, true, st));
    mv::GemmArgs u = a;  // gate/up + SwiGLU
    u.A = c->ws.a; u.B = c->draft_up_p; u.K = H; u.NQ = Id / 16; u.h = c->draft_h;
    n_wg = grid(u.NQ, mv::kStreamWavesUp, &u.ppw);
    MV_CHECK(mv::launch_gemm(g.wdtype, mv::EPI_UP, u, n_wg, st));
    mv::GemmArgs d = a;  // down
    d.A = c->draft_h; d.B = c->draft_down_p; d.K = Id; d.NQ = (H + 31) / 32; d.ybuf = c->ws.ybuf;
    n_wg = grid(d.NQ, mv::kStreamWavesDown, &d.ppw);
    MV_CHECK(mv::launch_gemm(g.wdtype, mv::EPI_DOWN, d, n_wg, st));
    // z <- z + block output; a = bf16(RMSNorm(z)) for the LM head
    MV_CHECK(mv::launch_norm_route(g.wdtype, false, c->draft_z, c->ws.ybuf, nullptr, c->draft_z, nullptr, c->ws.a, nullptr,
                                   nullptr, nullptr, c->draft_ones, B, H, 0, 0, 1, g.rms_eps, false, true, st));
    const int rc = run_lm_head(c, c->ws, 0, B, c->draft_ids, nullptr, false, st);
    if (rc) return rc;
  }
  MV_CHECK(mv::launch_draft_store(c->draft_ids, drafts, B, K, st));
  return ok();
}

MV_API void moe_verify_destroy(moe_verify_ctx* c) {
  if (!c) return;
  DeviceGuard dg(c->device);
  (void)hipDeviceSynchronize();
  delete c;
}

MV_API int moe_verify_profile(moe_verify_ctx* c, int enable) {
  if (!c) return fail(MOE_EINVAL, "context is NULL");
  DeviceGuard dg(c->device);
  if (dg.err != hipSuccess) return fail(MOE_EDEVICE, "device select: %s", hipGetErrorString(dg.err));
  const size_t need = 2 * (size_t)(4 * c->cfg.n_layers + 3);
  while (enable && c->ev.size() < need) {
    hipEvent_t e;
    // timing only: no system-scope fence at each record (its cache write-back and
    // invalidate would otherwise be counted into the launches around it)
    MV_CHECK(hipEventCreateWithFlags(&e, hipEventDisableSystemFence));
    c->ev.push_back(e);
  }
  c->ev_kind.assign(c->ev.size() / 2 + 1, 0);
  c->prof = enable != 0;
  c->n_pairs = 0;
  for (int i = 0; i < MOE_PROF_KINDS; ++i) {
    c->prof_ms[i] = 0.0;
    c->prof_n[i] = 0;
  }
  return ok();
}

MV_API int moe_verify_profile_read(moe_verify_ctx* c, double* ms, int64_t* launches) {
  if (!c) return fail(MOE_EINVAL, "context is NULL");
  DeviceGuard dg(c->device);
  if (dg.err != hipSuccess) return fail(MOE_EDEVICE, "device select: %s", hipGetErrorString(dg.err));
  if (c->n_pairs > 0) MV_CHECK(hipEventSynchronize(c->ev[2 * c->n_pairs - 1]));
  for (int i = 0; i < c->n_pairs; ++i) {
    float t = 0.f;
    MV_CHECK(hipEventElapsedTime(&t, c->ev[2 * i], c->ev[2 * i + 1]));
    c->prof_ms[c->ev_kind[i]] += t;
    c->prof_n[c->ev_kind[i]] += 1;
  }
  c->n_pairs = 0;
  for (int i = 0; i < MOE_PROF_KINDS; ++i) {
    if (ms) ms[i] = c->prof_ms[i];
    if (launches) launches[i] = c->prof_n[i];
  }
  return ok();
}

MV_API int moe_verify_expert_counts(moe_verify_ctx* c, int32_t* counts) {
  if (!c) return fail(MOE_EINVAL, "context is NULL");
  if (!counts) return fail(MOE_EINVAL, "counts is NULL");
  DeviceGuard dg(c->device);
  if (dg.err != hipSuccess) return fail(MOE_EDEVICE, "device select: %s", hipGetErrorString(dg.err));
  MV_CHECK(hipDeviceSynchronize());
  MV_CHECK(hipMemcpy(counts, c->ws.counts, (size_t)c->cfg.n_layers * c->cfg.n_routed * sizeof(int32_t),
                     hipMemcpyDeviceToHost));
  return ok();
}
