/*
 * moe_verify.h: C ABI of the MI355X (gfx950) greedy speculative-verification library.
 *
 * One verifier pass takes B sequences x (K+1) positions (position 0 of a sequence is
 * its last committed token, positions 1..K its drafted tokens) through the decoder's
 * mixture-of-experts FFN blocks and LM head, and picks each position's greedy token;
 * acceptance then keeps the longest prefix of drafts the verifier agrees with, plus
 * the verifier's own next token.
 *
 * Sources, by page title and paragraph (the pages have no numbered sections):
 *   - "jina-ocr-v1" model page, summary paragraph: three drafted tokens are checked
 *     greedily by the verifier; the output equals plain greedy decoding; a pass
 *     commits up to 2.7 tokens instead of one.
 *   - same page, architecture paragraph: 12 decoder layers, hidden 1280, 64 routed
 *     plus 2 shared experts, top-6 routing, a 129,280-token vocabulary.
 *   - same page, usage paragraph: speculation on or off changes speed, not text
 *     (so K = 0 is a legal pass and uses the same calls).
 *   - "Jina AI Releases jina-ocr-v1 ..." news page, FastMTP paragraph: the decoder
 *     keeps only the drafts that agree with its own choice.
 * Attention is not part of this path: the caller supplies each position's hidden
 * state at the input of the first MoE block.
 *
 * Block definition (readings of the pages, where they are silent): pre-norm
 * x <- x + MoE(RMSNorm(x)) with unit gain and eps inside the square root; router
 * softmax over the routed experts' logits (plus an optional bias), top-k with ties
 * to the lower expert index, gates renormalised over the k selected; bias-free
 * SwiGLU experts down(silu(gate x) * up x); shared experts always on with weight 1;
 * a final RMSNorm before the LM head; argmax ties to the lower vocabulary index.
 * Numerics with bf16 weights: every product takes bf16 activations (the RMSNorm
 * outputs and the SwiGLU output) and accumulates in float32. Each expert's output is
 * stored in bf16 before the gate-weighted sum, a rounding of at most 2^-9 of each
 * element, well inside the library's 2e-2 relative tolerance on a block's output; the
 * definition it is checked against keeps that output exact. The residual stream, router
 * logits, gates, the gated sum and the LM-head logits are float32.
 *
 * Conventions for every call:
 *   - Pointers named "device" are HIP device pointers; structs are host memory.
 *   - Matrices are row-major. Position row p = b*(K+1)+j.
 *   - Every call validates its arguments on the host before any HIP call and returns
 *     a status code (MOE_OK or a negative code); no exception crosses the ABI.
 *     moe_verify_last_error() gives a message for the last failing call on the
 *     calling thread.
 *   - moe_verify_step, accept_greedy and moe_verify_debug_layer only enqueue work on
 *     the given stream (a hipStream_t, or NULL for the default stream): they do not
 *     synchronise, allocate or copy to the host, so they can be captured in a HIP
 *     graph. Faults inside kernels surface at the caller's next synchronisation.
 *   - A context is used from one stream at a time; it is not thread-safe.
 */
#ifndef MOE_VERIFY_H
#define MOE_VERIFY_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct moe_verify_ctx moe_verify_ctx; /* opaque */

enum {
  MOE_OK = 0,
  MOE_EINVAL = -1,       /* bad argument (null pointer, size out of range, ...)      */
  MOE_ENOMEM = -2,       /* device allocation failed                                 */
  MOE_EDEVICE = -3,      /* a HIP runtime call failed                                */
  MOE_EUNSUPPORTED = -4  /* shape outside what the kernels cover (see config below)  */
};

typedef enum { MOE_F32 = 0, MOE_BF16 = 1 } moe_dtype;

/* Host struct. Shapes the kernels cover (else MOE_EUNSUPPORTED):
 *   1 <= n_routed <= 64 (one wavefront lane per routed expert), 1 <= top_k <= n_routed,
 *   0 <= n_shared <= 8, n_layers >= 1, vocab >= 0,
 *   hidden and inter multiples of 128 (bf16) or 64 (f32), and hidden a multiple of 256
 *   (bf16) or 128 (f32) when vocab > 0; hidden <= 4096 (bf16) or 2048 (f32),
 *   inter <= 16384, max_positions >= 1; and when bf16 weights can take the tiled GEMM
 *   (hidden >= 256 and max_positions >= 256, with inter >= 256 for the expert products or
 *   vocab > 0 for the LM head), its operands must stay below 4 GiB: max_positions*hidden*2
 *   bytes, and for the expert products (max_positions*(top_k+n_shared)+1)*inter*2 bytes. */
typedef struct {
  int32_t hidden;        /* H                                                        */
  int32_t n_routed;      /* E routed experts                                         */
  int32_t top_k;         /* k experts selected per position                          */
  int32_t n_shared;      /* S always-on shared experts                               */
  int32_t inter;         /* I, SwiGLU intermediate width of every expert              */
  int32_t n_layers;      /* L MoE blocks                                             */
  int32_t vocab;         /* V; 0 => no LM head: step returns hidden states only      */
  int32_t wdtype;        /* moe_dtype of weights and GEMM inputs (accumulate f32)    */
  float   rms_eps;       /* RMSNorm epsilon (gain is 1)                              */
  int32_t max_positions; /* workspace capacity: the largest B*(K+1) a step may use   */
} moe_verify_config;

/* Host struct of device pointers, read only during moe_verify_init (weights are
 * copied into a library-owned, kernel-friendly layout; the caller may free its
 * buffers when init returns). Element type is wdtype (bf16 = 16-bit bit patterns). */
typedef struct {
  const void  *router_w;    /* [L][E][H]                                             */
  const float *router_bias; /* [L][E] float32 added to router logits, or NULL        */
  const void  *w_gate;      /* [L][E+S][I][H]  rows 0..E-1 routed, E..E+S-1 shared   */
  const void  *w_up;        /* [L][E+S][I][H]                                        */
  const void  *w_down;      /* [L][E+S][H][I]                                        */
  const void  *lm_head;     /* [V][H]; must be NULL iff vocab == 0                   */
} moe_verify_weights;

/* Validate cfg (host only, no HIP call). Returns MOE_OK, MOE_EINVAL or MOE_EUNSUPPORTED. */
int moe_verify_check_config(const moe_verify_config *cfg);

/* Validate the arguments of a step against cfg (host only, no HIP call): B >= 1,
 * K >= 0, B*(K+1) <= max_positions, argmax required iff vocab > 0, hidden_out
 * required iff vocab == 0, hidden_in required. Flags are 0/1. */
int moe_verify_check_step(const moe_verify_config *cfg, int32_t B, int32_t K, int has_hidden_in,
                          int has_argmax, int has_hidden_out);

/* Create a context on the current HIP device: validate, allocate the workspace for
 * max_positions positions and the repacked weights, repack on `stream`, and wait for
 * the repack to finish. On failure *out is NULL and nothing stays allocated. */
int moe_verify_init(const moe_verify_config *cfg, const moe_verify_weights *weights, void *stream,
                    moe_verify_ctx **out);

/* One verifier pass over T = B*(K+1) positions.
 *   hidden_in  [T][H] float32 device: hidden state of each position at the input of
 *              the first MoE block (required).
 *   argmax_out [T] int32 device: greedy token per position (required iff vocab > 0).
 *   margin_out [T] float32 device: largest minus second-largest logit, or NULL.
 *   hidden_out [T][H] float32 device: residual stream after the last block, before
 *              the final norm, or NULL (required iff vocab == 0).
 * Outputs are written in stream order; all buffers are caller-owned. */
int moe_verify_step(moe_verify_ctx *ctx, const float *hidden_in, int32_t B, int32_t K,
                    int32_t *argmax_out, float *margin_out, float *hidden_out, void *stream);

/* A mixed pass: n_prefill prompt positions (e.g. the visual tokens of a new page) and
 * B*(K+1) verify positions go through the MoE blocks together, so one stream of the
 * expert weights serves both (a serving engine's mixed batch); the LM head and argmax run
 * on the verify positions only.
 *   hidden_in  [n_prefill + B*(K+1)][H] float32 device: prefill rows first, then the
 *              verify rows b*(K+1)+j (required);
 *   argmax_out [B*(K+1)] int32 device, margin_out [B*(K+1)] float32 device or NULL: as
 *              for moe_verify_step, for the verify rows;
 *   hidden_out [n_prefill + B*(K+1)][H] float32 device or NULL (required iff vocab == 0).
 * n_prefill >= 0 and n_prefill + B*(K+1) <= max_positions; otherwise as moe_verify_step
 * (n_prefill = 0 is exactly moe_verify_step). */
int moe_verify_step_mixed(moe_verify_ctx *ctx, const float *hidden_in, int32_t n_prefill, int32_t B,
                          int32_t K, int32_t *argmax_out, float *margin_out, float *hidden_out,
                          void *stream);

/* Bytes of the device array behind moe_verify_step_static (one copy per GPU). */
#define MOE_VERIFY_STATIC_SCRATCH_BYTES (32u << 20)

/* moe_verify_step for callers that cannot allocate device memory at all (code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc): the same pass, same
 * arguments, same results bit for bit, but every per-pass buffer (residual stream,
 * normalised rows, routing and plan, SwiGLU rows, expert outputs, LM-head partials) comes
 * from one file-scope device array of MOE_VERIFY_STATIC_SCRATCH_BYTES per GPU instead of
 * the context's workspace; the call allocates and frees nothing. MOE_EUNSUPPORTED when the
 * pass's buffers exceed that size (about 23 MB for 512 positions of the real-width model).
 * All calls on one GPU share that GPU's array, which keeps the last call's contents: calls
 * that overlap on one GPU (any context, any stream) race. moe_verify_expert_counts and
 * moe_verify_debug_plan describe the context's own passes, not these. */
int moe_verify_step_static(moe_verify_ctx *ctx, const float *hidden_in, int32_t B, int32_t K,
                           int32_t *argmax_out, float *margin_out, float *hidden_out, void *stream);

/* Greedy acceptance for B sequences of K drafts.
 *   draft_ids    [B][K] int32 device (ids outside [0, V) simply never match);
 *   argmax_ids   [B][K+1] int32 device (the step's argmax_out);
 *   accepted_len [B] int32 device out: n_b = number of leading drafts equal to the
 *                argmax at the same position, 0..K;
 *   committed    [B][K+1] int32 device out: argmax_ids[b][0..n_b], then -1.
 * Needs no context. B >= 1, K >= 0, all pointers non-NULL (draft_ids may be NULL
 * iff K == 0). */
int accept_greedy(const int32_t *draft_ids, const int32_t *argmax_ids, int32_t B, int32_t K,
                  int32_t *accepted_len, int32_t *committed, void *stream);

/* Free everything the context owns (waits for the device first). NULL is a no-op. */
void moe_verify_destroy(moe_verify_ctx *ctx);

/* Message of the last failing call on this thread ("" if none). Valid until the next
 * call on this thread. */
const char *moe_verify_last_error(void);

/* Test hook: run MoE block `layer` alone on x_in [T][H] float32 device (1 <= T <=
 * max_positions) and write its output m (before the residual add) to moe_out [T][H]
 * float32, and the routing: topk_id [T][k] int32 in slot order (logit descending) and
 * topk_w [T][k] float32 gates. Any of the three outputs may be NULL. */
int moe_verify_debug_layer(moe_verify_ctx *ctx, int32_t layer, const float *x_in, int32_t T,
                           float *moe_out, int32_t *topk_id, float *topk_w, void *stream);

/* Test hook: the final RMSNorm, the LM head and the argmax alone, on a caller-supplied
 * residual stream x_in [T][H] float32 device (e.g. a reference pass's hidden state after
 * its last block), 1 <= T <= max_positions: argmax_out [T] int32 device (required) and
 * margin_out [T] float32 device or NULL, computed exactly as moe_verify_step computes
 * them from its own last block ("jina-ocr-v1" model page, summary paragraph: the
 * verifier's greedy choice). MOE_EINVAL for a context without an LM head. */
int moe_verify_debug_head(moe_verify_ctx *ctx, const float *x_in, int32_t T, int32_t *argmax_out,
                          float *margin_out, void *stream);

/* Test hook: the routing plan of the last MoE block the context ran (the last block of the
 * last moe_verify_step or moe_verify_step_mixed, or the block of the last
 * moe_verify_debug_layer), over that pass's T positions (architecture paragraph: top-6 of
 * 64 routed experts; the plan groups each expert's rows for its expert GEMM):
 *   row_slot [T*k] int32 device out (required): the routed slot t*k + j held by each row of
 *            the expert-major order, in which expert e's rows follow expert e-1's and hold
 *            its slots in ascending slot order (a stable sort of the slots by expert);
 *   counts   [E] int32 device out, or NULL: the routed-slot count of each expert.
 * Row r belongs to expert e when counts[0] + ... + counts[e-1] <= r < counts[0] + ... +
 * counts[e]. MOE_EINVAL if no block has run on the context. */
int moe_verify_debug_plan(moe_verify_ctx *ctx, int32_t *row_slot, int32_t *counts, void *stream);

/* ---- draft block: drafts the next pass's K tokens on the device ---------------------- */

/* The draft block is a multi-token-prediction head ("jina-ocr-v1" model page, FastMTP
 * paragraph: it drafts three tokens ahead for the verifier to check greedily). The pages
 * do not give its shape; this library's reading: step i takes a hidden state h and a
 * token t, forms [RMSNorm(h), RMSNorm(E[t])] with E the verifier's LM-head matrix (tied
 * embedding), projects it 2H -> H (bias-free, output materialised in the weight type),
 * adds a pre-norm dense SwiGLU block down(silu(gate a) * up a) with a residual, applies
 * the final RMSNorm and the verifier's LM head, and drafts the greedy token (ties to the
 * lower index); the block's output hidden state and the draft feed step i + 1. */

/* Host struct of device pointers (element type = the context's wdtype), read only during
 * moe_draft_init. inter: a multiple of 128 (bf16) or 64 (f32) in [16, 16384]. */
typedef struct {
  int32_t     inter;   /* I_d, SwiGLU intermediate width of the draft block          */
  const void *proj;    /* [H][2H]: columns 0..H-1 act on RMSNorm(h), H..2H-1 on       */
                       /*          RMSNorm(E[t])                                      */
  const void *w_gate;  /* [I_d][H]                                                    */
  const void *w_up;    /* [I_d][H]                                                    */
  const void *w_down;  /* [H][I_d]                                                    */
} moe_draft_weights;

/* Attach draft-block weights to a context that has an LM head (vocab > 0): copy them
 * into the library's layout on `stream`, allocate the block's workspace for
 * max_positions sequences, and wait. Calling it again replaces the weights: it waits for
 * `stream`, frees the earlier call's buffers, then allocates and copies anew; if that call
 * fails after its argument checks, the context is left without a draft block. MOE_EINVAL for a context without
 * an LM head or a NULL pointer, MOE_EUNSUPPORTED for an inter outside the limits. */
int moe_draft_init(moe_verify_ctx *ctx, const moe_draft_weights *weights, void *stream);

/* K draft steps for B sequences right after a verifier pass of Kv drafts:
 *   hidden       [B*(Kv+1)][H] float32 device: that pass's hidden_out (required);
 *   accepted_len [B] int32 device and committed [B][Kv+1] int32 device: accept_greedy's
 *                outputs for that pass;
 *   drafts       [B][K] int32 device out: the next pass's drafts.
 * Step 1 of sequence b takes the hidden row b*(Kv+1) + n_b and the token
 * committed[b][n_b] (n_b = accepted_len[b]); later steps take the previous step's output.
 * B >= 1, Kv >= 0, K >= 1, B*(Kv+1) <= max_positions. Enqueues work on `stream` only (no
 * synchronisation, allocation or host copy: graph-capturable). It uses the context's
 * verify workspace, so it must not overlap a moe_verify_step on the same context. */
int moe_draft_step(moe_verify_ctx *ctx, const float *hidden, const int32_t *accepted_len,
                   const int32_t *committed, int32_t B, int32_t Kv, int32_t K, int32_t *drafts,
                   void *stream);

/* ---- measurement hooks (not on the verify path) ------------------------------------ */

/* Kernel classes timed by the profiling hook, in this order. */
enum {
  MOE_PROF_NORM_ROUTE = 0, /* combine + residual + RMSNorm + router + top-k (per block), final norm */
  MOE_PROF_PLAN = 1,       /* expert-major slot ordering + GEMM work list (per block)              */
  MOE_PROF_GEMM_UP = 2,    /* gate/up projections + SwiGLU (per block)                              */
  MOE_PROF_GEMM_DOWN = 3,  /* down projection + gate scaling (per block)                            */
  MOE_PROF_LM_HEAD = 4,    /* LM-head logits + per-tile top-1/top-2                                  */
  MOE_PROF_ARGMAX = 5,     /* argmax reduction across vocabulary tiles                              */
  MOE_PROF_KINDS = 6
};

/* Turn per-launch timing on (1) or off (0) and clear the totals. While on, every
 * moe_verify_step records a HIP event before and after each kernel launch on its stream
 * (do not capture such steps in a graph). Events are created here, not in the step, as
 * timing-only events without a system-scope fence. */
int moe_verify_profile(moe_verify_ctx *ctx, int enable);

/* Wait for the last profiled step, add its per-launch durations to the totals, and copy
 * the totals out: ms[MOE_PROF_KINDS] summed milliseconds, launches[MOE_PROF_KINDS]
 * launch counts (host arrays; either may be NULL). */
int moe_verify_profile_read(moe_verify_ctx *ctx, double *ms, int64_t *launches);

/* Wait for the device and copy the last step's routed-slot count of every routed expert
 * of every block to counts [L][E] int32 (host memory). */
int moe_verify_expert_counts(moe_verify_ctx *ctx, int32_t *counts);

#ifdef __cplusplus
}
#endif

#endif /* MOE_VERIFY_H */
