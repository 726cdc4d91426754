"""CPU oracle for greedy speculative verification through a mixture-of-experts decoder.

TEST INFRASTRUCTURE ONLY. Nothing but the tests, the package's smoke check and the
bench's CPU-baseline leg may import or call this module. The library's product path
never does, and this module imports nothing from the library.

It is the plain definition of what one verifier pass computes, written in numpy
float64, position by position where that is clearer and with library matmuls and
sorts as single steps. It shares no code, table or constant with the HIP kernels.

Sources (cited by page title and paragraph; the pages have no numbered sections):

* "jina-ocr-v1" model page, summary paragraph: drafted tokens are checked by the
  verifier greedily; the result is the same as plain greedy decoding, and a pass
  commits the accepted drafts plus one token of the verifier's own.
* same page, architecture paragraph: decoder of 12 layers, hidden 1280, 64 routed
  experts plus 2 shared ones under top-6 routing, vocabulary 129,280.
* same page, FastMTP paragraph, and usage paragraph: greedy verification makes the
  speculative path lossless; turning speculation on or off changes only speed.
* "Jina AI Releases jina-ocr-v1 ..." news page, paragraph on FastMTP: the decoder
  keeps only the drafts that agree with its own choice.

Where the pages are silent, this oracle takes these readings (the same list is in
the design notes):

1. router scores are a softmax over the routed experts' logits (optionally biased);
2. the k selected gates are renormalised to sum to one (a softmax over the k
   selected logits);
3. ties in top-k selection and in the LM-head argmax go to the lower index;
4. a router bias is added to the logits before selection and softmax;
5. shared experts have the routed experts' shape, are always on, weight 1;
6. each expert is a bias-free SwiGLU: down(silu(gate x) * up x);
7. blocks are pre-norm: x <- x + MoE(RMSNorm(x)), RMSNorm with gamma 1 and eps
   inside the square root, and a final RMSNorm before the LM head;
8. for bf16 weights (bf16 weights with float32 accumulation), bf16 is materialised
   at the activation input of every matrix product: the RMSNorm output (the input of
   the router, the experts and the LM head) and the SwiGLU output (the input of the
   down projection). Products are accumulated exactly (float64 here) and their
   results are kept unrounded: router logits, each expert's output (the down
   projection's result, before its gate), the gated sum and the logits; the
   residual stream is float32;
9. acceptance: the longest prefix of drafts equal to the verifier's argmax at the
   matching positions is accepted, and the verifier's token after it is added;
10. the draft block (the pages name FastMTP, a multi-token-prediction head that drafts
   three tokens ahead, without fixing its shape): one block applied K times. Step i
   takes a hidden state h and a token t (at step 1 the verifier's residual stream,
   before its final norm, at the last accepted position, and the last committed
   token), forms [RMSNorm(h), RMSNorm(E[t])] with E the LM-head matrix (tied token
   embedding), projects 2H -> H (bias-free), adds a pre-norm dense SwiGLU block with
   a residual, applies the final RMSNorm and the shared LM head, and drafts the
   greedy token; its hidden state and token feed step i + 1. bf16 is materialised
   as in reading 8, at the inputs of the products: the two normalised halves, the
   block's normalised input, its SwiGLU product and the LM-head input; the projection
   output and the block's output are float32 like the verifier's residual stream.
"""
from __future__ import annotations

from typing import Callable, List, Optional, Sequence

import numpy as np

# --------------------------------------------------------------------------- numbers


def bf16_bits_to_f64(bits) -> np.ndarray:
    """Value of bfloat16 bit patterns (uint16): the high half of a float32."""
    u = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return u.view(np.float32).astype(np.float64)


def as_f64(w, wdtype: str) -> np.ndarray:
    """Weights as float64: bf16 bit patterns are widened, float32 values kept."""
    return bf16_bits_to_f64(w) if wdtype == "bf16" else np.asarray(w, dtype=np.float64)


def round_bf16(x) -> np.ndarray:
    """Nearest bfloat16 value of each element (8 significant bits, ties to even).

    Written from the format's definition: x = m * 2**e with 0.5 <= |m| < 1, keep 8
    significant bits of m with round-half-even, scale back. Valid for zero and for
    normal bf16 magnitudes (|x| >= 2**-126), which is all this method produces.
    """
    x = np.asarray(x, dtype=np.float64)
    nz = x[x != 0]
    if nz.size and np.min(np.abs(nz)) < 2.0 ** -126:
        raise ValueError("round_bf16: subnormal magnitude outside the oracle's range")
    m, e = np.frexp(x)
    return np.ldexp(np.rint(m * 256.0), e - 8)


# --------------------------------------------------------------------------- layer parts


def rms_norm(x, eps: float) -> np.ndarray:
    """RMSNorm with unit gain: x / sqrt(mean(x^2) + eps) over the last axis (reading 7)."""
    x = np.asarray(x, dtype=np.float64)
    return x / np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + eps)


def router_logits(a, w_router, bias=None) -> np.ndarray:
    """Router logits r = a W_r^T (+ bias) for every position and routed expert (readings 1, 4)."""
    r = np.asarray(a, np.float64) @ np.asarray(w_router, np.float64).T
    if bias is not None:
        r = r + np.asarray(bias, np.float64)[None, :]
    return r


def select_topk(r, k: int):
    """Top-k experts per position, architecture paragraph's top-6 routing (reading 3).

    Returns (ids [T,k] in slot order: logit descending, lower index first on equal
    logits; gap [T] = k-th largest minus (k+1)-th largest logit, +inf when k == E).
    A stable sort of -r keeps the lower index first among equal logits.
    """
    r = np.asarray(r, np.float64)
    order = np.argsort(-r, axis=1, kind="stable")
    ids = order[:, :k]
    if k < r.shape[1]:
        srt = np.take_along_axis(r, order, axis=1)
        gap = srt[:, k - 1] - srt[:, k]
    else:
        gap = np.full(r.shape[0], np.inf)
    return ids, gap


def gate_weights(r, ids) -> np.ndarray:
    """Gates of the selected experts: softmax of their logits (readings 1, 2).

    Equal to the full softmax over all routed experts renormalised over the selection.
    """
    sel = np.take_along_axis(np.asarray(r, np.float64), ids, axis=1)
    z = np.exp(sel - sel.max(axis=1, keepdims=True))
    return z / z.sum(axis=1, keepdims=True)


def silu(z) -> np.ndarray:
    """silu(z) = z * sigmoid(z)."""
    z = np.asarray(z, np.float64)
    return z / (1.0 + np.exp(-z))


def expert_ffn(a_rows, w_gate, w_up, w_down, round_bf16_h: bool) -> np.ndarray:
    """One SwiGLU expert on a set of positions (reading 6): (silu(a Wg^T) * (a Wu^T)) Wd^T.

    With round_bf16_h (bf16 weights, reading 8) the SwiGLU product, the input of the
    down projection, is rounded to bf16; the expert's output is exact.
    """
    h = silu(a_rows @ w_gate.T) * (a_rows @ w_up.T)
    if round_bf16_h:
        h = round_bf16(h)
    return h @ w_down.T


def moe_layer(cfg, weights, layer: int, x) -> dict:
    """One pre-norm MoE block on positions x [T,H] float32 (architecture paragraph).

    Returns a dict with
      a     [T,H]  normalised (and bf16-rounded) block input,
      r     [T,E]  router logits,
      ids   [T,k]  selected experts in slot order,
      gates [T,k]  their gates,
      gap   [T]    routing boundary gap r_(k) - r_(k+1),
      m     [T,H]  block output (routed mixture plus shared experts),
      x_next[T,H]  float32(x + m).
    """
    bf = cfg.wdtype == "bf16"
    E, S, k = cfg.n_routed, cfg.n_shared, cfg.top_k
    x = np.asarray(x, np.float32)
    u = rms_norm(x, cfg.rms_eps)
    a = round_bf16(u) if bf else u
    bias = None if weights.router_bias is None else weights.router_bias[layer]
    r = router_logits(a, as_f64(weights.router[layer], cfg.wdtype), bias)
    ids, gap = select_topk(r, k)
    gates = gate_weights(r, ids)

    m = np.zeros(x.shape, np.float64)
    for e in range(E):
        tok, slot = np.nonzero(ids == e)
        if tok.size == 0:
            continue
        y = expert_ffn(a[tok], as_f64(weights.w_gate[layer, e], cfg.wdtype),
                       as_f64(weights.w_up[layer, e], cfg.wdtype),
                       as_f64(weights.w_down[layer, e], cfg.wdtype), bf)
        m[tok] += gates[tok, slot][:, None] * y
    for s in range(S):
        m += expert_ffn(a, as_f64(weights.w_gate[layer, E + s], cfg.wdtype),
                        as_f64(weights.w_up[layer, E + s], cfg.wdtype),
                        as_f64(weights.w_down[layer, E + s], cfg.wdtype), bf)
    x_next = (x.astype(np.float64) + m).astype(np.float32)
    return {"a": a, "r": r, "ids": ids, "gates": gates, "gap": gap, "m": m, "x_next": x_next}


def final_norm(cfg, x) -> np.ndarray:
    """Final RMSNorm before the LM head (reading 7), bf16-rounded for bf16 weights."""
    u = rms_norm(np.asarray(x, np.float32), cfg.rms_eps)
    return round_bf16(u) if cfg.wdtype == "bf16" else u


def lm_head_argmax(a, lm_head, wdtype: str, chunk: int = 8192):
    """Greedy choice per position over the LM head logits a W_lm^T (summary paragraph).

    The logits are formed chunk by chunk of vocabulary rows (float64) and never kept
    whole. Returns (ids [T] with the lower index winning ties, margin [T] = largest
    minus second largest logit over the other indices, top1 [T]).
    """
    a = np.asarray(a, np.float64)
    T, V = a.shape[0], lm_head.shape[0]
    best = np.full(T, -np.inf)
    best_id = np.zeros(T, np.int64)
    second = np.full(T, -np.inf)
    rows = np.arange(T)
    for c0 in range(0, V, chunk):
        logits = a @ as_f64(lm_head[c0:c0 + chunk], wdtype).T
        i1 = np.argmax(logits, axis=1)            # first occurrence: lowest index
        v1 = logits[rows, i1]
        rest = logits.copy()
        rest[rows, i1] = -np.inf
        v2 = rest.max(axis=1) if logits.shape[1] > 1 else np.full(T, -np.inf)
        take = v1 > best                          # equal value later in the vocab loses
        second = np.where(take, np.maximum(best, v2), np.maximum(second, v1))
        best_id = np.where(take, c0 + i1, best_id)
        best = np.where(take, v1, best)
    return best_id, best - second, best


# --------------------------------------------------------------------------- the pass


def verify_step(cfg, weights, x0, layers: Optional[int] = None) -> dict:
    """One verifier pass over positions x0 [T,H] (row b*(K+1)+j is position j of sequence b).

    Runs the MoE blocks, then (when the config has a vocabulary) the final norm and the
    LM-head argmax. Positions are independent (attention is outside this path), so any
    subset of rows can be passed on its own. Returns per-layer dicts and the final
    hidden state x_L (before the final norm), ids, margin.
    """
    x = np.asarray(x0, np.float32)
    n_layers = cfg.n_layers if layers is None else layers
    per_layer = []
    for l in range(n_layers):
        out = moe_layer(cfg, weights, l, x)
        x = out.pop("x_next")
        out.pop("a")
        out.pop("r")
        per_layer.append(out)
    res = {"layers": per_layer, "hidden_out": x}
    if cfg.vocab > 0 and weights.lm_head is not None:
        a = final_norm(cfg, x)
        ids, margin, top1 = lm_head_argmax(a, weights.lm_head, cfg.wdtype)
        res.update(ids=ids, margin=margin, top1=top1)
    return res


def accept(drafts, verifier_ids, B: int, K: int):
    """Greedy acceptance (summary paragraph; news page's FastMTP paragraph).

    Draft i of sequence b is accepted while it equals the verifier's choice at position
    b*(K+1)+i and every earlier draft was accepted. The pass commits the n accepted
    drafts plus the verifier's choice after them, i.e. verifier_ids[b, 0..n]; the
    rest of the committed row is -1. Returns (accepted_len [B], committed [B, K+1]).
    """
    d = np.asarray(drafts, np.int64).reshape(B, K)
    y = np.asarray(verifier_ids, np.int64).reshape(B, K + 1)
    n = np.zeros(B, np.int32)
    committed = np.full((B, K + 1), -1, np.int32)
    for b in range(B):
        i = 0
        while i < K and d[b, i] == y[b, i]:
            i += 1
        n[b] = i
        committed[b, : i + 1] = y[b, : i + 1]
    return n, committed


# --------------------------------------------------------------------------- decoding loops

NextToken = Callable[[List[List[int]]], Sequence[int]]


def greedy_decode(next_token: NextToken, prompt: Sequence[int], n_new: int) -> List[int]:
    """Plain greedy decoding: one verifier call per token."""
    out = list(prompt)
    while len(out) < len(prompt) + n_new:
        out.append(int(next_token([out])[0]))
    return out


def speculative_decode(next_token: NextToken, draft: Callable[[List[int], int], Sequence[int]],
                       prompt: Sequence[int], n_new: int, K: int):
    """Draft K tokens, verify all K+1 prefixes in one pass, accept greedily, repeat.

    ``next_token(prefixes)`` returns the verifier's greedy choice after each prefix;
    ``draft(prefix, K)`` proposes K ids. Returns (tokens, number of verifier passes).
    """
    out = list(prompt)
    passes = 0
    while len(out) < len(prompt) + n_new:
        d = [int(v) for v in draft(out, K)]
        y = [int(v) for v in next_token([out + d[:j] for j in range(K + 1)])]
        n, committed = accept(np.array([d], np.int64).reshape(1, K), np.array(y), 1, K)
        out += [int(v) for v in committed[0, : n[0] + 1]]
        passes += 1
    return out[: len(prompt) + n_new], passes


# --------------------------------------------------------------------------- draft block


def draft_inputs(hidden, accepted_len, committed, K: int):
    """Inputs of the first draft step after a verifier pass (reading 10): per sequence b,
    the verifier's hidden row b*(K+1) + n_b (n_b accepted drafts) and the last committed
    token committed[b][n_b] (the verifier's own token after the accepted drafts)."""
    n = np.asarray(accepted_len, np.int64)
    B = n.shape[0]
    hidden = np.asarray(hidden, np.float32).reshape(B, K + 1, -1)
    com = np.asarray(committed, np.int64).reshape(B, K + 1)
    rows = np.arange(B)
    return hidden[rows, n], com[rows, n]


def draft_step(cfg, weights, dweights, h, tok, K: int) -> dict:
    """K recursive steps of the draft block (reading 10) for B sequences.

    h [B,H] float32 hidden states, tok [B] tokens. Returns drafts [B,K] (int64),
    margin [B,K] (top-1 minus top-2 LM logit of each draft) and hidden [K,B,H] (the
    block's float32 output after each step, the next step's h).
    """
    bf = cfg.wdtype == "bf16"
    rnd = round_bf16 if bf else (lambda v: np.asarray(v, np.float64))
    wp = as_f64(dweights.proj, cfg.wdtype)
    wg, wu, wd = (as_f64(w, cfg.wdtype) for w in (dweights.w_gate, dweights.w_up, dweights.w_down))
    h = np.asarray(h, np.float32)
    tok = np.asarray(tok, np.int64)
    B = h.shape[0]
    drafts = np.zeros((B, K), np.int64)
    margins = np.zeros((B, K))
    hidden = np.zeros((K, B, h.shape[1]), np.float32)
    for i in range(K):
        emb = as_f64(weights.lm_head[tok], cfg.wdtype)
        u = np.concatenate([rnd(rms_norm(h, cfg.rms_eps)), rnd(rms_norm(emb, cfg.rms_eps))], axis=1)
        x = (u @ wp.T).astype(np.float32)                  # projection output, the block's residual
        a = rnd(rms_norm(x, cfg.rms_eps))
        y = expert_ffn(a, wg, wu, wd, bf)                   # the same SwiGLU form as an expert
        x = (x.astype(np.float64) + y).astype(np.float32)
        ids, margin, _ = lm_head_argmax(final_norm(cfg, x), weights.lm_head, cfg.wdtype)
        drafts[:, i], margins[:, i], hidden[i] = ids, margin, x
        h, tok = x, ids
    return {"drafts": drafts, "margin": margins, "hidden": hidden}
