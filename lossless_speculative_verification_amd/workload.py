"""Seeded synthetic inputs for the MoE greedy speculative-verification step.

This module holds shapes, seeds and random draws only: none of the method's
arithmetic. Both the CPU oracle (through the tests and the bench) and the HIP
library take their inputs from here, so the two sides see identical arrays.

Workload shapes follow the jina-ocr-v1 model page ("jina-ocr-v1", paragraph on
the architecture): decoder hidden size 1280, 64 routed + 2 shared experts under
top-6 routing, 12 layers, vocabulary 129,280; the verifier pass covers three
drafted tokens (summary paragraph), batch 32 mirrors the concurrency-32
throughput run (efficiency paragraph), the 57.6% acceptance rate is the L4
speculative-decoding paragraph's, and 1,156 visual tokens per page is the
dynamic-resolution cap (architecture paragraph).

Random streams: ``numpy.random.default_rng([seed, layer, tid, index])`` with

    tid 0 router, 1 gate, 2 up, 3 down (index = expert, shared experts after
          the routed ones), 4 LM head (layer = L, index = 1024-row chunk),
    5 hidden states, 6 draft coin flips, 7 random draft ids (layer 0, index 0),
    8 draft-block projection, 9 draft-block gate, 10 up, 11 down (layer = L + 1,
          index 0).

Weights are standard normal float32 draws times the standard deviation
(float32 multiply), then rounded to bfloat16 by torch's round-to-nearest-even
conversion for the bf16 workloads; the fp32 workload keeps the float32 values.
bf16 arrays are returned as ``numpy.uint16`` bit patterns.
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field, replace
from typing import Optional

import numpy as np

TID_ROUTER, TID_GATE, TID_UP, TID_DOWN, TID_LM, TID_HIDDEN, TID_COIN, TID_DRAFT = range(8)
TID_MTP_PROJ, TID_MTP_GATE, TID_MTP_UP, TID_MTP_DOWN = range(8, 12)
DRAFT_INTER = 1792  # intermediate width of the draft block's dense SwiGLU (chosen: 2 x 896)
LM_CHUNK_ROWS = 1024


@dataclass(frozen=True)
class Workload:
    """One synthetic verify-step workload (shapes, dtype, seed, draft statistics)."""

    name: str
    hidden: int            # H
    n_routed: int          # E
    top_k: int             # k
    n_shared: int          # S
    inter: int             # I, SwiGLU intermediate width per expert
    n_layers: int          # L
    vocab: int             # V; 0 means no LM head (hidden states out only)
    wdtype: str            # "f32" or "bf16"
    batch: int             # B sequences
    drafts: int            # K drafted tokens per sequence
    p_match: float         # probability that a draft equals the verifier's choice
    seed: int
    rms_eps: float = 1e-6
    weight_std: float = 0.02
    bias_value: float = 0.0     # router bias added to the first n_biased experts
    n_biased: int = 0

    @property
    def positions(self) -> int:
        return self.batch * (self.drafts + 1)

    def with_(self, **kw) -> "Workload":
        return replace(self, **kw)


WORKLOADS = {
    # 1 layer, H=128, 8 routed top-2 + 1 shared, I=64, V=1000, fp32, B=1, K=3.
    "tiny_fp32": Workload("tiny_fp32", 128, 8, 2, 1, 64, 1, 1000, "f32", 1, 3, 0.6, 1000),
    # 1 real-width layer + LM head, bf16 weights, B=1, K=3.
    "layer1_bf16": Workload("layer1_bf16", 1280, 64, 6, 2, 896, 1, 129280, "bf16", 1, 3, 0.576, 1001),
    # 12 layers + LM head, B=32, K=3 (128 positions): the batched decode verify step.
    "decode_b32_k3": Workload("decode_b32_k3", 1280, 64, 6, 2, 896, 12, 129280, "bf16", 32, 3, 0.576, 1002),
    # Same weights, K=1 (64 positions).
    "decode_b32_k1": Workload("decode_b32_k1", 1280, 64, 6, 2, 896, 12, 129280, "bf16", 32, 1, 0.576, 1002),
    # One layer over 32 pages x 1,156 visual tokens = 36,992 positions, no LM head.
    "prefill_32x1156": Workload("prefill_32x1156", 1280, 64, 6, 2, 896, 1, 0, "bf16", 36992, 0, 0.0, 1003),
    # 12 layers + LM head, B=128, K=3, router bias +3.0 on experts 0..7, p=0.8.
    "skewed_b128_k3": Workload("skewed_b128_k3", 1280, 64, 6, 2, 896, 12, 129280, "bf16", 128, 3, 0.8, 1004,
                               bias_value=3.0, n_biased=8),
    # Same shape with bias +1.367 on experts 0..7: about 70% of the routed slots land on them
    # (the share the skewed stress case asks for; +3.0 puts nearly all there), while every
    # expert still gets some.
    "skewed70_b128_k3": Workload("skewed70_b128_k3", 1280, 64, 6, 2, 896, 12, 129280, "bf16", 128, 3, 0.8, 1004,
                                 bias_value=1.367, n_biased=8),
}


@dataclass
class Weights:
    """Decoder weights in the layouts the library's init call takes.

    router [L][E][H]; router_bias [L][E] float32 or None;
    w_gate, w_up [L][E+S][I][H]; w_down [L][E+S][H][I]; lm_head [V][H] or None.
    Matrices are numpy.uint16 bf16 bit patterns (wdtype "bf16") or float32.
    """

    wdtype: str
    router: np.ndarray
    router_bias: Optional[np.ndarray]
    w_gate: np.ndarray
    w_up: np.ndarray
    w_down: np.ndarray
    lm_head: Optional[np.ndarray]
    extra: dict = field(default_factory=dict)


def _threads() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def _to_bf16_bits(x: np.ndarray) -> np.ndarray:
    import torch

    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def _draw(seed: int, layer: int, tid: int, index: int, shape, std: float, wdtype: str) -> np.ndarray:
    rng = np.random.default_rng([seed, layer, tid, index])
    w = rng.standard_normal(shape, dtype=np.float32) * np.float32(std)
    return _to_bf16_bits(w) if wdtype == "bf16" else w


def make_weights(wl: Workload, layers: Optional[range] = None, lm_head: bool = True) -> Weights:
    """Draw every weight of ``wl`` (or only ``layers``; the others stay zero-sized).

    Generation runs in a thread pool (numpy's generators release the GIL); the
    values do not depend on the thread count.
    """
    L, E, S, H, I, V = wl.n_layers, wl.n_routed, wl.n_shared, wl.hidden, wl.inter, wl.vocab
    layers = range(L) if layers is None else layers
    dt = np.uint16 if wl.wdtype == "bf16" else np.float32
    router = np.zeros((L, E, H), dt)
    w_gate = np.zeros((L, E + S, I, H), dt)
    w_up = np.zeros((L, E + S, I, H), dt)
    w_down = np.zeros((L, E + S, H, I), dt)
    jobs = []
    for l in layers:
        jobs.append((router, (l,), l, TID_ROUTER, 0, (E, H)))
        for e in range(E + S):
            jobs.append((w_gate, (l, e), l, TID_GATE, e, (I, H)))
            jobs.append((w_up, (l, e), l, TID_UP, e, (I, H)))
            jobs.append((w_down, (l, e), l, TID_DOWN, e, (H, I)))
    lm = None
    if lm_head and V > 0:
        lm = np.zeros((V, H), dt)
        for c in range(0, V, LM_CHUNK_ROWS):
            rows = min(LM_CHUNK_ROWS, V - c)
            jobs.append((lm, (slice(c, c + rows),), L, TID_LM, c // LM_CHUNK_ROWS, (rows, H)))

    def run(job):
        dst, idx, layer, tid, index, shape = job
        dst[idx] = _draw(wl.seed, layer, tid, index, shape, wl.weight_std, wl.wdtype)

    with ThreadPoolExecutor(_threads()) as ex:
        list(ex.map(run, jobs))

    bias = None
    if wl.n_biased > 0:
        bias = np.zeros((L, E), np.float32)
        bias[:, : wl.n_biased] = np.float32(wl.bias_value)
    return Weights(wl.wdtype, router, bias, w_gate, w_up, w_down, lm)


def make_hidden(wl: Workload, positions: Optional[int] = None) -> np.ndarray:
    """Layer-0 hidden states, N(0, 1) float32, shape [T][H] (row b*(K+1)+j)."""
    T = wl.positions if positions is None else positions
    rng = np.random.default_rng([wl.seed, 0, TID_HIDDEN, 0])
    return rng.standard_normal((T, wl.hidden), dtype=np.float32)


def make_drafts(wl: Workload, verifier_ids: np.ndarray) -> np.ndarray:
    """Draft ids [B][K] int32: the verifier's own choice with probability p, else uniform in [0, V).

    ``verifier_ids`` is the verifier's argmax per position, shape [B*(K+1)]; draft i of
    sequence b is compared against position b*(K+1)+i, so it is taken from there.
    """
    B, K, V = wl.batch, wl.drafts, max(wl.vocab, 1)
    y = np.asarray(verifier_ids, dtype=np.int64).reshape(B, K + 1)
    coins = np.random.default_rng([wl.seed, 0, TID_COIN, 0]).random((B, K))
    ids = np.random.default_rng([wl.seed, 0, TID_DRAFT, 0]).integers(0, V, (B, K))
    return np.where(coins < wl.p_match, y[:, :K], ids).astype(np.int32)


@dataclass
class DraftWeights:
    """Weights of the draft block (multi-token-prediction head) in the layouts its init
    call takes: proj [H][2H] (input = [normalised hidden, normalised token embedding]),
    w_gate, w_up [I_d][H], w_down [H][I_d]; bf16 bit patterns or float32 as the
    verifier's. The token embedding is the verifier's LM-head matrix (tied)."""

    wdtype: str
    inter: int
    proj: np.ndarray
    w_gate: np.ndarray
    w_up: np.ndarray
    w_down: np.ndarray


def make_draft_weights(wl: Workload, inter: int = DRAFT_INTER) -> DraftWeights:
    """Seeded N(0, weight_std) draft-block weights for ``wl`` (streams tid 8..11, layer L + 1)."""
    H, L = wl.hidden, wl.n_layers
    d = lambda tid, shape: _draw(wl.seed, L + 1, tid, 0, shape, wl.weight_std, wl.wdtype)
    return DraftWeights(wl.wdtype, inter, d(TID_MTP_PROJ, (H, 2 * H)), d(TID_MTP_GATE, (inter, H)),
                        d(TID_MTP_UP, (inter, H)), d(TID_MTP_DOWN, (H, inter)))
