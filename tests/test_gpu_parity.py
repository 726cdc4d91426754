"""GPU parity of the HIP verify path against the CPU oracle, through the C ABI.

Every case prints its name and shape before touching the GPU. Inputs are the seeded
synthetic workloads; expected values come only from the oracle on the same inputs.
"""
import numpy as np
import pytest
import torch

import oracle as O
from lossless_speculative_verification_amd import binding as bnd
from lossless_speculative_verification_amd import workload as W

from gpu_cases import (DEV, GATE, TOL, context, decisive_positions, end_to_end_rel_err, log, oracle_step, row_rel_err,
                       run_debug_layer, run_step)

pytestmark = pytest.mark.gpu

WL = W.WORKLOADS


# ----------------------------------------------------------------------------- acceptance kernel


@pytest.mark.parametrize("B,K", [(1, 0), (1, 1), (3, 2), (32, 3), (129, 5), (1000, 3)])
def test_accept_kernel_bit_exact(B, K):
    log(f"[accept] B={B} K={K}")
    rng = np.random.default_rng(B * 100 + K)
    y = rng.integers(0, 50, (B, K + 1)).astype(np.int32)
    d = np.where(rng.random((B, K)) < 0.7, y[:, :K], rng.integers(-3, 50, (B, K))).astype(np.int32)
    n_ref, c_ref = O.accept(d, y, B, K)
    dd, yd = torch.from_numpy(d).to(DEV), torch.from_numpy(y).to(DEV)
    n = torch.full((B,), -9, dtype=torch.int32, device=DEV)
    c = torch.full((B, K + 1), -9, dtype=torch.int32, device=DEV)
    bnd.accept_greedy(dd, yd, B, K, n, c)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(n.cpu().numpy(), n_ref)
    np.testing.assert_array_equal(c.cpu().numpy(), c_ref)


# ----------------------------------------------------------------------------- full step checks


def _check_step(wl, ref, ids, margin, hout, x, rows=None, min_decisive=1):
    """Compare a GPU pass (restricted to `rows` when the oracle ran on a sample)."""
    sel = slice(None) if rows is None else list(rows)
    tol = TOL[wl.wdtype]
    dec = decisive_positions(ref)
    assert dec.sum() >= min_decisive, f"only {dec.sum()} decisive positions"
    err = end_to_end_rel_err(hout[sel][dec], ref["hidden_out"][dec], x[sel][dec], wl.n_layers)
    log(f"  decisive {dec.sum()}/{len(dec)}  hidden rel err {err:.3e} (tol {tol})")
    assert err <= tol
    if wl.vocab > 0:
        np.testing.assert_array_equal(ids[sel][dec], ref["ids"][dec])
        assert np.all(ids >= 0) and np.all(ids < wl.vocab)
        dm = np.abs(margin[sel][dec] - ref["margin"][dec]).max()
        log(f"  argmax exact on decisive; margin max abs diff {dm:.2e}")
        assert dm < (1e-4 if wl.wdtype == "f32" else 2e-2)
    return dec


def _check_accept(wl, ref_ids, gpu_ids, dec):
    """Accept on the GPU with drafts built from the oracle's choices; exact on sequences
    whose positions are all decisive."""
    B, K = wl.batch, wl.drafts
    drafts = W.make_drafts(wl, ref_ids)
    n_ref, c_ref = O.accept(drafts, ref_ids, B, K)
    dd = torch.from_numpy(drafts).to(DEV)
    yd = torch.from_numpy(gpu_ids.astype(np.int32)).to(DEV)
    n = torch.empty(B, dtype=torch.int32, device=DEV)
    c = torch.empty(B, K + 1, dtype=torch.int32, device=DEV)
    bnd.accept_greedy(dd, yd, B, K, n, c)
    torch.cuda.synchronize()
    seq_ok = dec.reshape(B, K + 1).all(axis=1)
    np.testing.assert_array_equal(n.cpu().numpy()[seq_ok], n_ref[seq_ok])
    np.testing.assert_array_equal(c.cpu().numpy()[seq_ok], c_ref[seq_ok])
    log(f"  accept exact on {seq_ok.sum()}/{B} sequences; mean accepted {n_ref.mean():.3f}")


def test_tiny_fp32_step():
    wl = WL["tiny_fp32"]
    x = W.make_hidden(wl)
    ref = oracle_step(wl)
    ids, margin, hout = run_step(wl)
    dec = _check_step(wl, ref, ids, margin, hout, x)
    _check_accept(wl, ref["ids"], ids, dec)


@pytest.mark.parametrize("B,K", [(1, 0), (67, 0), (16, 3), (9, 7)])
def test_tiny_fp32_shapes(B, K):
    """T = 1, a ragged T spanning several 16-row tiles and two work items per expert,
    the capacity limit, and a long draft block."""
    wl = WL["tiny_fp32"].with_(batch=B, drafts=K)
    x = W.make_hidden(wl)
    ref = O.verify_step(wl, W.make_weights(wl), x)
    ids, margin, hout = run_step(wl, x, B, K)
    _check_step(wl, ref, ids, margin, hout, x)


def test_tiny_fp32_debug_layer():
    wl = WL["tiny_fp32"]
    x = W.make_hidden(wl, 200)
    ref = O.moe_layer(wl, W.make_weights(wl), 0, x)
    m, tid, tw = run_debug_layer(wl, 0, x)
    dec = ref["gap"] > GATE
    np.testing.assert_array_equal(tid[dec], ref["ids"][dec])
    assert np.abs(tw[dec] - ref["gates"][dec]).max() < 1e-5
    np.testing.assert_allclose(tw.sum(axis=1), 1.0, atol=1e-5)
    err = row_rel_err(m[dec], ref["m"][dec])
    log(f"  decisive {dec.sum()}/200 m rel err {err:.2e}")
    assert err <= TOL["f32"]


@pytest.mark.parametrize("B,K", [(16, 3), (1100, 3)])
def test_wider_fp32_model(B, K):
    """Float32 weights at a wider shape than the tiny model (hidden 512: eight 256-byte
    blocks per row, 16 routed experts top-4 + 1 shared, two stacked blocks, vocabulary
    2,000): 64 positions (the split norm/router kernel, the self-planning gate/up) and
    4,400 positions (the 16-position norm/router kernel and the chunked plan), against the
    oracle at the float32 tolerance."""
    wl = WL["tiny_fp32"].with_(name="fp32_wide", hidden=512, inter=256, n_routed=16, top_k=4, n_shared=1,
                               n_layers=2, vocab=2000, batch=B, drafts=K, seed=1010)
    log(f"[fp32 wide] B={B} K={K} T={wl.positions}")
    x = W.make_hidden(wl)
    ref = oracle_step(wl)
    ids, margin, hout = run_step(wl, x, B, K)
    dec = _check_step(wl, ref, ids, margin, hout, x, min_decisive=int(0.5 * wl.positions))
    _check_accept(wl, ref["ids"], ids, dec)


@pytest.mark.parametrize("wdtype,H,B,K,L", [("bf16", 4096, 16, 3, 2), ("bf16", 4096, 75, 3, 2), ("bf16", 4096, 1100, 3, 1),
                                             ("f32", 2048, 16, 3, 2), ("f32", 2048, 1100, 3, 1)])
def test_widest_rows(wdtype, H, B, K, L):
    """The widest rows the library takes (hidden 4,096 in bf16, 2,048 in float32): the
    norm/router kernels' widest register layouts (four float4 per lane and quarter in the
    split kernel, sixteen per lane in the 16-position kernel) and contractions of 32 K
    blocks in the streaming and tiled GEMMs and the LM head, at 64, 300 and 4,400
    positions (8 routed experts top-2 + 1 shared, vocabulary 1,000)."""
    base = WL["layer1_bf16"] if wdtype == "bf16" else WL["tiny_fp32"]
    wl = base.with_(name=f"wide_{wdtype}_{H}_b{B}", hidden=H, inter=256, n_routed=8, top_k=2, n_shared=1,
                    n_layers=L, vocab=1000, batch=B, drafts=K, seed=2020)
    log(f"[widest rows] {wdtype} H={H} B={B} K={K} L={L} T={wl.positions}")
    x = W.make_hidden(wl)
    ref = oracle_step(wl)
    ids, margin, hout = run_step(wl, x, B, K)
    dec = _check_step(wl, ref, ids, margin, hout, x, min_decisive=int(0.5 * wl.positions))
    _check_accept(wl, ref["ids"], ids, dec)


@pytest.mark.parametrize("wdtype,B,K", [("bf16", 16, 3), ("bf16", 75, 3), ("f32", 16, 3)])
def test_widest_intermediate(wdtype, B, K):
    """The widest expert the library takes (intermediate 16,384, hidden 256): down
    contractions of 128 K blocks (16,384 elements of h per row) and 1,024 gate/up column
    pairs per expert, streaming (64 positions) and tiled (300)."""
    base = WL["layer1_bf16"] if wdtype == "bf16" else WL["tiny_fp32"]
    wl = base.with_(name=f"wide_inter_{wdtype}_b{B}", hidden=256, inter=16384, n_routed=8, top_k=2, n_shared=1,
                    n_layers=2, vocab=1000, batch=B, drafts=K, seed=3030)
    log(f"[widest intermediate] {wdtype} I=16384 B={B} K={K} T={wl.positions}")
    x = W.make_hidden(wl)
    ref = oracle_step(wl)
    ids, margin, hout = run_step(wl, x, B, K)
    dec = _check_step(wl, ref, ids, margin, hout, x, min_decisive=int(0.5 * wl.positions))
    _check_accept(wl, ref["ids"], ids, dec)


def test_layer1_bf16_step():
    wl = WL["layer1_bf16"]
    x = W.make_hidden(wl)
    ref = oracle_step(wl)
    ids, margin, hout = run_step(wl)
    dec = _check_step(wl, ref, ids, margin, hout, x, min_decisive=0)
    _check_accept(wl, ref["ids"], ids, dec)


def test_layer1_bf16_speculation_off():
    wl = WL["layer1_bf16"].with_(drafts=0)
    from gpu_cases import host_weights
    x = W.make_hidden(wl)
    ref = O.verify_step(wl, host_weights(wl), x)
    ids, margin, hout = run_step(wl, x, 1, 0)
    _check_step(wl, ref, ids, margin, hout, x, min_decisive=0)


def test_layer1_bf16_debug_layer_256_positions():
    wl = WL["layer1_bf16"]
    from gpu_cases import host_weights
    x = W.make_hidden(wl, 256)
    ref = O.moe_layer(wl, host_weights(wl), 0, x)
    m, tid, tw = run_debug_layer(wl, 0, x)
    dec = ref["gap"] > GATE
    assert dec.sum() > 150
    np.testing.assert_array_equal(tid[dec], ref["ids"][dec])
    assert np.abs(tw[dec] - ref["gates"][dec]).max() < 1e-3
    err = row_rel_err(m[dec], ref["m"][dec])
    log(f"  decisive {dec.sum()}/256 m rel err {err:.2e}")
    assert err <= TOL["bf16"]


# ----------------------------------------------------------------------------- both expert-GEMM kernels

# A narrow bf16 model without LM head: H = 384 ends the down projection in a partial
# 256-column tile of the tiled kernel, 16 routed experts top-4 give ragged per-expert
# row counts, one shared expert, two blocks. Position counts straddle the switch from
# the streaming expert kernel (fewer than 256 positions) to the tiled one, and 5000
# positions (20,000 routed slots) take the multi-workgroup routing plan.
SMALL_BF16 = WL["layer1_bf16"].with_(name="small_bf16", hidden=384, inter=256, n_routed=16, top_k=4, n_shared=1,
                                     vocab=0, n_layers=2, drafts=0)


@pytest.mark.parametrize("T", [255, 256, 300, 1100, 5000])
def test_small_bf16_both_gemm_paths(T):
    from gpu_cases import host_weights
    wl = SMALL_BF16.with_(batch=T)
    x = W.make_hidden(wl)
    w = host_weights(wl)
    ref = O.moe_layer(wl, w, 0, x)
    m, tid, tw = run_debug_layer(wl, 0, x)
    dec = ref["gap"] > GATE
    assert dec.sum() > T // 2
    np.testing.assert_array_equal(tid[dec], ref["ids"][dec])
    assert np.abs(tw[dec] - ref["gates"][dec]).max() < 1e-3
    err = row_rel_err(m[dec], ref["m"][dec])
    log(f"  layer 0: decisive {dec.sum()}/{T} m rel err {err:.2e}")
    assert err <= TOL["bf16"]
    full = O.verify_step(wl, w, x)
    _, _, hout = run_step(wl, x, T, 0)
    _check_step(wl, full, None, None, hout, x, min_decisive=T // 4)


@pytest.mark.parametrize("wdtype,E,k,S,T", [("f32", 8, 1, 0, 200), ("f32", 8, 8, 1, 200), ("bf16", 64, 1, 2, 300),
                                             ("bf16", 64, 64, 0, 260), ("bf16", 16, 16, 1, 1100),
                                             ("f32", 1, 1, 1, 64), ("bf16", 1, 1, 0, 300)])
def test_routing_extremes(wdtype, E, k, S, T):
    """Top-1 routing (every gate exactly 1), every expert selected (k = E: a dense softmax
    mixture; at 260 and 1,100 positions on the tiled GEMM with every expert hot), no
    shared expert, and a single routed expert (every position on it: a dense block), through
    one block, against the oracle."""
    base = WL["tiny_fp32"] if wdtype == "f32" else SMALL_BF16
    wl = base.with_(name=f"route_{wdtype}_{E}_{k}_{S}", n_routed=E, top_k=k, n_shared=S, n_layers=1, vocab=0,
                    batch=T, drafts=0, seed=1020 + E + k + S)
    log(f"[routing extremes] {wdtype} E={E} k={k} S={S} T={T}")
    from gpu_cases import host_weights
    x = W.make_hidden(wl)
    ref = O.moe_layer(wl, host_weights(wl), 0, x)
    m, tid, tw = run_debug_layer(wl, 0, x)
    dec = ref["gap"] > GATE  # +inf when k = E: nothing is left out
    assert dec.sum() > T // 2
    gtol = 1e-5 if wdtype == "f32" else 1e-3
    if k == E:
        # every expert once per position; the slot order (decreasing logit) is not compared,
        # since 64 logits per position hold near-equal neighbours: gates by expert instead
        np.testing.assert_array_equal(np.sort(tid, axis=1), np.broadcast_to(np.arange(E), (T, E)))
        g_gpu, g_ref = np.zeros((T, E)), np.zeros((T, E))
        np.put_along_axis(g_gpu, tid.astype(np.int64), tw, axis=1)
        np.put_along_axis(g_ref, np.asarray(ref["ids"], np.int64), ref["gates"], axis=1)
        assert np.abs(g_gpu - g_ref).max() < gtol
    else:
        np.testing.assert_array_equal(tid[dec], ref["ids"][dec])
        assert np.abs(tw[dec] - ref["gates"][dec]).max() < gtol
    np.testing.assert_allclose(tw.sum(axis=1), 1.0, atol=1e-5)
    if k == 1:
        np.testing.assert_array_equal(tw, 1.0)
    err = row_rel_err(m[dec], ref["m"][dec])
    log(f"  decisive {dec.sum()}/{T} m rel err {err:.2e}")
    assert err <= TOL[wdtype]


# 300 positions: streaming LM head; 256 and 448: the tiled LM head (items of 256 rows, the
# second 3/4 full), with the split plan's cold experts (fewer than 64 rows) among 16
@pytest.mark.parametrize("B,K", [(75, 3), (300, 0), (64, 3), (112, 3)])
def test_small_bf16_step_with_lm_head(B, K):
    """H = 512 with a 1000-token LM head, through the tiled expert kernel (>= 256
    positions): greedy ids exact on decisive positions, acceptance exact."""
    from gpu_cases import host_weights
    wl = SMALL_BF16.with_(name="small_bf16_lm", hidden=512, vocab=1000, batch=B, drafts=K, p_match=0.6)
    x = W.make_hidden(wl)
    ref = O.verify_step(wl, host_weights(wl), x)
    ids, margin, hout = run_step(wl, x, B, K)
    dec = _check_step(wl, ref, ids, margin, hout, x, min_decisive=wl.positions // 4)
    _check_accept(wl, ref["ids"], ids, dec)


# ----------------------------------------------------------------------------- 12-layer decode


@pytest.mark.parametrize("name", ["decode_b32_k3", "decode_b32_k1"])
def test_decode_step(name):
    wl = WL[name]
    x = W.make_hidden(wl)
    ref = oracle_step(wl)
    ids, margin, hout = run_step(wl)
    dec = _check_step(wl, ref, ids, margin, hout, x, min_decisive=5)
    _check_accept(wl, ref["ids"], ids, dec)


@pytest.mark.parametrize("layer", [0, 5, 11])
def test_decode_debug_layer(layer):
    wl = WL["decode_b32_k3"]
    from gpu_cases import host_weights
    x = W.make_hidden(wl)
    ref = O.moe_layer(wl, host_weights(wl), layer, x)
    m, tid, tw = run_debug_layer(wl, layer, x)
    dec = ref["gap"] > GATE
    np.testing.assert_array_equal(tid[dec], ref["ids"][dec])
    err = row_rel_err(m[dec], ref["m"][dec])
    log(f"  layer {layer}: decisive {dec.sum()}/128 m rel err {err:.2e}")
    assert err <= TOL["bf16"]


def test_decode_deterministic_and_batch_invariant():
    wl = WL["decode_b32_k3"]
    x = W.make_hidden(wl)
    a = run_step(wl)
    b = run_step(wl)
    for u, v in zip(a, b):
        np.testing.assert_array_equal(u, v)
    # sequence 5 alone (its 4 positions) gives bitwise the same results as inside the batch
    rows = slice(20, 24)
    ids1, margin1, hout1 = run_step(wl, x[rows].copy(), 1, 3)
    np.testing.assert_array_equal(ids1, a[0][rows])
    np.testing.assert_array_equal(margin1, a[1][rows])
    np.testing.assert_array_equal(hout1, a[2][rows])


# ----------------------------------------------------------------------------- skewed routing


@pytest.mark.parametrize("name", ["skewed_b128_k3", "skewed70_b128_k3"])
def test_skewed_step_sampled(name):
    wl = WL[name]
    x = W.make_hidden(wl)
    seqs = np.random.default_rng(5).choice(wl.batch, 16, replace=False)
    rows = tuple(int(s * (wl.drafts + 1) + j) for s in sorted(seqs) for j in range(wl.drafts + 1))
    ref = oracle_step(wl, rows)
    ids, margin, hout = run_step(wl)
    dec = _check_step(wl, ref, ids, margin, hout, x, rows=rows, min_decisive=1)
    hot = np.mean([np.isin(l["ids"], np.arange(wl.n_biased)).mean() for l in ref["layers"]])
    log(f"  hot-expert slot fraction (sample) {hot:.3f}")


def test_skewed_streaming_step():
    """Hot experts on a decode-sized pass (128 positions, the streaming path, whose gate/up
    GEMM builds the routing plan itself): experts with more than one 32-row work item."""
    wl = WL["skewed_b128_k3"].with_(name="skewed_b32_k3", batch=32)
    x = W.make_hidden(wl)
    ref = oracle_step(wl)
    most = max(int(np.bincount(l["ids"].ravel(), minlength=wl.n_routed).max()) for l in ref["layers"])
    log(f"  largest per-expert slot count {most}")
    assert most > 32, "the case must give some expert more than one work item"
    ids, margin, hout = run_step(wl)
    _check_step(wl, ref, ids, margin, hout, x, min_decisive=5)


# ----------------------------------------------------------------------------- prefill shape


def test_prefill_sampled():
    wl = WL["prefill_32x1156"]
    x = W.make_hidden(wl)
    rows = tuple(int(r) for r in np.sort(np.random.default_rng(6).choice(wl.positions, 384, replace=False)))
    ref = oracle_step(wl, rows)
    _, _, hout = run_step(wl)
    dec = _check_step(wl, ref, None, None, hout, x, rows=rows, min_decisive=200)
    m, tid, tw = run_debug_layer(wl, 0, x)
    lay = ref["layers"][0]
    d = lay["gap"] > GATE
    np.testing.assert_array_equal(tid[list(rows)][d], lay["ids"][d])
    err = row_rel_err(m[list(rows)][d], lay["m"][d])
    log(f"  debug-layer m rel err {err:.2e} on {d.sum()} sampled rows")
    assert err <= TOL["bf16"]
    # the step's block output and the debug hook's agree exactly (same kernels, same order)
    np.testing.assert_array_equal(hout, (x + m).astype(np.float32))


def test_largest_pass_sampled():
    """The largest pass the prefill-shaped model takes (261,882 positions, the work-list
    bound of its configuration): one block on the tiled path with the chunked plan (768
    chunks), checked on 256 sampled rows including the first and the last."""
    wl = WL["prefill_32x1156"].with_(name="prefill_max", batch=261882)
    x = W.make_hidden(wl)
    rng = np.random.default_rng(7)
    rows = tuple(sorted({0, wl.positions - 1} | {int(r) for r in rng.choice(wl.positions, 254, replace=False)}))
    ref = oracle_step(wl, rows)
    _, _, hout = run_step(wl, x)
    _check_step(wl, ref, None, None, hout, x, rows=rows, min_decisive=120)


def test_step_rejects_oversize():
    wl = WL["tiny_fp32"]
    c = context(wl)
    T = c.cfg.max_positions + 4
    xd = torch.zeros(T, wl.hidden, device=DEV)
    ids = torch.empty(T, dtype=torch.int32, device=DEV)
    with pytest.raises(bnd.MoeVerifyError) as ei:
        c.step(xd, T, 0, ids)
    assert ei.value.code == bnd.MOE_EINVAL


def test_graph_replay_matches_eager():
    """The step + acceptance captured in a HIP graph reproduce the eager results on every
    replay, with eager work and synchronisations between replays."""
    wl = WL["layer1_bf16"]
    c = context(wl)
    x = torch.from_numpy(W.make_hidden(wl)).to(DEV)
    T, B, K = wl.positions, wl.batch, wl.drafts
    ids = torch.empty(T, dtype=torch.int32, device=DEV)
    margin = torch.empty(T, dtype=torch.float32, device=DEV)
    n = torch.empty(B, dtype=torch.int32, device=DEV)
    com = torch.empty(B, K + 1, dtype=torch.int32, device=DEV)
    drafts = torch.zeros(B, K, dtype=torch.int32, device=DEV)

    def step():
        c.step(x, B, K, ids, margin)
        bnd.accept_greedy(drafts, ids, B, K, n, com)

    log("[graph] eager reference")
    step()
    torch.cuda.synchronize()
    ref = (ids.clone(), margin.clone(), n.clone(), com.clone())
    drafts.copy_(ids.view(B, K + 1)[:, :K])  # all drafts agree -> everything accepted
    step()
    torch.cuda.synchronize()
    ref = (ids.clone(), margin.clone(), n.clone(), com.clone())
    assert int(n[0]) == K
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        step()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    log("[graph] capture")
    with torch.cuda.graph(g):
        step()
    for i in range(4):
        ids.fill_(-1); margin.zero_(); n.fill_(-1); com.fill_(-2)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for u, v in zip((ids, margin, n, com), ref):
            assert torch.equal(u, v), f"replay {i} differs"
        c.step(x, B, K, ids, margin)  # eager work between replays
        torch.cuda.synchronize()
