"""GPU grading of the greedy choice, the acceptance and the routing plan against the oracle.

The LM head is graded teacher-forced: the library's final norm, LM head and argmax run on
the oracle's own residual stream after the last block (moe_verify_debug_head), so every
position whose oracle top-1/top-2 margin exceeds the gate is compared, whatever the
routing on the way did. Acceptance of sequence b is graded when the oracle's positions
0..n_b are all decisive (n_b = the oracle's accepted length): then the GPU must accept the
same drafts and commit the same tokens ("jina-ocr-v1" model page, summary paragraph: the
greedy check keeps the output identical to plain greedy decoding).

Every case prints its name and shape before touching the GPU.
"""
import numpy as np
import pytest
import torch

import oracle as O
from lossless_speculative_verification_amd import binding as bnd
from lossless_speculative_verification_amd import workload as W

from gpu_cases import DEV, GATE, TOL, context, host_weights, log, oracle_step, row_rel_err, run_debug_layer

pytestmark = pytest.mark.gpu

WL = W.WORKLOADS


def _head(wl, x, c=None):
    """Teacher-forced final norm + LM head + argmax on residual rows x [T][H]."""
    T = x.shape[0]
    c = c or context(wl, max(T, wl.positions))
    xd = torch.from_numpy(np.ascontiguousarray(x, np.float32)).to(DEV)
    ids = torch.full((T,), -7, dtype=torch.int32, device=DEV)
    margin = torch.empty(T, dtype=torch.float32, device=DEV)
    log(f"[debug_head] {wl.name} T={T}")
    c.debug_head(xd, T, ids, margin)
    torch.cuda.synchronize()
    return ids.cpu().numpy(), margin.cpu().numpy()


def _grade_accept(wl, ref_ids, ref_margin, gpu_ids, drafts):
    """Acceptance on the GPU from the GPU's ids vs the oracle's from its own ids; graded
    on sequences whose oracle positions 0..n_b are decisive. Returns the graded count."""
    B, K = wl.batch, wl.drafts
    n_ref, c_ref = O.accept(drafts, ref_ids, B, K)
    n = torch.empty(B, dtype=torch.int32, device=DEV)
    c = torch.empty(B, K + 1, dtype=torch.int32, device=DEV)
    bnd.accept_greedy(torch.from_numpy(drafts).to(DEV), torch.from_numpy(gpu_ids.astype(np.int32)).to(DEV), B, K, n,
                      c)
    torch.cuda.synchronize()
    dec = (ref_margin > GATE).reshape(B, K + 1)
    graded = np.array([dec[b, : n_ref[b] + 1].all() for b in range(B)])
    np.testing.assert_array_equal(n.cpu().numpy()[graded], n_ref[graded])
    np.testing.assert_array_equal(c.cpu().numpy()[graded], c_ref[graded])
    return int(graded.sum()), n_ref


def _check_head(wl, ref, ids, margin):
    dec = ref["margin"] > GATE
    np.testing.assert_array_equal(ids[dec], ref["ids"][dec])
    assert np.all((ids >= 0) & (ids < wl.vocab))
    dm = np.abs(margin[dec] - ref["margin"][dec]).max()
    assert dm < (1e-4 if wl.wdtype == "f32" else 2e-2), dm
    return dec


# ----------------------------------------------------------------------------- teacher-forced head


@pytest.mark.parametrize("name,min_pos,min_seq", [
    ("decode_b32_k3", 115, 26),
    ("decode_b32_k1", 58, 27),
    ("skewed_b128_k3", 460, 95),
    ("skewed70_b128_k3", 460, 95),
])
def test_head_teacher_forced_batched(name, min_pos, min_seq):
    """Batched configs: the greedy ids of every decisive position (all 128 / 64 / 512 rows,
    the 512-position pass through four 128-row blocks of the LM head) and the acceptance of
    every graded sequence."""
    wl = WL[name]
    ref = oracle_step(wl)
    ids, margin = _head(wl, ref["hidden_out"])
    dec = _check_head(wl, ref, ids, margin)
    graded, n_ref = _grade_accept(wl, ref["ids"], ref["margin"], ids, W.make_drafts(wl, ref["ids"]))
    log(f"  {name}: ids exact on {dec.sum()}/{len(dec)} decisive positions; acceptance exact on {graded}/{wl.batch} "
        f"graded sequences (mean accepted {n_ref.mean():.3f})")
    assert dec.sum() >= min_pos and graded >= min_seq


@pytest.mark.parametrize("name,draws,min_seq", [("tiny_fp32", 24, 12), ("layer1_bf16", 16, 8)])
def test_head_teacher_forced_single_sequence(name, draws, min_seq):
    """B = 1 configs (one sequence of K = 3 drafts per pass): the same weights over several
    seeded hidden-state and draft draws, each graded like the batched passes."""
    wl = WL[name]
    w = host_weights(wl)
    graded = positions = 0
    for d in range(draws):
        wd = wl.with_(seed=wl.seed + 7919 * (d + 1))  # hidden states and drafts only; weights stay wl's
        x = W.make_hidden(wd)
        ref = O.verify_step(wl, w, x)
        ids, margin = _head(wl, ref["hidden_out"])
        positions += int(_check_head(wl, ref, ids, margin).sum())
        graded += _grade_accept(wl, ref["ids"], ref["margin"], ids, W.make_drafts(wd, ref["ids"]))[0]
    log(f"  {name}: {positions}/{4 * draws} decisive positions exact; {graded}/{draws} sequences graded")
    assert graded >= min_seq


def test_head_matches_step_on_its_own_hidden_state():
    """The hook computes what the pass computes: fed the pass's own hidden_out it returns the
    pass's ids and margins bit for bit."""
    wl = WL["decode_b32_k3"]
    c = context(wl)
    x = torch.from_numpy(W.make_hidden(wl)).to(DEV)
    T = wl.positions
    ids = torch.empty(T, dtype=torch.int32, device=DEV)
    margin = torch.empty(T, dtype=torch.float32, device=DEV)
    hout = torch.empty_like(x)
    log("[step] decode_b32_k3 for the head hook")
    c.step(x, wl.batch, wl.drafts, ids, margin, hout)
    torch.cuda.synchronize()
    ids2, margin2 = _head(wl, hout.cpu().numpy(), c)
    np.testing.assert_array_equal(ids2, ids.cpu().numpy())
    np.testing.assert_array_equal(margin2, margin.cpu().numpy())


# ----------------------------------------------------------------------------- ties


def _tie_model(V, T):
    """One small MoE block (its output does not matter here) and a full-width LM head."""
    wl = WL["layer1_bf16"].with_(name=f"tie_v{V}", n_routed=8, top_k=2, n_shared=1, inter=256, vocab=V, batch=T,
                                 drafts=0)
    return wl


# 20,010: a last column pair with 10 real columns; 448 and 512 positions: the LM head runs
# on the tiled GEMM (256-row items of 256-column tiles; the second item of 448 is 3/4 full)
# instead of the streaming kernel
@pytest.mark.parametrize("V,T", [(129280, 136), (20010, 136), (129280, 448), (20010, 512)])
def test_lm_head_constructed_ties(V, T):
    """Identical LM-head rows j1 < j2 (< j3) give bitwise equal logits: the argmax must be
    the lowest index and the margin exactly 0. Pairs sit in one lane, in one wavefront's
    two column pairs, in two wavefronts of a workgroup, in different workgroups (column
    tiles), across the 512-column boundary, at the padded last column pair, and in the
    second row block of positions."""
    wl = _tie_model(V, T)
    w = W.make_weights(wl)
    x = W.make_hidden(wl)
    a = O.final_norm(wl, x)  # the normalised rows the LM head sees
    lm = w.lm_head
    last = V - 1
    ties = [(100, 101), (200, 232), (300, 480), (1000, V // 2), (5, last), (last - 2, last - 1), (7000, 8000, 9000),
            (64, 65, 96), (511, 512), (3, 4000)]
    assert len({j for js in ties for j in js}) == sum(len(js) for js in ties)  # no row planted twice
    owners = list(range(8)) + [128, T - 1]
    planted = {}
    for t, js in zip(owners, ties):
        row = O.round_bf16(0.05 * np.sign(a[t]))  # logit 0.05 * sum |a| (about 51) for position t
        bits = torch.from_numpy(row.astype(np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
        for j in js:
            lm[j] = bits
        planted[t] = js
    dw = bnd.upload_weights(w, DEV)
    c = bnd.MoeVerify(wl, dw, T)
    del dw
    ids, margin = _head(wl, x, c)
    for t, js in planted.items():
        assert ids[t] == js[0], (t, js, ids[t])
        assert margin[t] == 0.0, (t, margin[t])
    # the other positions against the oracle (same modified head)
    ref_ids, ref_margin, _ = O.lm_head_argmax(a, lm, "bf16")
    rest = np.array([t not in planted for t in range(T)])
    assert np.all(ref_ids[list(planted)] == [js[0] for js in planted.values()])
    dec = rest & (ref_margin > GATE)
    np.testing.assert_array_equal(ids[dec], ref_ids[dec])
    log(f"  {len(planted)} planted ties resolved to the lowest index; {dec.sum()} other positions exact")
    c.close()


@pytest.mark.parametrize("T", [128, 4100])
def test_router_constructed_ties(T):
    """Identical router rows (experts 3 and 40, in different router wavefronts; 10 and 11,
    neighbouring lanes) give equal logits: the lower index always takes the earlier slot,
    and the higher one is never selected without its twin. T = 4100 takes the large-pass
    norm/router kernel."""
    wl = WL["layer1_bf16"].with_(name="router_tie", hidden=512, inter=256, vocab=0, batch=T, drafts=0)
    w = W.make_weights(wl)
    w.router[0, 40] = w.router[0, 3]
    w.router[0, 11] = w.router[0, 10]
    x = W.make_hidden(wl)
    dw = bnd.upload_weights(w, DEV)
    c = bnd.MoeVerify(wl, dw, T)
    del dw
    xd = torch.from_numpy(x).to(DEV)
    m = torch.empty_like(xd)
    tid = torch.empty(T, wl.top_k, dtype=torch.int32, device=DEV)
    tw = torch.empty(T, wl.top_k, dtype=torch.float32, device=DEV)
    log(f"[debug_layer] router ties T={T}")
    c.debug_layer(0, xd, T, m, tid, tw)
    torch.cuda.synchronize()
    tid, tw = tid.cpu().numpy(), tw.cpu().numpy()
    both = 0
    for lo, hi in ((3, 40), (10, 11)):
        has_lo, has_hi = (tid == lo).any(axis=1), (tid == hi).any(axis=1)
        assert not np.any(has_hi & ~has_lo), f"expert {hi} selected without its lower twin {lo}"
        for t in np.nonzero(has_lo & has_hi)[0]:
            i, j = int(np.nonzero(tid[t] == lo)[0][0]), int(np.nonzero(tid[t] == hi)[0][0])
            assert j == i + 1 and tw[t, i] == tw[t, j], (t, tid[t], tw[t])
            both += 1
    ref = O.moe_layer(wl, w, 0, x)
    np.testing.assert_array_equal(tid[ref["gap"] > GATE], ref["ids"][ref["gap"] > GATE])
    log(f"  {both} rows hold both twins, lower index first with equal gates")
    assert both > 0
    c.close()


# ----------------------------------------------------------------------------- routing plan and counts


def _plan(c, wl, T):
    rs = torch.full((T * wl.top_k,), -1, dtype=torch.int32, device=DEV)
    cnt = torch.full((wl.n_routed,), -1, dtype=torch.int32, device=DEV)
    c.debug_plan(rs, cnt)
    torch.cuda.synchronize()
    return rs.cpu().numpy(), cnt.cpu().numpy()


SMALL_BF16 = WL["layer1_bf16"].with_(name="small_bf16", hidden=384, inter=256, n_routed=16, top_k=4, n_shared=1,
                                     vocab=0, n_layers=2, drafts=0)


@pytest.mark.parametrize("name,T", [("decode_b32_k3", 128), ("skewed_b128_k3", 512), ("small", 300),
                                    ("small", 5000)])
def test_routing_plan_is_a_stable_sort_by_expert(name, T):
    """The plan's expert-major row order is the stable sort of the slots t*k + j by their
    expert, and its counts are the histogram of the routed ids (one path each: the plan
    built inside the streaming gate/up GEMM at 128 positions, the one-workgroup plan at 300
    and 512, the chunked plan at 5,000); the ids themselves match the oracle's on decisive
    rows."""
    wl = SMALL_BF16.with_(batch=T) if name == "small" else WL[name]
    x = W.make_hidden(wl, T)
    m, tid, tw = run_debug_layer(wl, 0, x)
    c = context(wl, max(T, wl.positions))
    row_slot, counts = _plan(c, wl, T)
    flat = tid.reshape(-1).astype(np.int64)
    np.testing.assert_array_equal(counts, np.bincount(flat, minlength=wl.n_routed))
    np.testing.assert_array_equal(row_slot, np.argsort(flat, kind="stable"))
    ref = O.moe_layer(wl, host_weights(wl), 0, x)
    dec = ref["gap"] > GATE
    np.testing.assert_array_equal(tid[dec], ref["ids"][dec])
    log(f"  plan of {T * wl.top_k} slots exact; {int((counts > 0).sum())} experts touched; "
        f"{dec.sum()}/{T} rows decisive")


@pytest.mark.parametrize("name", ["decode_b32_k3", "skewed_b128_k3"])
def test_expert_counts_match_oracle(name):
    """Per-block routed-slot counts of a full pass (the bench's byte count comes from them)
    against the oracle's routing: equal up to the rows whose routing the oracle does not
    decide, each of which can move at most 2k counts."""
    from gpu_cases import run_step

    wl = WL[name]
    ref = oracle_step(wl)
    run_step(wl)
    counts = context(wl).expert_counts()
    undecided = np.zeros(wl.positions, bool)
    worst = 0
    for l, lay in enumerate(ref["layers"]):
        undecided |= ~(lay["gap"] > GATE)  # a row off the oracle's path stays off it
        expect = np.bincount(lay["ids"].reshape(-1), minlength=wl.n_routed)
        diff = int(np.abs(counts[l] - expect).sum())
        assert diff <= 2 * wl.top_k * int(undecided.sum()), (l, diff, int(undecided.sum()))
        assert counts[l].sum() == wl.positions * wl.top_k
        worst = max(worst, diff)
    log(f"  {name}: counts within {worst} of the oracle's ({int(undecided.sum())} rows undecided somewhere)")


# ----------------------------------------------------------------------------- skewed blocks, every row


@pytest.mark.parametrize("name", ["skewed_b128_k3", "skewed70_b128_k3"])
@pytest.mark.parametrize("layer", [0, 11])
def test_skewed_debug_layer_all_rows(name, layer):
    """One block of the skewed configs (512 positions, the tiled expert GEMM with hot
    experts of several 256-row items) teacher-forced on every row."""
    wl = WL[name]
    x = W.make_hidden(wl)
    ref = O.moe_layer(wl, host_weights(wl), layer, x)
    m, tid, tw = run_debug_layer(wl, layer, x)
    dec = ref["gap"] > GATE
    np.testing.assert_array_equal(tid[dec], ref["ids"][dec])
    assert np.abs(tw[dec] - ref["gates"][dec]).max() < 1e-3
    err = row_rel_err(m[dec], ref["m"][dec])
    hot = float(np.isin(ref["ids"], np.arange(wl.n_biased)).mean())
    log(f"  {name} layer {layer}: decisive {dec.sum()}/{wl.positions}, m rel err {err:.2e}, hot share {hot:.3f}")
    assert err <= TOL["bf16"] and dec.sum() >= 0.8 * wl.positions


# ----------------------------------------------------------------------------- tiled paths at their edges


@pytest.mark.parametrize("T,bias", [(300, 3.0), (512, 3.0)])
def test_half_height_down_tiles(T, bias):
    """A small skewed pass whose down GEMM runs every 256-row item as two 128-row halves
    (the doubled tiles and the streaming items fit one round of compute units): hot experts
    with a partial second half (300 positions: about 224 rows each) or an empty one (512:
    a 127-row second item), shared experts' 44-row item; one block on every row."""
    wl = WL["skewed_b128_k3"].with_(name=f"half_down_t{T}", n_layers=1, vocab=0, batch=T, drafts=0, bias_value=bias)
    x = W.make_hidden(wl)
    ref = O.moe_layer(wl, host_weights(wl), 0, x)
    counts = np.bincount(ref["ids"].ravel(), minlength=wl.n_routed)
    hot = counts >= 64  # the split plan's tile experts
    n_items = int(np.ceil(counts[hot] / 256).sum()) + wl.n_shared * -(-T // 256)
    units = int(np.ceil(counts[~hot] / 32).sum()) * (wl.hidden // 32)
    nt = -(-(wl.hidden // 32) // 8)
    n_cu = torch.cuda.get_device_properties(0).multi_processor_count
    log(f"  items {n_items}, down tiles {n_items * nt} x 2 + {units} streaming units; hot rows {sorted(counts[hot])}")
    assert 2 * n_items * nt + -(-units // 8) <= n_cu  # the half-height mode is taken
    m, tid, tw = run_debug_layer(wl, 0, x)
    dec = ref["gap"] > GATE
    np.testing.assert_array_equal(tid[dec], ref["ids"][dec])
    assert np.abs(tw[dec] - ref["gates"][dec]).max() < 1e-3
    err = row_rel_err(m[dec], ref["m"][dec])
    log(f"  decisive {dec.sum()}/{wl.positions}, m rel err {err:.2e}")
    assert err <= TOL["bf16"] and dec.sum() >= 0.8 * wl.positions


def test_split_plan_with_every_workgroup_tiled():
    """2,048 positions with 8 hot experts (bias +1.6): the tiles (hot and shared experts)
    exceed one round of compute units, so every workgroup runs streaming items of the cold
    experts (fewer than 64 rows each) after its tiles; one block on every row."""
    wl = WL["skewed70_b128_k3"].with_(name="split_full_t2048", n_layers=1, vocab=0, batch=2048, drafts=0,
                                      bias_value=1.6)
    x = W.make_hidden(wl)
    ref = O.moe_layer(wl, host_weights(wl), 0, x)
    counts = np.bincount(ref["ids"].ravel(), minlength=wl.n_routed)
    cold = int((counts[wl.n_biased:] < 64).sum())
    log(f"  cold experts (< 64 rows): {cold} of {wl.n_routed - wl.n_biased}; hot rows {counts[:wl.n_biased].min()}+")
    assert cold >= 40 and counts[: wl.n_biased].min() > 512  # both lists in use, tiles beyond one round
    m, tid, tw = run_debug_layer(wl, 0, x)
    dec = ref["gap"] > GATE
    np.testing.assert_array_equal(tid[dec], ref["ids"][dec])
    assert np.abs(tw[dec] - ref["gates"][dec]).max() < 1e-3
    err = row_rel_err(m[dec], ref["m"][dec])
    log(f"  decisive {dec.sum()}/{wl.positions}, m rel err {err:.2e}")
    assert err <= TOL["bf16"] and dec.sum() >= 0.8 * wl.positions


@pytest.mark.parametrize("T", [256, 384, 512, 640, 700])
def test_tiled_lm_head_small_model(T):
    """The tiled LM head with the shortest contraction it takes (hidden 256: eight steps per
    tile) and a vocabulary of 1,000 (four column tiles, the last one partial), against the
    oracle's full-logit argmax; 700 rows: a third item three quarters full; 640 rows: a half
    full one (tiled); 384 rows: a half-full second item (the streaming head runs)."""
    wl = WL["layer1_bf16"].with_(name=f"lm_small_t{T}", hidden=256, inter=256, n_routed=8, top_k=2, n_shared=1,
                                 vocab=1000, n_layers=1, batch=T, drafts=0)
    w = W.make_weights(wl)
    x = W.make_hidden(wl)
    a = O.final_norm(wl, x)
    ref_ids, ref_margin, _ = O.lm_head_argmax(a, w.lm_head, "bf16")
    dw = bnd.upload_weights(w, DEV)
    c = bnd.MoeVerify(wl, dw, T)
    del dw
    ids, margin = _head(wl, x, c)
    dec = ref_margin > GATE
    np.testing.assert_array_equal(ids[dec], ref_ids[dec])
    assert np.all((ids >= 0) & (ids < wl.vocab))
    assert np.abs(margin[dec] - ref_margin[dec]).max() < 2e-2
    log(f"  decisive {dec.sum()}/{T} exact")
    assert dec.sum() >= 0.8 * T
    c.close()
