"""GPU parity of the mixed pass (moe_verify_step_mixed): prompt-prefill positions and
verify positions through the MoE blocks together, LM head on the verify positions only.

Positions are independent on this path (attention is outside it), so the oracle's
expected values are its plain pass over all rows (hidden states) and over the verify
rows (greedy tokens).
"""
import numpy as np
import pytest
import torch

import oracle as O
from lossless_speculative_verification_amd import binding as bnd
from lossless_speculative_verification_amd import workload as W
from gpu_cases import DEV, GATE, TOL, context, decisive_positions, end_to_end_rel_err, host_weights, log

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("name,n_prefill,B,K", [("tiny_fp32", 37, 4, 3), ("layer1_bf16", 300, 4, 3),
                                                ("layer1_bf16", 41, 2, 1)])
def test_mixed_pass_matches_oracle(name, n_prefill, B, K):
    wl = W.WORKLOADS[name]
    Tv = B * (K + 1)
    T = n_prefill + Tv
    wts = host_weights(wl)
    x = W.make_hidden(wl, T)
    log(f"[mixed] {name} n_prefill={n_prefill} B={B} K={K}")
    c = context(wl, T)
    xd = torch.from_numpy(x).to(DEV)
    ids = torch.full((Tv,), -7, dtype=torch.int32, device=DEV)
    margin = torch.empty(Tv, dtype=torch.float32, device=DEV)
    hout = torch.empty_like(xd)
    c.step_mixed(xd, n_prefill, B, K, ids, margin, hout)
    torch.cuda.synchronize()
    ids, hout = ids.cpu().numpy(), hout.cpu().numpy()
    # every row's hidden state, with the blocks only
    ref_all = O.verify_step(wl.with_(vocab=0), wts, x)
    assert end_to_end_rel_err(hout, ref_all["hidden_out"], x, wl.n_layers) < TOL[wl.wdtype]
    # the verify rows' greedy tokens
    ref = O.verify_step(wl, wts, x[n_prefill:])
    dec = decisive_positions(ref)
    assert dec.sum() >= Tv // 2
    assert np.array_equal(ids[dec], ref["ids"][dec])


def test_mixed_pass_without_prefill_is_the_plain_step():
    wl = W.WORKLOADS["layer1_bf16"]
    c = context(wl, wl.positions)
    x = torch.from_numpy(W.make_hidden(wl)).to(DEV)
    T, B, K = wl.positions, wl.batch, wl.drafts
    a1, a2 = (torch.empty(T, dtype=torch.int32, device=DEV) for _ in range(2))
    m1, m2 = (torch.empty(T, dtype=torch.float32, device=DEV) for _ in range(2))
    c.step(x, B, K, a1, m1)
    c.step_mixed(x, 0, B, K, a2, m2)
    torch.cuda.synchronize()
    assert torch.equal(a1, a2) and torch.equal(m1, m2)


def test_mixed_pass_rejects_oversize():
    wl = W.WORKLOADS["tiny_fp32"]
    c = context(wl)
    P = c.cfg.max_positions
    xd = torch.zeros(P + 8, wl.hidden, device=DEV)
    ids = torch.empty(8, dtype=torch.int32, device=DEV)
    with pytest.raises(bnd.MoeVerifyError) as ei:
        c.step_mixed(xd, P, 2, 3, ids)
    assert ei.value.code == bnd.MOE_EINVAL
    with pytest.raises(bnd.MoeVerifyError) as ei:
        c.step_mixed(xd, -1, 2, 3, ids)
    assert ei.value.code == bnd.MOE_EINVAL


def test_mixed_pass_bench_size_sampled():
    """The bench's mixed pass: one page of 1,156 prefill positions and a B=32, K=3 verify
    through the 12-block model; the oracle follows 48 sampled prefill rows and every verify
    row."""
    wl = W.WORKLOADS["decode_b32_k3"]
    n_pre, B, K = 1156, wl.batch, wl.drafts
    Tv = B * (K + 1)
    wts = host_weights(wl)
    x = W.make_hidden(wl, n_pre + Tv)
    log("[mixed] bench size, sampled rows")
    c = context(wl, n_pre + Tv)
    xd = torch.from_numpy(x).to(DEV)
    ids = torch.empty(Tv, dtype=torch.int32, device=DEV)
    hout = torch.empty_like(xd)
    c.step_mixed(xd, n_pre, B, K, ids, None, hout)
    torch.cuda.synchronize()
    ids, hout = ids.cpu().numpy(), hout.cpu().numpy()
    rng = np.random.default_rng(12)
    # 12 blocks: about a fifth of the positions have every routing gap (and the LM margin)
    # above the gate, so the comparison runs on those rows
    pre = np.array(sorted(rng.choice(n_pre, 48, replace=False).tolist()))
    ref_pre = O.verify_step(wl.with_(vocab=0), wts, x[pre])
    dp = decisive_positions(ref_pre)
    assert dp.sum() >= 2, dp.sum()
    assert end_to_end_rel_err(hout[pre][dp], ref_pre["hidden_out"][dp], x[pre][dp], wl.n_layers) < TOL[wl.wdtype]
    vrows = np.arange(Tv)
    ref = O.verify_step(wl, wts, x[n_pre + vrows])
    dec = decisive_positions(ref)
    assert dec.sum() >= 4, dec.sum()
    assert np.array_equal(ids[dec], ref["ids"][dec])
    assert end_to_end_rel_err(hout[n_pre + vrows][dec], ref["hidden_out"][dec], x[n_pre + vrows][dec],
                              wl.n_layers) < TOL[wl.wdtype]
