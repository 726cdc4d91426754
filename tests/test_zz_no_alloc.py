"""GPU test of moe_verify_step_static, the verify pass whose per-pass buffers live in the
library's static device array: through the C ABI it must reproduce moe_verify_step bit for
bit, on two calls in a row (the second with fewer positions, so stale contents of the
array from the first must not leak into it), and refuse a pass too large for the array.
"""
import numpy as np
import pytest
import torch

from lossless_speculative_verification_amd import binding as bnd
from lossless_speculative_verification_amd import workload as W

from gpu_cases import DEV, context, log

pytestmark = pytest.mark.gpu


def _pass(c, wl, x, B, K, static):
    T = B * (K + 1)
    ids = torch.full((T,), -7, dtype=torch.int32, device=DEV)
    margin = torch.full((T,), -7.0, dtype=torch.float32, device=DEV)
    hout = torch.full((T, wl.hidden), -7.0, dtype=torch.float32, device=DEV)
    log(f"[{'static' if static else 'step'}] {wl.name} B={B} K={K}")
    (c.step_static if static else c.step)(x, B, K, ids, margin, hout)
    torch.cuda.synchronize()
    return ids.cpu().numpy(), margin.cpu().numpy(), hout.cpu().numpy()


# skewed_b128_k3: 512 positions (tiled expert GEMM with the split plan, tiled LM head), then
# 128 (streaming kernels) on the same array
@pytest.mark.parametrize("name", ["decode_b32_k3", "layer1_bf16", "skewed_b128_k3"])
def test_static_step_equals_step_on_two_calls(name):
    wl = W.WORKLOADS[name]
    c = context(wl)
    x = torch.from_numpy(W.make_hidden(wl)).to(DEV)
    B, K = wl.batch, wl.drafts
    small_B = max(1, B // 4)
    for b in (B, small_B):  # a full pass, then a smaller one on the same array
        xs = x[: b * (K + 1)].contiguous()
        ref = _pass(c, wl, xs, b, K, static=False)
        got = _pass(c, wl, xs, b, K, static=True)
        for u, v in zip(got, ref):
            np.testing.assert_array_equal(u, v)
        assert np.all((got[0] >= 0) & (got[0] < wl.vocab))


def test_static_step_prefill_sized_without_lm_head():
    """Hidden states only (no LM head), through the tiled expert GEMM (256+ positions)."""
    wl = W.WORKLOADS["layer1_bf16"].with_(name="static_small", hidden=384, inter=256, n_routed=16, top_k=4,
                                          n_shared=1, vocab=0, n_layers=2, batch=600, drafts=0)
    c = context(wl)
    x = torch.from_numpy(W.make_hidden(wl)).to(DEV)
    for T in (600, 300):
        xs = x[:T].contiguous()
        ref = torch.empty_like(xs)
        got = torch.full_like(xs, -7.0)
        log(f"[step/static] {wl.name} T={T}")
        c.step(xs, T, 0, None, None, ref)
        c.step_static(xs, T, 0, None, None, got)
        torch.cuda.synchronize()
        assert torch.equal(got, ref)


def test_static_step_rejects_a_pass_larger_than_the_array():
    wl = W.WORKLOADS["layer1_bf16"].with_(name="static_big", hidden=384, inter=256, n_routed=16, top_k=4,
                                          n_shared=1, vocab=0, n_layers=1, batch=5000, drafts=0)
    c = context(wl)
    x = torch.zeros(5000, wl.hidden, dtype=torch.float32, device=DEV)
    out = torch.empty_like(x)
    log("[static] oversize pass")
    with pytest.raises(bnd.MoeVerifyError) as ei:
        c.step_static(x, 5000, 0, None, None, out)
    assert ei.value.code == bnd.MOE_EUNSUPPORTED
    assert "static scratch" in bnd.last_error()
