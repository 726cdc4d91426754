"""Throughput of the greedy speculative-verification step on one MI355X.

A step = one verifier pass (moe_verify_step over B*(K+1) positions through all MoE
blocks and the LM head) + greedy acceptance (accept_greedy), on seeded synthetic
inputs already resident in HBM. The metric counts verified tokens: the tokens a pass
commits, sum_b (accepted_b + 1).

Default workload: 12 MoE blocks + LM head at hidden 1280, 64 routed top-6 + 2 shared
experts, intermediate 896, vocabulary 129,280, bf16 weights; B = 32 sequences, K = 3
drafts (128 positions); drafts agree with the verifier with probability 0.576.

Prints one JSON line. Run: python bench.py [--steps K] [--warmup W] [--workload NAME]
"""
import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E peak, GB/s
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 MFMA peak
TILED_MIN_POSITIONS = 256       # the library's switch to the tiled expert GEMM (bf16)
SELF_PLAN_MAX_SLOTS = 4096      # the library's limit for the plan built inside the streaming gate/up GEMM

METRIC = "verified tokens/sec per verify step (B=32,K=3,12 layers); % HBM roofline"


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def algorithmic(wl, counts):
    """Algorithmic HBM bytes and flops of one step, from the step's actual routing.

    Bytes: per block, the weights of every routed expert that received a slot plus the
    shared experts (3*H*I elements each) and the router (E*H); the LM head (V*H); the
    hidden states in (T*H fp32) and the argmax out (T*4). Intermediate buffers are not
    counted. Flops: 2 per multiply-add of the router, the experts' T*(k+S) rows and the
    LM head; the gate/up launch alone does T*(k+S) rows x 2 x (2I x H).
    """
    w = 2 if wl.wdtype == "bf16" else 4
    H, I, E, S, k, V, T = wl.hidden, wl.inter, wl.n_routed, wl.n_shared, wl.top_k, wl.vocab, wl.positions
    touched = (counts > 0).sum(axis=1)  # per block
    expert_bytes = [(int(n) + S) * 3 * H * I * w for n in touched]
    total = sum(expert_bytes) + wl.n_layers * E * H * w + V * H * w + T * H * 4 + T * 4
    up_bytes = [(int(n) + S) * 2 * H * I * w for n in touched]
    flops = wl.n_layers * (T * (k + S) * 6 * H * I + 2 * T * E * H) + 2 * T * V * H
    return {"step_bytes": total, "up_bytes_per_launch": float(np.mean(up_bytes)),
            "up_flops_per_launch": T * (k + S) * 4 * H * I,
            "down_bytes_per_launch": float(np.mean([(int(n) + S) * H * I * w for n in touched])),
            "lm_bytes": V * H * w, "flops": flops, "touched_per_block": float(np.mean(touched))}


def cpu_baseline(wl, weights, x, drafts_fn, min_seconds=10.0, max_passes=5):
    """The CPU oracle, as it stands, on full verifier passes of the same workload: passes are
    repeated until about min_seconds of CPU work (at most max_passes), and the rate is the
    committed tokens over the total time."""
    import oracle as O

    try:
        from threadpoolctl import threadpool_info
        cores = max([d.get("num_threads", 1) for d in threadpool_info()] or [1])
    except Exception:
        cores = len(os.sched_getaffinity(0))
    committed, passes = 0, 0
    t0 = time.perf_counter()
    while passes < max_passes and (passes == 0 or time.perf_counter() - t0 < min_seconds):
        ref = O.verify_step(wl, weights, x)
        n, _ = O.accept(drafts_fn(ref["ids"]), ref["ids"], wl.batch, wl.drafts)
        committed += int(n.sum()) + wl.batch
        passes += 1
    dt = time.perf_counter() - t0
    return {"value": committed / dt, "unit": "verified tokens/s", "cores": int(cores), "kind": "oracle",
            "sample": f"{passes} full verifier pass(es) of {wl.name} ({wl.positions} positions, {wl.n_layers} blocks "
                      f"+ LM head) and their acceptance, float64 numpy, {dt:.1f} s"}


def _time(fn, steps, warmup):
    import torch

    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(steps):
        fn()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / steps


def sweep(args):
    """Draft length K x batch B on the 12-block decode model (one weight set, one context).

    The pages find that the best draft length depends on launch overhead (eager K=3 vs
    graphs K=1 on an L4 at batch 1, "L4 speculative" paragraph of the model page). Here
    every point is timed both as eager launches and as one replayed HIP graph; the
    number of routed experts a block touches grows with the positions of a pass, which
    sets the weight bytes per pass at small batch.
    """
    import torch

    from lossless_speculative_verification_amd import binding as bnd
    from lossless_speculative_verification_amd import workload as W

    base = W.WORKLOADS["decode_b32_k3"]
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    log("[sweep] generating weights")
    dw = bnd.upload_weights(W.make_weights(base), dev)
    ctx = bnd.MoeVerify(base, dw, 32 * 4)
    del dw
    torch.cuda.empty_cache()
    for B in (1, 4, 32):
        for K in (0, 1, 3):
            wl = base.with_(batch=B, drafts=K)
            T = wl.positions
            x = torch.from_numpy(W.make_hidden(wl)).to(dev)
            ids = torch.empty(T, dtype=torch.int32, device=dev)
            n_acc = torch.zeros(B, dtype=torch.int32, device=dev)
            committed = torch.empty(B, K + 1, dtype=torch.int32, device=dev)
            ctx.step(x, B, K, ids)
            torch.cuda.synchronize()
            counts = ctx.expert_counts()
            drafts = torch.from_numpy(W.make_drafts(wl, ids.cpu().numpy())).to(dev)

            def step():
                ctx.step(x, B, K, ids)
                bnd.accept_greedy(drafts, ids, B, K, n_acc, committed)

            step()
            torch.cuda.synchronize()
            ref = (ids.clone(), n_acc.clone())
            g = torch.cuda.CUDAGraph()
            s = torch.cuda.Stream()
            s.wait_stream(torch.cuda.current_stream())
            with torch.cuda.stream(s):
                step()
            torch.cuda.current_stream().wait_stream(s)
            torch.cuda.synchronize()
            with torch.cuda.graph(g):
                step()
            ids.fill_(-1)
            g.replay()
            torch.cuda.synchronize()
            assert torch.equal(ids, ref[0]) and torch.equal(n_acc, ref[1]), "graph replay differs from eager"
            ms_graph = _time(g.replay, args.steps, args.warmup)
            ms_eager = _time(step, args.steps, args.warmup)
            com = int(n_acc.sum().item()) + B
            acc = algorithmic(wl, counts)
            line = {"sweep": "decode_kxb", "B": B, "K": K, "positions": T, "committed_per_step": com,
                    "ms_graph": round(ms_graph, 4), "ms_eager": round(ms_eager, 4),
                    "tokens_per_s_graph": round(com / (ms_graph * 1e-3), 1),
                    "tokens_per_s_eager": round(com / (ms_eager * 1e-3), 1),
                    "tokens_per_s_per_seq_graph": round(com / B / (ms_graph * 1e-3), 1),
                    "touched_experts_per_block": acc["touched_per_block"],
                    "hbm_frac_graph": round(acc["step_bytes"] / (ms_graph * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}
            print(json.dumps(line), flush=True)
            del g
    ctx.close()


def draft_bench(args):
    """Cost of the draft block and of the closed loop, on the 12-block decode model.

    One draft step streams the block's projection and SwiGLU weights and the LM head;
    with random weights its drafts are meaningless, so only time and bytes are reported.
    The loop step is one verifier pass (B=32, K=3) + acceptance + K=3 draft steps, the
    drafts feeding the next pass, captured in one HIP graph.
    """
    import torch

    from lossless_speculative_verification_amd import binding as bnd
    from lossless_speculative_verification_amd import workload as W

    wl = W.WORKLOADS["decode_b32_k3"]
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    log("[draft] generating weights")
    dw_h = W.make_draft_weights(wl)
    dw = bnd.upload_weights(W.make_weights(wl), dev)
    ctx = bnd.MoeVerify(wl, dw)
    del dw
    ctx.draft_init(bnd.upload_draft_weights(dw_h, dev))
    torch.cuda.empty_cache()
    B, K, T, H = wl.batch, wl.drafts, wl.positions, wl.hidden
    x = torch.from_numpy(W.make_hidden(wl)).to(dev)
    ids = torch.empty(T, dtype=torch.int32, device=dev)
    hout = torch.empty_like(x)
    n_acc = torch.empty(B, dtype=torch.int32, device=dev)
    com = torch.empty(B, K + 1, dtype=torch.int32, device=dev)
    drafts = torch.zeros(B, K, dtype=torch.int32, device=dev)

    def draft():
        ctx.draft_step(hout, n_acc, com, B, K, K, drafts)

    def loop():
        ctx.step(x, B, K, ids, None, hout)
        bnd.accept_greedy(drafts, ids, B, K, n_acc, com)
        draft()

    loop()
    torch.cuda.synchronize()
    graphs = {}
    for name, fn in (("draft", draft), ("loop", loop)):
        g = torch.cuda.CUDAGraph()
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):
            fn()
        torch.cuda.current_stream().wait_stream(s)
        torch.cuda.synchronize()
        with torch.cuda.graph(g):
            fn()
        graphs[name] = g
    ms_draft = _time(graphs["draft"].replay, args.steps, args.warmup)
    ms_loop = _time(graphs["loop"].replay, args.steps, args.warmup)
    w = 2 if wl.wdtype == "bf16" else 4
    per_step = (H * 2 * H + 3 * H * dw_h.inter + wl.vocab * H) * w + B * H * w
    line = {"bench": "draft_block", "workload": wl.name, "B": B, "K": K, "draft_inter": dw_h.inter,
            "ms_draft": round(ms_draft, 4), "draft_bytes": K * per_step,
            "draft_hbm_gbs": round(K * per_step / (ms_draft * 1e-3) / 1e9, 1),
            "draft_hbm_frac": round(K * per_step / (ms_draft * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
            "ms_loop": round(ms_loop, 4), "loop_positions_per_s": round(T / (ms_loop * 1e-3), 1), "mode": "hip_graph"}
    print(json.dumps(line), flush=True)
    ctx.close()


def mixed_bench(args):
    """One page's prefill (1,156 visual-token positions) and a B=32, K=3 verify in one pass
    (one stream of the expert weights for both) against the two passes run one after the
    other, on the 12-block decode model."""
    import torch

    from lossless_speculative_verification_amd import binding as bnd
    from lossless_speculative_verification_amd import workload as W

    wl = W.WORKLOADS["decode_b32_k3"]
    n_pre, B, K = 1156, wl.batch, wl.drafts
    Tv = B * (K + 1)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    log("[mixed] generating weights")
    dw = bnd.upload_weights(W.make_weights(wl), dev)
    ctx = bnd.MoeVerify(wl, dw, n_pre + Tv)
    del dw
    torch.cuda.empty_cache()
    x = torch.from_numpy(W.make_hidden(wl, n_pre + Tv)).to(dev)
    ids = torch.empty(Tv, dtype=torch.int32, device=dev)
    first = torch.empty(1, dtype=torch.int32, device=dev)  # the page's first token

    def mixed():
        ctx.step_mixed(x, n_pre, B, K, ids)

    def separate():
        ctx.step_mixed(x[: n_pre + 1], n_pre, 1, 0, first)  # prefill pass: LM head on its last position
        ctx.step(x[n_pre:], B, K, ids)

    res = {}
    for name, fn in (("mixed", mixed), ("separate", separate)):
        fn()
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):
            fn()
        torch.cuda.current_stream().wait_stream(s)
        torch.cuda.synchronize()
        with torch.cuda.graph(g):
            fn()
        res[name] = _time(g.replay, args.steps, args.warmup)
    line = {"bench": "mixed_pass", "workload": wl.name, "n_prefill": n_pre, "B": B, "K": K,
            "ms_mixed": round(res["mixed"], 4), "ms_separate": round(res["separate"], 4),
            "speedup": round(res["separate"] / res["mixed"], 3),
            "positions_per_s_mixed": round((n_pre + Tv) / (res["mixed"] * 1e-3), 1), "mode": "hip_graph"}
    print(json.dumps(line), flush=True)
    ctx.close()


def expected_committed(wl):
    """Expected tokens a pass commits per sequence when each draft equals the verifier's
    choice with probability p independently: sum_{i=0..K} p^i (the bonus token, then each
    further token needs one more agreeing draft)."""
    return sum(wl.p_match ** i for i in range(wl.drafts + 1))


def timed_pass(ctx, wl, x, args):
    """Time one step (verifier pass + acceptance) of wl on resident inputs x.

    Drafts agree with the verifier's greedy choice with probability p; they are built from
    one untimed pass's argmax (the verifier's own choices, as a drafter would see them).
    The step is captured in a HIP graph (unless --eager) whose replays must reproduce the
    eager result exactly, then timed over args.steps replays after args.warmup.
    """
    import torch

    from lossless_speculative_verification_amd import binding as bnd
    from lossless_speculative_verification_amd import workload as W

    dev = x.device
    T, B, K = wl.positions, wl.batch, wl.drafts
    ids = torch.empty(T, dtype=torch.int32, device=dev)
    margin = torch.empty(T, dtype=torch.float32, device=dev)
    n_acc = torch.zeros(B, dtype=torch.int32, device=dev)
    committed = torch.empty(B, K + 1, dtype=torch.int32, device=dev)
    hidden_out = torch.empty_like(x) if wl.vocab == 0 else None

    ctx.step(x, B, K, ids if wl.vocab else None, margin if wl.vocab else None, hidden_out)
    torch.cuda.synchronize()
    counts = ctx.expert_counts()
    y0 = ids.cpu().numpy() if wl.vocab else np.zeros(T, np.int32)
    drafts = torch.from_numpy(W.make_drafts(wl, y0)).to(dev) if K > 0 else torch.empty(B, 0, dtype=torch.int32,
                                                                                        device=dev)

    def step():
        ctx.step(x, B, K, ids if wl.vocab else None, margin if wl.vocab else None, hidden_out)
        if wl.vocab:
            bnd.accept_greedy(drafts, ids, B, K, n_acc, committed)

    # eager reference outputs, then (default) capture the step in a HIP graph
    step()
    torch.cuda.synchronize()
    out = ids if wl.vocab else hidden_out  # what the pass produces
    ref_out, ref_n = out.clone(), n_acc.clone()
    mode = "eager"
    run = step
    if not args.eager:
        g = torch.cuda.CUDAGraph()
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):
            step()  # warm the capture stream
        torch.cuda.current_stream().wait_stream(s)
        torch.cuda.synchronize()
        with torch.cuda.graph(g):
            step()
        run = g.replay
        mode = "hip_graph"
        for _ in range(3):  # replays must reproduce the eager result exactly
            out.fill_(-1)
            run()
            torch.cuda.synchronize()
            assert torch.equal(out, ref_out) and torch.equal(n_acc, ref_n), "graph replay differs from eager"

    for _ in range(args.warmup):
        run()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    if args.flush_mall:
        # each step timed on its own, after 1 GiB of writes has evicted the weights from the
        # memory-side cache; the timed region holds the step only
        scrub = torch.empty(1 << 28, dtype=torch.float32, device=dev)
        total = 0.0
        for i in range(args.steps):
            scrub.fill_(float(i))
            e0.record()
            run()
            e1.record()
            torch.cuda.synchronize()
            total += e0.elapsed_time(e1)
        ms = total / args.steps
        del scrub
    else:
        e0.record()
        for _ in range(args.steps):
            run()
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / args.steps

    # eager timing for reference (launch overhead visible)
    for _ in range(3):
        step()
    torch.cuda.synchronize()
    e0.record()
    for _ in range(args.steps):
        step()
    e1.record()
    torch.cuda.synchronize()
    ms_eager = e0.elapsed_time(e1) / args.steps
    com = int(n_acc.sum().item()) + B if wl.vocab else 0
    return {"ms": ms, "ms_eager": ms_eager, "counts": counts, "mode": mode, "committed": com, "ids": ids,
            "margin": margin, "hidden_out": hidden_out}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    # about 0.25 s of decode steps: the first ~0.15 s of steps after set-up run 2-3 % slower
    # (graph and eager alike) before the step time settles
    ap.add_argument("--warmup", type=int, default=200)
    ap.add_argument("--workload", default="decode_b32_k3")
    ap.add_argument("--eager", action="store_true", help="time eager launches instead of a HIP graph")
    ap.add_argument("--flush-mall", action="store_true",
                    help="overwrite 1 GiB between timed steps (each step timed alone) so no weight is still in "
                         "the 256 MB memory-side cache when a step starts")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--sweep", action="store_true",
                    help="time the 12-block decode model over K in {0,1,3} x B in {1,4,32}, HIP graph and eager "
                         "(one JSON line per point instead of the bench line)")
    ap.add_argument("--draft", action="store_true",
                    help="time the draft block (K steps after a B=32, K=3 pass of the 12-block model) and the "
                         "closed verify + accept + draft loop (one JSON line instead of the bench line)")
    ap.add_argument("--mixed", action="store_true",
                    help="time a mixed pass (one 1,156-token page prefill + a B=32, K=3 verify) against the two "
                         "passes run separately, 12-block model (one JSON line instead of the bench line)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only copy 256 MiB device to device (scale reference for the HBM byte counters)")
    args = ap.parse_args()
    if args.copy_calibration:
        import torch

        n = 256 << 20
        src = torch.ones(n // 4, dtype=torch.float32, device="cuda:0")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes": n, "launches": 3}))
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}); the verify step is "
              "data-parallel over sequences with no exchange, see the design notes.", file=sys.stderr)
        sys.exit(2)

    if args.sweep:
        sweep(args)
        return
    if args.draft:
        draft_bench(args)
        return
    if args.mixed:
        mixed_bench(args)
        return

    import torch

    from lossless_speculative_verification_amd import binding as bnd
    from lossless_speculative_verification_amd import workload as W

    wl = W.WORKLOADS[args.workload]
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    log(f"[bench] {wl.name}: generating weights")
    t0 = time.perf_counter()
    weights = W.make_weights(wl)
    x_h = W.make_hidden(wl)
    log(f"[bench] generated in {time.perf_counter() - t0:.1f} s; uploading + repacking")
    dw = bnd.upload_weights(weights, dev)
    ctx = bnd.MoeVerify(wl, dw)
    del dw
    torch.cuda.empty_cache()

    x = torch.from_numpy(x_h).to(dev)
    r = timed_pass(ctx, wl, x, args)
    ms, ms_eager, counts, mode = r["ms"], r["ms_eager"], r["counts"], r["mode"]
    T, B, K = wl.positions, wl.batch, wl.drafts
    ids, margin, hidden_out = r["ids"], r["margin"], r["hidden_out"]

    # per-kernel durations from HIP events the library records around each launch
    ctx.profile(True)
    for _ in range(args.steps):
        ctx.step(x, B, K, ids if wl.vocab else None, margin if wl.vocab else None, hidden_out)
        prof = ctx.profile_read()
    ctx.profile(False)

    acc = algorithmic(wl, counts)
    committed_per_step = r["committed"]
    per_kind = {k: {"avg_us": 1000.0 * v[0] / max(v[1], 1), "launches_per_step": v[1] / args.steps}
                for k, v in prof.items()}
    up_us = per_kind["gemm_up"]["avg_us"]
    # The library runs the expert GEMMs on the LDS-tiled kernel for bf16 passes of at
    # least TILED_MIN_POSITIONS positions (matrix-core bound there), else on the streaming
    # kernel (bound by the weight stream).
    tiled = wl.wdtype == "bf16" and T >= TILED_MIN_POSITIONS
    # streaming passes of at most SELF_PLAN_MAX_SLOTS routed slots build the plan inside
    # the gate/up kernel (k_moe_gemm_planned)
    planned = not tiled and T * wl.top_k <= SELF_PLAN_MAX_SLOTS
    dt = "bf16" if wl.wdtype == "bf16" else "float"
    kernel = "k_moe_tiled<0>" if tiled else (f"k_moe_gemm_planned<{dt}" if planned else f"k_moe_gemm<{dt},0")
    # measured HBM bytes per launch of the same kernel (rocprofv3 counters, see profiles/),
    # only while the counters were taken on the current kernel sources
    from lossless_speculative_verification_amd import profiling
    rec = profiling.read_traffic(os.path.join(ROOT, "profiles", f"traffic_{wl.name}.md"), kernel)
    traffic_up = rec["bytes"] if rec else None
    up_gbs = acc["up_bytes_per_launch"] / (up_us * 1e-6) / 1e9
    up_tfs = acc["up_flops_per_launch"] / (up_us * 1e-6) / 1e12
    step_gbs = acc["step_bytes"] / (ms * 1e-3) / 1e9
    if tiled:
        roof = {"bound": "mfma", "kernel": "gate/up expert GEMM + SwiGLU (k_moe_tiled, LDS-tiled MFMA, one launch "
                                           "per block)",
                "achieved": round(up_tfs, 1), "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                "frac": round(up_tfs / MFMA_BF16_PEAK_TFLOPS, 4), "traffic": traffic_up,
                "algorithmic_flops_per_launch": acc["up_flops_per_launch"], "avg_launch_us": round(up_us, 2)}
    else:
        roof = {"bound": "hbm", "kernel": "gate/up expert GEMM + SwiGLU (%s, one launch per block)"
                                          % ("k_moe_gemm_planned" if planned else "k_moe_gemm"),
                "achieved": round(up_gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(up_gbs / HBM_PEAK_GBS, 4), "traffic": traffic_up,
                "algorithmic_bytes_per_launch": round(acc["up_bytes_per_launch"]), "avg_launch_us": round(up_us, 2)}

    cpu = None
    if not args.no_cpu_baseline and wl.n_layers * wl.positions <= 12 * 512:
        log("[bench] timing the CPU oracle on one pass")
        cpu = cpu_baseline(wl, weights, x_h, lambda y: W.make_drafts(wl, y))

    value = committed_per_step / (ms * 1e-3) if wl.vocab else T / (ms * 1e-3)
    out = {
        "metric": METRIC if wl.name == "decode_b32_k3" else f"verified tokens/sec per verify step ({wl.name})",
        "value": round(value, 1),
        "unit": "tokens/s" if wl.vocab else "positions/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": wl.wdtype, "data": "synthetic",
        "config": {"workload": wl.name, "B": B, "K": K, "blocks": wl.n_layers, "hidden": wl.hidden,
                   "routed_experts": wl.n_routed, "top_k": wl.top_k, "shared_experts": wl.n_shared,
                   "inter": wl.inter, "vocab": wl.vocab, "positions": T, "mode": mode,
                   "mall_flushed": bool(args.flush_mall)},
        "roofline": roof,
        "step_roofline": {"bound": "hbm", "achieved": round(step_gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                          "frac": round(step_gbs / HBM_PEAK_GBS, 4), "algorithmic_bytes": acc["step_bytes"],
                          "mfma_frac": round(acc["flops"] / (ms * 1e-3) / 1e12 / MFMA_BF16_PEAK_TFLOPS, 4)},
        "cpu_baseline": cpu,
        "positions_per_s": round(T / (ms * 1e-3), 1),
        "committed_per_step": committed_per_step,
        "eager_ms_per_step": round(ms_eager, 4),
        "kernels_us": {k: round(v["avg_us"], 2) for k, v in per_kind.items()},
        "touched_experts_per_block": acc["touched_per_block"],
    }
    if wl.n_biased > 0:  # share of the routed slots that land on the biased ("hot") experts
        out["hot_slot_frac"] = round(float(counts[:, : wl.n_biased].sum() / max(counts.sum(), 1)), 4)
    if wl.vocab:
        # the sampled value rides on one seeded draft draw; the expectation over draft draws
        # at the same step time is B * sum_{i=0..K} p^i tokens per step
        out["value_expected"] = round(B * expected_committed(wl) / (ms * 1e-3), 1)
        out["committed_per_step_expected"] = round(B * expected_committed(wl), 2)
    if wl.name == "decode_b32_k3" and not args.flush_mall:
        # the K = 1 operating point of the same model and weights (the pages' best K with graphs)
        wl1 = W.WORKLOADS["decode_b32_k1"]
        log("[bench] K = 1 operating point")
        r1 = timed_pass(ctx, wl1, torch.from_numpy(W.make_hidden(wl1)).to(dev), args)
        acc1 = algorithmic(wl1, r1["counts"])
        out["k1"] = {"workload": wl1.name, "B": wl1.batch, "K": wl1.drafts, "positions": wl1.positions,
                     "ms_per_step": round(r1["ms"], 4),
                     "value": round(r1["committed"] / (r1["ms"] * 1e-3), 1),
                     "value_expected": round(wl1.batch * expected_committed(wl1) / (r1["ms"] * 1e-3), 1),
                     "committed_per_step": r1["committed"],
                     "step_hbm_frac": round(acc1["step_bytes"] / (r1["ms"] * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}
    print(json.dumps(out), flush=True)
    ctx.close()


if __name__ == "__main__":
    main()
