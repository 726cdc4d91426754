"""CPU tests of the measurement tooling: rocprofv3 trace and counter summaries.

The bench's roofline `traffic` and the committed profile summaries come from these
functions, so their arithmetic is checked on small synthetic inputs of the same format.
"""
import csv
import os
import sqlite3

import pytest

from lossless_speculative_verification_amd import profiling as P


def _trace_db(path, launches):
    """A minimal stand-in for the rocpd `kernels` view: name, start, end (ns), grid_x."""
    db = sqlite3.connect(path)
    db.execute("create table kernels (name text, start integer, end integer, grid_x integer, "
               "vgpr_count integer, accum_vgpr_count integer, lds_size integer)")
    db.executemany("insert into kernels values (?, ?, ?, ?, 0, 0, 0)", launches)
    db.commit()
    db.close()


def _steps(t0, n, grid, dur_ns):
    """n verify steps of three kernels each, the first with the given grid, back to back."""
    out, t = [], t0
    for _ in range(n):
        for name, g in (("mv::k_norm(int)", grid), ("mv::k_gemm(int)", 4096), ("mv::k_accept(int)", 256)):
            out.append((name, t, t + dur_ns[name], g))
            t += dur_ns[name]
    return out


def test_step_breakdown_groups_pass_shapes(tmp_path):
    # steps of two shapes interleaved in time: each gets its own table and span
    d1 = {"mv::k_norm(int)": 8000, "mv::k_gemm(int)": 50000, "mv::k_accept(int)": 4000}
    d2 = {"mv::k_norm(int)": 6000, "mv::k_gemm(int)": 30000, "mv::k_accept(int)": 4000}
    rows = _steps(0, 5, 65536, d1) + _steps(10**9, 4, 32768, d2)
    db = str(tmp_path / "t.db")
    _trace_db(db, rows)
    out = P.step_breakdown(db)
    blocks = [b for b in out.split("\n\n") if "steps of" in b]
    assert len(blocks) == 2
    # a step runs from one acceptance to the next: the first run's first step has none
    # before it (4 complete steps), the second run's first one follows the first run's last
    assert blocks[0].startswith("4 steps of 3 kernels, first kernel grid 65536 threads")
    assert "step span median 62.0 us" in blocks[0]
    assert "| `k_gemm` | 1 | 50.00 | 50.0 |" in out
    assert "4 steps of 3 kernels, first kernel grid 32768 threads" in out
    assert "step span median 40.0 us" in out


def test_step_breakdown_without_steps(tmp_path):
    db = str(tmp_path / "t.db")
    _trace_db(db, [("mv::k_norm(int)", 0, 10, 64)])
    assert P.step_breakdown(db) == "(no complete steps in the trace)"


def _counter_csv(path, rows):
    os.makedirs(os.path.dirname(path), exist_ok=True)
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"])
        w.writeheader()
        for r in rows:
            w.writerow(r)


def test_counter_medians_and_copy_scale(tmp_path):
    d = tmp_path / "pmc" / "host"
    _counter_csv(str(d / "run_counter_collection.csv"), [
        {"Dispatch_Id": i, "Kernel_Name": "void mv::k_x<unsigned short>(int)", "Counter_Name": "FETCH_SIZE",
         "Counter_Value": v} for i, v in enumerate([10.0, 30.0, 20.0])])
    med = P.counter_medians(str(tmp_path / "pmc"))
    assert med == {"k_x<bf16>": 20.0}
    # a copy of 4096 bytes that reads 2 counter units: 2048 bytes per unit
    c = tmp_path / "copy"
    _counter_csv(str(c / "run_counter_collection.csv"), [
        {"Dispatch_Id": 0, "Kernel_Name": "copy", "Counter_Name": "FETCH_SIZE", "Counter_Value": 2.0}])
    assert P.copy_scale(str(c), 4096) == pytest.approx(2048.0)


def test_read_traffic_requires_current_sources(tmp_path):
    sha = P.source_sha()
    f = tmp_path / "traffic_w.md"
    f.write_text("\n".join([
        "```",
        f"traffic_bytes_per_launch k_old<0> 100 fetch 60 write 40 sha256 {'0' * 64}",
        f"traffic_bytes_per_launch k_new<0> 300 fetch 200 write 100 sha256 {sha}",
        "```"]))
    assert P.read_traffic(str(f), "k_old") is None  # counters of another build
    rec = P.read_traffic(str(f), "k_new")
    assert rec == {"kernel": "k_new<0>", "bytes": 300, "fetch": 200, "write": 100}
    assert P.read_traffic(str(tmp_path / "missing.md"), "k_new") is None


def test_committed_traffic_records_parse():
    # every committed traffic summary carries machine-readable records of its kernels
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    paths = [os.path.join(root, "profiles", n) for n in os.listdir(os.path.join(root, "profiles"))
             if n.startswith("traffic_") and n.endswith(".md")]
    assert paths
    for p in paths:
        with open(p) as fh:
            recs = [P.TRAFFIC_RE.match(line.strip()) for line in fh]
        recs = [m for m in recs if m]
        assert recs, p
        for m in recs:
            assert int(m.group(2)) == int(m.group(3)) + int(m.group(4))


def test_source_hash_ignores_comments_only():
    # comments and layout leave the hashed code unchanged; a code change does not
    a = "int f(int x) {  // doubles\n  return 2 * x; /* no overflow check */\n}\n"
    b = "/* header */\nint f(int x) {\n\n    return 2 * x;\n}   // end\n"
    c = "int f(int x) {\n  return 3 * x;\n}\n"
    assert P.code_text(a) == P.code_text(b)
    assert P.code_text(a) != P.code_text(c)
    # comment markers inside string and character literals are code
    s = 'asm volatile("s_nop 0 // x" ::); char q = \'/\';\n'
    assert P.code_text(s) == s.strip()


def test_step_breakdown_ends_passes_without_acceptance_at_the_final_norm(tmp_path):
    # no acceptance kernel (no LM head): a step ends with the norm kernel without router
    out, t = [], 0
    for _ in range(5):
        for name, dur in (("mv::k_norm_route_split<unsigned short, true, 1, 2, 40>(int)", 9000),
                          ("mv::k_moe_tiled<0>(int)", 50000),
                          ("mv::k_norm_route_split<unsigned short, false, 1, 2, 40>(int)", 5000)):
            out.append((name, t, t + dur, 512))
            t += dur
    db = str(tmp_path / "t.db")
    _trace_db(db, out)
    res = P.step_breakdown(db)
    assert res.startswith("4 steps of 3 kernels, first kernel grid 512 threads; step span median 64.0 us "
                          "(first kernel start to final norm end)")
    assert "| `k_moe_tiled<0>` | 1 | 50.00 | 50.0 |" in res
