"""Summaries of rocprofv3 output for the measurement notes (kernel trace and HBM counters).

    python -m lossless_speculative_verification_amd.profiling trace DB
        per-kernel launch count and duration statistics of a --kernel-trace database
        (rocpd SQLite), steady state of the verify step included;
    python -m lossless_speculative_verification_amd.profiling traffic --workload W \\
            --fetch DIR --write DIR --copy-fetch DIR --copy-write DIR --copy-bytes N --out FILE
        per-launch HBM bytes of every kernel from two --pmc runs (FETCH_SIZE, then
        WRITE_SIZE; rocprofv3 csv output) of the bench, each scaled by what the same
        counter reads for a plain copy of N bytes (--copy-calibration mode of bench.py);
    python -m lossless_speculative_verification_amd.profiling mfma DIR
        per-kernel MFMA-busy percentage and bf16 MFMA flop rate from one --pmc run with
        MfmaUtil and SQ_INSTS_VALU_MFMA_MOPS_BF16 plus --kernel-trace (csv output).

The traffic file records the sha256 of the kernel sources' code (comments aside); bench.py
reports a kernel's traffic only while that hash still matches the sources (counters of an
older build would describe other kernels).
"""
from __future__ import annotations

import argparse
import collections
import csv
import glob
import hashlib
import os
import re
import sqlite3
import statistics
from typing import Dict, Optional

PKG = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG, "csrc")
TRAFFIC_RE = re.compile(r"^traffic_bytes_per_launch\s+(\S+)\s+(\d+)\s+fetch\s+(\d+)\s+write\s+(\d+)\s+sha256\s+(\w+)")


_TOKEN_RE = re.compile(r'("(?:\\.|[^"\\\n])*"|\'(?:\\.|[^\'\\\n])*\')|//[^\n]*|/\*.*?\*/', re.S)


def code_text(src: str) -> str:
    """The source with its comments removed, horizontal whitespace collapsed and blank lines
    dropped: what the compiler sees, so that an edit of comments alone keeps the hash."""
    s = _TOKEN_RE.sub(lambda m: m.group(1) if m.group(1) else " ", src)
    lines = (" ".join(line.split()) for line in s.splitlines())
    return "\n".join(line for line in lines if line)


def source_sha() -> str:
    """sha256 over the code (comments aside) of the HIP sources and headers the library is
    built from."""
    h = hashlib.sha256()
    for p in sorted(glob.glob(os.path.join(CSRC, "*.hip")) + glob.glob(os.path.join(CSRC, "*.h"))):
        with open(p, encoding="utf-8") as f:
            h.update(os.path.basename(p).encode())
            h.update(code_text(f.read()).encode())
    return h.hexdigest()


def short_name(name: str) -> str:
    n = name.split("(")[0].replace("void ", "").replace("mv::", "")
    return n.replace("unsigned short", "bf16")


def trace_table(db_path: str) -> str:
    """Markdown table: kernel, calls, avg/min/max/total microseconds, grid, registers."""
    db = sqlite3.connect(db_path)
    rows = db.execute(
        "select name, count(*), avg(end-start)/1000.0, min(end-start)/1000.0, max(end-start)/1000.0, "
        "sum(end-start)/1000.0, max(grid_x), max(vgpr_count), max(accum_vgpr_count), max(lds_size) "
        "from kernels group by name order by sum(end-start) desc").fetchall()
    out = ["| kernel | calls | avg us | min us | max us | total us | grid (threads) | vgpr/agpr (trace) | lds B |",
           "|---|---|---|---|---|---|---|---|---|"]
    for r in rows:
        out.append(f"| `{short_name(r[0])[:60]}` | {r[1]} | {r[2]:.2f} | {r[3]:.2f} | {r[4]:.2f} | {r[5]:.1f} | "
                   f"{r[6]} | {r[7]}/{r[8]} | {r[9]} |")
    out += ["", "The register column is the value the trace database records, which for these kernels is half "
                "the registers the compiler allocates per lane (e.g. 128 for the 252-register gate/up kernel)."]
    return "\n".join(out)


def step_breakdown(db_path: str, marker: Optional[str] = None) -> str:
    """Per-kernel medians within whole steps, one table per pass shape: steps are grouped
    by their kernel count and the grid of their first kernel (the routing norm's grid
    follows the number of positions). A step ends with the kernel named by marker: by
    default the acceptance kernel, or, in passes without one (no LM head), the final norm
    (the norm kernel without router)."""
    db = sqlite3.connect(db_path)
    rows = db.execute("select name, start, end, grid_x from kernels order by start").fetchall()
    names = [short_name(r[0]) for r in rows]
    if marker is None:
        marker = "k_accept" if any(n.startswith("k_accept") for n in names) else "k_norm_route_split<"
        final = marker != "k_accept"
    else:
        final = False
    acc = [i for i, n in enumerate(names) if n.startswith(marker) and (not final or ", false," in n)]
    steps = [rows[a + 1:b + 1] for a, b in zip(acc[:-1], acc[1:])]
    if not steps:
        return "(no complete steps in the trace)"
    groups = collections.defaultdict(list)
    for s in steps:
        groups[(len(s), s[0][3])].append(s)
    out = []
    for (n, grid), ss in sorted(groups.items(), key=lambda kv: -len(kv[1])):
        if len(ss) < 3:
            continue
        durs = collections.defaultdict(list)
        for s in ss:
            for name, a, b, _ in s:
                durs[short_name(name)].append((b - a) / 1000.0)
        spans = [(s[-1][2] - s[0][1]) / 1000.0 for s in ss]
        out += [f"{len(ss)} steps of {n} kernels, first kernel grid {grid} threads; step span median "
                f"{statistics.median(spans):.1f} us (first kernel start to {'final norm' if final else 'acceptance'} end)", "",
                "| kernel | launches/step | median us | us/step |", "|---|---|---|---|"]
        for k, v in durs.items():
            per = len(v) // len(ss)
            out.append(f"| `{k[:60]}` | {per} | {statistics.median(v):.2f} | {sum(v) / len(ss):.1f} |")
        out.append("")
    return "\n".join(out).rstrip() if out else "(no complete steps in the trace)"


def counter_medians(csv_dir: str) -> Dict[str, float]:
    """Median counter value (as rocprofv3 reports it) per kernel name, from a --pmc csv run."""
    paths = glob.glob(os.path.join(csv_dir, "**", "*counter_collection.csv"), recursive=True)
    if not paths:
        raise FileNotFoundError(f"no *counter_collection.csv under {csv_dir}")
    vals = collections.defaultdict(list)
    for p in paths:
        with open(p) as f:
            for r in csv.DictReader(f):
                vals[short_name(r["Kernel_Name"])].append(float(r["Counter_Value"]))
    return {k: statistics.median(v) for k, v in vals.items()}


def copy_scale(csv_dir: str, copy_bytes: int) -> float:
    """Bytes per counter unit: the copy's true bytes over the largest counter reading."""
    med = counter_medians(csv_dir)
    reading = max(med.values())
    return copy_bytes / reading


def read_traffic(path: str, kernel_prefix: str) -> Optional[dict]:
    """Traffic record of the first kernel starting with kernel_prefix, if the file's source
    hash matches the current sources; else None."""
    if not os.path.exists(path):
        return None
    sha = source_sha()
    with open(path) as f:
        for line in f:
            m = TRAFFIC_RE.match(line.strip().strip("`"))
            if m and m.group(1).startswith(kernel_prefix) and m.group(5) == sha:
                return {"kernel": m.group(1), "bytes": int(m.group(2)), "fetch": int(m.group(3)),
                        "write": int(m.group(4))}
    return None


def _col(row: dict, *names: str) -> str:
    """The first column of a rocprofv3 csv row whose name matches one of names (case and
    underscores ignored)."""
    norm = {k.replace("_", "").lower(): k for k in row}
    for n in names:
        k = norm.get(n.replace("_", "").lower())
        if k is not None:
            return row[k]
    raise KeyError(f"none of {names} in {sorted(row)}")


def mfma_table(csv_dir: str, peak_flops: float = 2.5e15) -> str:
    """Markdown table per kernel from one --pmc run with MfmaUtil and
    SQ_INSTS_VALU_MFMA_MOPS_BF16 plus --kernel-trace (csv output): median MFMA-busy percentage
    (busy cycles of the matrix units over active cycles of all SIMDs), bf16 MFMA flops per
    launch (MOPS x 512), the launch's duration in that run, and the resulting rate against the
    dense bf16 peak."""
    cpaths = glob.glob(os.path.join(csv_dir, "**", "*counter_collection.csv"), recursive=True)
    tpaths = glob.glob(os.path.join(csv_dir, "**", "*kernel_trace.csv"), recursive=True)
    if not cpaths or not tpaths:
        raise FileNotFoundError(f"need *counter_collection.csv and *kernel_trace.csv under {csv_dir}")
    dur = {}
    for p in tpaths:
        with open(p) as f:
            for r in csv.DictReader(f):
                dur[_col(r, "Dispatch_Id")] = (float(_col(r, "End_Timestamp")) - float(_col(r, "Start_Timestamp"))) * 1e-9
    per = collections.defaultdict(lambda: collections.defaultdict(dict))  # kernel -> dispatch -> counter -> value
    for p in cpaths:
        with open(p) as f:
            for r in csv.DictReader(f):
                d = _col(r, "Dispatch_Id")
                per[short_name(_col(r, "Kernel_Name"))][d][_col(r, "Counter_Name")] = float(_col(r, "Counter_Value"))
    out = ["| kernel | launches | MFMA busy % (median) | bf16 MFMA flops / launch | launch us (this run) | "
           f"PFLOP/s | of {peak_flops / 1e15:.1f} PFLOP/s |", "|---|---|---|---|---|---|---|"]
    rows = []
    for k, ds in per.items():
        util = [v.get("MfmaUtil") for v in ds.values() if v.get("MfmaUtil") is not None]
        flops = [v["SQ_INSTS_VALU_MFMA_MOPS_BF16"] * 512 for v in ds.values() if "SQ_INSTS_VALU_MFMA_MOPS_BF16" in v]
        secs = [dur[d] for d in ds if d in dur]
        if not flops or max(flops) == 0:
            continue
        f, t = statistics.median(flops), statistics.median(secs) if secs else float("nan")
        rows.append((f * len(ds), f"| `{k[:60]}` | {len(ds)} | {statistics.median(util) if util else float('nan'):.1f} | "
                                  f"{f:.4g} | {t * 1e6:.1f} | {f / t / 1e15:.3f} | {f / t / peak_flops:.3f} |"))
    out += [r for _, r in sorted(rows, key=lambda x: -x[0])]
    return "\n".join(out)


def main():
    ap = argparse.ArgumentParser()
    sub = ap.add_subparsers(dest="cmd", required=True)
    t = sub.add_parser("trace")
    t.add_argument("db")
    r = sub.add_parser("traffic")
    r.add_argument("--workload", required=True)
    r.add_argument("--fetch", required=True)
    r.add_argument("--write", required=True)
    r.add_argument("--copy-fetch", required=True)
    r.add_argument("--copy-write", required=True)
    r.add_argument("--copy-bytes", type=int, required=True)
    r.add_argument("--out", required=True)
    r.add_argument("--command", default="")
    m = sub.add_parser("mfma")
    m.add_argument("csv_dir")
    args = ap.parse_args()
    if args.cmd == "mfma":
        print(mfma_table(args.csv_dir))
        return
    if args.cmd == "trace":
        print(trace_table(args.db))
        print()
        print(step_breakdown(args.db))
        return
    fs = copy_scale(args.copy_fetch, args.copy_bytes)
    ws = copy_scale(args.copy_write, args.copy_bytes)
    fetch = counter_medians(args.fetch)
    write = counter_medians(args.write)
    sha = source_sha()
    lines = [f"# HBM traffic per launch: {args.workload}", "",
             "FETCH_SIZE and WRITE_SIZE medians per kernel launch, each scaled by what the same counter "
             f"reads for a plain copy of {args.copy_bytes} bytes (bytes per counter unit: fetch {fs:.1f}, "
             f"write {ws:.1f}).", ""]
    if args.command:
        lines += ["Commands (repo root, one MI355X):", "", "```", args.command, "```", ""]
    lines += ["| kernel | fetch bytes | write bytes | total |", "|---|---|---|---|"]
    recs = []
    for k in sorted(set(fetch) | set(write), key=lambda k: -(fetch.get(k, 0) * fs + write.get(k, 0) * ws)):
        fb, wb = int(fetch.get(k, 0) * fs), int(write.get(k, 0) * ws)
        lines.append(f"| `{k[:60]}` | {fb} | {wb} | {fb + wb} |")
        recs.append(f"traffic_bytes_per_launch {k.replace(' ', '')} {fb + wb} fetch {fb} write {wb} sha256 {sha}")
    lines += ["", "Machine-readable lines (kernel, bytes per launch, source hash of the build measured):", "", "```"]
    lines += recs + ["```", ""]
    with open(args.out, "w") as f:
        f.write("\n".join(lines))
    print("\n".join(lines))


if __name__ == "__main__":
    main()
