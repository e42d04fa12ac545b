"""Helpers that turn rocprofv3 output into the short summaries kept under
``profiles/`` and give bench.py the measured HBM traffic of a kernel.

Two summaries are produced:

* a kernel-time table from ``rocprofv3 --kernel-trace --stats`` (the
  ``*_kernel_stats.csv`` file), and
* the HBM bytes of one launch of a kernel, from two ``rocprofv3 --pmc`` runs
  (``FETCH_SIZE``, then ``WRITE_SIZE``; both report KiB per dispatch), each
  scaled by what the same counter reads for a plain device copy of known
  size (``bench.py --copy-calibration``).  The summary records a digest of
  the source files that define the measured kernel; bench.py reports the
  traffic only while those files still have that digest, i.e. while the
  kernel is the one measured.

Command line:
  python -m block_draft_decoding_amd.profiling stats STATS_CSV OUT_MD TITLE COMMAND [BENCH_JSON]
  python -m block_draft_decoding_amd.profiling traffic --tag TAG --kernel-regex RE \\
      --fetch CSV --write CSV --copy-fetch CSV --copy-write CSV --copy-bytes N \\
      --commands CMDS_TXT --out OUT_MD
"""
from __future__ import annotations

import argparse
import csv
import glob
import hashlib
import json
import os
import re
import sys
from typing import Dict, List, Optional

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "block_draft_decoding_amd", "csrc")
TRAFFIC_MD = os.path.join(ROOT, "profiles", "hbm_traffic_gemm_gate_up_traj2d3d_L385.md")


# source files that define each kernel tag's code (its kernel, the helpers it
# includes, and the launch plan)
KERNEL_SOURCES = {"gemm": ("gemm.hip", "gemm.h", "lds_pipe.h", "common.h")}


def kernel_files(tag: Optional[str]) -> Optional[tuple]:
    if tag and tag.startswith("gemm"):
        return KERNEL_SOURCES["gemm"]
    return None


def source_digest(files: Optional[tuple] = None) -> str:
    """sha256 over the given library sources (default: all kernel and host
    sources), sorted by name."""
    h = hashlib.sha256()
    for p in sorted(glob.glob(os.path.join(CSRC, "*"))):
        name = os.path.basename(p)
        if os.path.splitext(p)[1] in (".hip", ".h", ".cpp") and (files is None or name in files):
            h.update(name.encode())
            with open(p, "rb") as f:
                h.update(f.read())
    return h.hexdigest()[:16]


def short_kernel_name(n: str) -> str:
    n = n.replace("fpd::(anonymous namespace)::", "").replace("fpd::", "").replace("(anonymous namespace)::", "")
    n = n.replace("unsigned short", "bf16")
    m = re.match(r"(?:void )?([A-Za-z0-9_]+)(<[^(]*>)?", n)
    base = m.group(1) if m else n
    targs = m.group(2) if m and m.group(2) else ""
    for a, b in (("MapPlain", "plain"), ("MapRope", "rope"), ("MapGlu", "glu"), ("EpiResid", "resid"),
                 ("EpiStore", "store"), ("EpiQkv<bf16>", "qkv"), ("EpiCtx<bf16>", "ctx"),
                 ("EpiGlu<bf16>", "swiglu"), ("true", "paired"), ("false", "plain")):
        targs = targs.replace(a, b)
    return base + targs


def stats_markdown(stats_csv: str, title: str, command: str, bench_json: Optional[str] = None) -> str:
    rows = list(csv.DictReader(open(stats_csv)))
    lines = [f"# {title}", "", "Command (run from the repository root on one MI355X):", "", "```", command, "```", "",
             "| kernel | calls | avg µs | min µs | max µs | % of GPU time |", "|---|---:|---:|---:|---:|---:|"]
    for r in rows:
        lines.append(f"| `{short_kernel_name(r['Name'])}` | {r['Calls']} | {float(r['AverageNs']) / 1e3:.1f} | "
                     f"{float(r['MinNs']) / 1e3:.1f} | {float(r['MaxNs']) / 1e3:.1f} | {float(r['Percentage']):.2f} |")
    if bench_json:
        with open(bench_json) as f:
            b = json.loads(f.read().strip().splitlines()[-1])
        r = b["roofline"]
        lines += ["", f"bench.py line of the same build (same command without the profiler, run right after "
                      f"it): {b['value']:.0f} drafted tokens/s, {b['ms_per_step']} ms "
                      f"per block; dominant kernel `{r['kernel']}` {r['avg_launch_ms'] * 1e3:.1f} µs per launch "
                      f"({r['achieved']} {r['unit']}, {100 * r['frac']:.1f}% of peak)."]
    lines += ["", f"Library source digest: `{source_digest()}`"]
    return "\n".join(lines) + "\n"


def counter_per_dispatch(csv_dir_or_file: str, counter: str, kernel_regex: str) -> Dict[str, float]:
    """Mean value of `counter` per dispatch of the kernels matching the regex
    (summed over the counter's instances within a dispatch)."""
    path = csv_dir_or_file
    if os.path.isdir(path):
        found = glob.glob(os.path.join(path, "**", "*counter_collection.csv"), recursive=True)
        if not found:
            raise FileNotFoundError(f"no counter_collection.csv under {path}")
        path = found[0]
    per: Dict[str, float] = {}
    rx = re.compile(kernel_regex)
    for r in csv.DictReader(open(path)):
        if r["Counter_Name"] != counter or not rx.search(r["Kernel_Name"]):
            continue
        per[r["Dispatch_Id"]] = per.get(r["Dispatch_Id"], 0.0) + float(r["Counter_Value"])
    if not per:
        raise ValueError(f"no {counter} samples for /{kernel_regex}/ in {path}")
    vals = sorted(per.values())
    return {"mean": sum(vals) / len(vals), "n": len(vals), "min": vals[0], "max": vals[-1]}


def traffic_summary(args) -> str:
    fetch = counter_per_dispatch(args.fetch, "FETCH_SIZE", args.kernel_regex)
    write = counter_per_dispatch(args.write, "WRITE_SIZE", args.kernel_regex)
    cf = counter_per_dispatch(args.copy_fetch, "FETCH_SIZE", args.copy_regex)
    cw = counter_per_dispatch(args.copy_write, "WRITE_SIZE", args.copy_regex)
    kib = args.copy_bytes / 1024.0
    f_fetch, f_write = kib / cf["mean"], kib / cw["mean"]
    fetch_b = fetch["mean"] * 1024.0 * f_fetch
    write_b = write["mean"] * 1024.0 * f_write
    rec = {"tag": args.tag, "workload": args.workload, "kernel_regex": args.kernel_regex, "fetch_bytes": round(fetch_b),
           "write_bytes": round(write_b), "traffic_bytes": round(fetch_b + write_b),
           "copy_factor_fetch": round(f_fetch, 4), "copy_factor_write": round(f_write, 4),
           "source_files": list(kernel_files(args.tag) or ()), "source_digest": source_digest(kernel_files(args.tag))}
    cmds = open(args.commands).read().strip() if args.commands else ""
    lines = [f"# HBM traffic of one `{args.tag}` launch (64-waypoint 2D+3D trajectory block, L=385, bf16)", "",
             "Counters from four `rocprofv3 --pmc` runs (run from the repository root on one MI355X):", "",
             "```", cmds, "```", "",
             "| quantity | per dispatch | dispatches |", "|---|---:|---:|",
             f"| FETCH_SIZE, kernel (KiB) | {fetch['mean']:.0f} | {fetch['n']} |",
             f"| WRITE_SIZE, kernel (KiB) | {write['mean']:.0f} | {write['n']} |",
             f"| FETCH_SIZE, copy of {args.copy_bytes} B (KiB) | {cf['mean']:.0f} | {cf['n']} |",
             f"| WRITE_SIZE, copy of {args.copy_bytes} B (KiB) | {cw['mean']:.0f} | {cw['n']} |", "",
             f"Scale factors (copy bytes / counter bytes): fetch {f_fetch:.4f}, write {f_write:.4f}.  "
             f"HBM traffic per launch: {fetch_b / 1e6:.1f} MB read + {write_b / 1e6:.1f} MB written = "
             f"{(fetch_b + write_b) / 1e6:.1f} MB.", "",
             "Machine-readable record (bench.py reports `traffic` for this kernel and workload only while the "
             "kernel's source files have this digest):", "", "```json", json.dumps(rec), "```"]
    return "\n".join(lines) + "\n"


def read_traffic(tag: str, workload: str, path: str = TRAFFIC_MD) -> Optional[int]:
    """Measured HBM bytes per launch of `tag` in `workload`, or None when no
    measurement of that kernel in that workload exists or the kernel's
    source files changed since it was taken."""
    try:
        text = open(path).read()
    except OSError:
        return None
    m = re.search(r"```json\s*(\{.*?\})\s*```", text, re.S)
    if not m:
        return None
    rec = json.loads(m.group(1))
    if rec.get("tag") != tag or rec.get("workload") != workload:
        return None
    if rec.get("source_digest") != source_digest(kernel_files(tag)):
        return None
    return int(rec["traffic_bytes"])


def main(argv: Optional[List[str]] = None) -> int:
    ap = argparse.ArgumentParser(description="rocprofv3 summaries for profiles/")
    sub = ap.add_subparsers(dest="cmd", required=True)
    s = sub.add_parser("stats")
    s.add_argument("stats_csv")
    s.add_argument("out_md")
    s.add_argument("title")
    s.add_argument("command")
    s.add_argument("bench_json", nargs="?")
    t = sub.add_parser("traffic")
    t.add_argument("--tag", required=True)
    t.add_argument("--workload", required=True, help="bench.py workload the counters were taken on")
    t.add_argument("--kernel-regex", required=True)
    t.add_argument("--copy-regex", default="copy|Copy|elementwise")
    t.add_argument("--fetch", required=True)
    t.add_argument("--write", required=True)
    t.add_argument("--copy-fetch", required=True)
    t.add_argument("--copy-write", required=True)
    t.add_argument("--copy-bytes", type=int, required=True)
    t.add_argument("--commands", default=None)
    t.add_argument("--out", default=TRAFFIC_MD)
    a = ap.parse_args(argv)
    if a.cmd == "stats":
        with open(a.out_md, "w") as f:
            f.write(stats_markdown(a.stats_csv, a.title, a.command, a.bench_json))
    else:
        with open(a.out, "w") as f:
            f.write(traffic_summary(a))
    return 0


if __name__ == "__main__":
    sys.exit(main())
