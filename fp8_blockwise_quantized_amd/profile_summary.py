"""Summaries of rocprofv3 CSV output for the library's kernels.

    python -m fp8_blockwise_quantized_amd.profile_summary trace DIR [--title T] [--cmd C]
    python -m fp8_blockwise_quantized_amd.profile_summary counters DIR [--title T] [--cmd C]

`trace` reads the *_kernel_stats.csv of a `rocprofv3 --kernel-trace --stats
--output-format csv` run; `counters` reads the *_counter_collection.csv of a
`rocprofv3 --pmc ... --output-format csv` run.  Each prints a markdown table
per kernel kind (average over its dispatches) with the command that made it.
Kernel kinds are named from the template arguments of the GEMM kernels:
forward (row-block scales, fused 1x128 output), dgrad (row-block scales,
BF16 output), wgrad (row x column scales), grouped variants, power-of-two
variant (P2), tile 256x256 or 128x128.
"""
from __future__ import annotations

import argparse
import collections
import csv
import glob
import os
import re
import sys


def kind(name: str) -> str:
    """Short kind of a kernel from its demangled name."""
    m = re.search(r"k_gemm_fp8<jet::GemmCfg<(\d+), (\d+), (\d+), (\d+), (\d+), (\w+), (\d+)>, (\d+), (\d+), "
                  r"(\w+), (\w+), (\d+), (\w+)>", name)
    if m:
        wmw, wnw, tm, tn, _, _, _, mode, out, acc, fuseq, grp, p2 = m.groups()
        tile = f"{int(wmw) * int(tm) * 16}x{int(wnw) * int(tn) * 16}"
        if mode == "1":
            k = "wgrad"
        elif fuseq == "true":
            k = "fwd+fused-quant"
        else:
            k = "dgrad/fwd (bf16)" if out == "0" else "fwd/dgrad (f32)"
        g = {"0": "", "1": "grouped-rows ", "2": "grouped-contraction "}[grp]
        return f"gemm {g}{k} {tile}{' P2' if p2 == 'true' else ''}{' accumulate' if acc == 'true' else ''}"
    m = re.search(r"k_gemm_fp8_skinny<(\d+), (\d+), (\d+), (\d+), (\w+), (\w+)>", name)
    if m:
        mt, nst, ws, out, fq, p2 = m.groups()
        return f"gemm small-M forward ({int(mt) * 16}-row groups){' P2' if p2 == 'true' else ''}"
    m = re.search(r"jet::(k_\w+)(<[^(]*>)?", name)
    if m:
        return m.group(1) + (m.group(2) or "")
    return name.split("(")[0][:80]


def _csv(d: str, suffix: str) -> str:
    hits = glob.glob(os.path.join(d, "**", f"*{suffix}"), recursive=True)
    if not hits:
        raise SystemExit(f"no *{suffix} under {d}")
    return sorted(hits)[0]


def trace(d: str):
    rows = list(csv.DictReader(open(_csv(d, "_kernel_stats.csv"))))
    agg = collections.OrderedDict()
    for r in rows:
        k = kind(r["Name"])
        a = agg.setdefault(k, {"calls": 0, "total_ns": 0.0, "min": float("inf"), "max": 0.0})
        a["calls"] += int(r["Calls"])
        a["total_ns"] += float(r["TotalDurationNs"])
        a["min"] = min(a["min"], float(r["MinNs"]))
        a["max"] = max(a["max"], float(r["MaxNs"]))
    out = ["| kernel kind | calls | average us | min us | max us | total ms |", "|---|---|---|---|---|---|"]
    for k, a in sorted(agg.items(), key=lambda kv: -kv[1]["total_ns"]):
        out.append(f"| {k} | {a['calls']} | {a['total_ns'] / a['calls'] / 1e3:.2f} | {a['min'] / 1e3:.2f} | "
                   f"{a['max'] / 1e3:.2f} | {a['total_ns'] / 1e6:.3f} |")
    return out


def counters(d: str):
    rows = list(csv.DictReader(open(_csv(d, "_counter_collection.csv"))))
    disp = collections.OrderedDict()
    for r in rows:
        v = disp.setdefault(r["Dispatch_Id"], {"name": r["Kernel_Name"]})
        v[r["Counter_Name"]] = float(r["Counter_Value"])
    names = []
    agg = collections.OrderedDict()
    for v in disp.values():
        if "jet::" not in v["name"]:
            continue
        k = kind(v["name"])
        for c, x in v.items():
            if c == "name":
                continue
            if c not in names:
                names.append(c)
            agg.setdefault(k, collections.defaultdict(list))[c].append(x)
    out = ["| kernel kind | dispatches | " + " | ".join(names) + " |", "|---|---|" + "---|" * len(names)]
    for k, cs in agg.items():
        n = len(next(iter(cs.values())))
        vals = []
        for c in names:
            xs = cs.get(c, [])
            m = sum(xs) / len(xs) if xs else float("nan")
            vals.append(f"{m:.1f}" if abs(m) < 1e4 else f"{m:.4g}")
        out.append(f"| {k} | {n} | " + " | ".join(vals) + " |")
    return out


def main(argv=None):
    ap = argparse.ArgumentParser()
    ap.add_argument("what", choices=("trace", "counters"))
    ap.add_argument("dir")
    ap.add_argument("--title", default="")
    ap.add_argument("--cmd", default="")
    a = ap.parse_args(argv)
    lines = []
    if a.title:
        lines += [f"## {a.title}", ""]
    if a.cmd:
        lines += ["Command:", "", f"    {a.cmd}", ""]
    lines += trace(a.dir) if a.what == "trace" else counters(a.dir)
    print("\n".join(lines))


if __name__ == "__main__":
    sys.exit(main())
