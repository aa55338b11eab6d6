"""Summaries of rocprofv3 CSV output for the library's kernels.

    python -m fp8_blockwise_quantized_amd.profile_summary trace DIR [--title T] [--cmd C]
    python -m fp8_blockwise_quantized_amd.profile_summary counters DIR [--title T] [--cmd C]
    python -m fp8_blockwise_quantized_amd.profile_summary hbm WORKLOAD FETCH_DIR WRITE_DIR --out JSON
        [--cmd C --cmd C]

`trace` reads the *_kernel_stats.csv of a `rocprofv3 --kernel-trace --stats
--output-format csv` run; `counters` reads the *_counter_collection.csv of a
`rocprofv3 --pmc ... --output-format csv` run.  Each prints a markdown table
per kernel kind (average over its dispatches) with the command that made it.
`hbm` turns a FETCH_SIZE pass and a WRITE_SIZE pass of one bench.py
workload (run with --copy-probe, so each pass also counts three 1 GiB device
copies) into HBM bytes per launch of each of the bench's kernel names, scaled
by the copy's known bytes over its counter reading, and writes the JSON that
bench.py reads for the `traffic` field (stamped with the SHA-256 of the
kernel sources it covers, so a later change to them voids it).
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
    m = re.search(r"k_gemm_fp8_skinny<(\d+), (\d+), (\d+), (\d+), (\d+), (\w+), (\w+)>", name)
    if m:
        mt, nst, ws, ks, out, fq, p2 = m.groups()
        return f"gemm small-M forward ({int(mt) * 16}-row groups){' P2' if p2 == 'true' else ''}"
    m = re.search(r"\b(k_\w+)(<[^(]*>)?\(", name)
    if m:
        return m.group(1) + (m.group(2) or "")
    return name.split("(")[0][:80]


def _csv(d: str, suffix: str) -> str:
    hits = glob.glob(os.path.join(d, "**", f"*{suffix}"), recursive=True)
    if not hits:
        raise SystemExit(f"no *{suffix} under {d}")
    return sorted(hits)[0]


def trace(d: str, by_grid: bool = False):
    """Per kernel kind: calls, average, min, max and total duration.  With
    by_grid, from the per-dispatch trace, one row per (kind, grid) so that
    launches of one kernel on different shapes (decode layers) stay apart."""
    agg = collections.OrderedDict()
    if by_grid:
        rows = list(csv.DictReader(open(_csv(d, "_kernel_trace.csv"))))
        for r in rows:
            name = r["Kernel_Name"]
            if "jet::" not in name:
                continue
            wg = int(r.get("Workgroup_Size_X") or 1) * int(r.get("Workgroup_Size_Y") or 1)
            gx, gy, gz = (int(r.get(f"Grid_Size_{a}") or 1) for a in "XYZ")
            grid = f"{gx // max(int(r.get('Workgroup_Size_X') or 1), 1)} x {gy} x {gz}"
            dur = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"]))
            k = (kind(name), grid)
            a = agg.setdefault(k, {"calls": 0, "total_ns": 0.0, "min": float("inf"), "max": 0.0})
            a["calls"] += 1
            a["total_ns"] += dur
            a["min"] = min(a["min"], dur)
            a["max"] = max(a["max"], dur)
        out = ["| kernel kind | grid (workgroups) | calls | average us | min us | max us | total ms |",
               "|---|---|---|---|---|---|---|"]
        for (k, g), a in sorted(agg.items(), key=lambda kv: -kv[1]["total_ns"]):
            out.append(f"| {k} | {g} | {a['calls']} | {a['total_ns'] / a['calls'] / 1e3:.2f} | "
                       f"{a['min'] / 1e3:.2f} | {a['max'] / 1e3:.2f} | {a['total_ns'] / 1e6:.3f} |")
        return out
    rows = list(csv.DictReader(open(_csv(d, "_kernel_stats.csv"))))
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


# ---- hbm: FETCH_SIZE / WRITE_SIZE passes -> HBM bytes per launch ----

CSRC = os.path.join(os.path.dirname(os.path.abspath(__file__)), "csrc")
# kernel sources whose change voids a workload's counters
HBM_SOURCES = {"train": ("gemm.hip", "quant.hip"), "pow2": ("gemm.hip", "quant.hip"),
               "qwen": ("gemm.hip", "quant.hip"), "moe": ("gemm.hip", "quant.hip"),
               "decode": ("gemm.hip",), "decode_invariant": ("gemm.hip",), "decode_pow2": ("gemm.hip",),
               "fused": ("fused.hip",), "kv": ("kvcache.hip",)}


def source_shas(workload: str) -> dict:
    import hashlib
    return {f: hashlib.sha256(open(os.path.join(CSRC, f), "rb").read()).hexdigest()
            for f in HBM_SOURCES[workload]}


def _dispatches(d: str):
    """[(dispatch id, kernel name, value)] of a one-counter pass, in dispatch order."""
    rows = list(csv.DictReader(open(_csv(d, "_counter_collection.csv"))))
    out = {}
    for r in rows:
        out[int(r["Dispatch_Id"])] = (r["Kernel_Name"], float(r["Counter_Value"]))
    return [(i, n, v) for i, (n, v) in sorted(out.items())]


def _bench_name(workload: str, name: str) -> str | None:
    """The bench.py kernel name of a library dispatch (None: not one the
    workload's line reports)."""
    k = kind(name)
    sfx = "_pow2" if workload == "pow2" else ""
    if workload in ("train", "pow2", "qwen"):
        if k.split("<")[0] == "k_quant_128x128":
            return "quant_w128x128" + sfx
        if k.startswith("k_quant_1x128_128x1_T"):
            return ("quant_1x128_128x1_T_requant" if "<true" in k else "quant_1x128_128x1_T_bf16") + sfx
        if k.startswith("gemm ") and "grouped" not in k and "small-M" not in k:
            g = "gemm_fwd" if "fwd+fused" in k else "gemm_wgrad" if "wgrad" in k else "gemm_dgrad"
            return g + sfx
        return None
    if workload == "moe":
        if "grouped-rows fwd+fused" in k:
            return "grouped_fwd"
        if "grouped-rows" in k:
            return "grouped_dgrad"
        if "grouped-contraction" in k:
            return "grouped_wgrad"
        return None
    if workload == "fused":
        return {"k_rmsnorm_quant_1x128": "rmsnorm_quant_1x128",
                "k_swiglu_quant_1x128": "swiglu_quant_1x128"}.get(k.split("<")[0])
    return None


def hbm(workload: str, fetch_dir: str, write_dir: str, out: str, cmds):
    sides = {}
    for side, d in (("fetch", fetch_dir), ("write", write_dir)):
        ds = _dispatches(d)
        copies = [v for (_, n, v) in ds if "copyBuffer" in n]
        big = [v for v in copies if v >= 0.9 * max(copies)] if copies else []
        if len(big) != 3:
            raise SystemExit(f"{d}: expected the three 1 GiB calibration copies, found {len(big)}")
        # a 1 GiB copy reads and writes 1 GiB: KiB expected / KiB counted
        factor = 1048576.0 / (sum(big) / 3)
        jet = [(n, v) for (_, n, v) in ds if "jet::" in n]
        sides[side] = (factor, jet)
    per = collections.OrderedDict()
    ff, fj = sides["fetch"]
    wf, wj = sides["write"]
    if len(fj) != len(wj):
        raise SystemExit(f"the passes saw {len(fj)} and {len(wj)} library dispatches")
    if workload.startswith("decode"):
        # one call = the weight-streaming kernel (+ its finishing pass); calls in layer order
        layers = ["fwd_qkv", "fwd_o", "fwd_gate_up", "fwd_down"]
        variant = {"decode": "split_k", "decode_invariant": "batch_invariant", "decode_pow2": "pow2"}[workload]
        calls = []
        for (n, f), (_, w) in zip(fj, wj):
            if "k_gemm_fp8_skinny" in n or "k_gemm_fp8_decode" in n:
                calls.append([f, w])
            elif "k_skinny_finish" in n and calls:
                calls[-1][0] += f
                calls[-1][1] += w
        for i, (f, w) in enumerate(calls):
            per.setdefault(f"{layers[i % 4]}_{variant}", []).append((f, w))
    elif workload == "kv":
        # kv_calibrate = clear + amax (whose last workgroup writes the scales);
        # then the prefill append, then the decode append
        appends, cal = 0, None
        for (n, f), (_, w) in zip(fj, wj):
            k = kind(n)
            if k.startswith("k_kv_clear"):
                cal = [f, w]
            elif k.startswith("k_kv_amax"):
                per.setdefault("kv_calibrate", []).append((cal[0] + f, cal[1] + w))
            elif k.startswith("k_kv_append"):
                per.setdefault("kv_append_prefill" if appends % 2 == 0 else "kv_append_decode", []).append((f, w))
                appends += 1
    else:
        for (n, f), (_, w) in zip(fj, wj):
            b = _bench_name(workload, n)
            if b is not None:
                per.setdefault(b, []).append((f, w))
    kernels = {}
    for b, xs in per.items():
        fk = sum(x[0] for x in xs) / len(xs)
        wk = sum(x[1] for x in xs) / len(xs)
        kernels[b] = {"launches": len(xs), "fetch_kib_raw": round(fk, 3), "write_kib_raw": round(wk, 3),
                      "hbm_read_bytes": round(fk * 1024 * ff), "hbm_write_bytes": round(wk * 1024 * wf),
                      "hbm_bytes_per_launch": round((fk * ff + wk * wf) * 1024)}
    doc = {"workload": workload, "sources_sha256": source_shas(workload), "commands": list(cmds),
           "calibration": {"fetch_factor": ff, "write_factor": wf,
                           "what": "three 1 GiB device copies per pass; factor = 1 GiB / the copy's counted KiB"},
           "kernels": kernels}
    import json
    with open(out, "w") as fh:
        json.dump(doc, fh, indent=1)
    lines = [f"| {b} | {v['launches']} | {v['fetch_kib_raw']:.0f} | {v['write_kib_raw']:.0f} | "
             f"{v['hbm_bytes_per_launch'] / 1e6:.2f} |" for b, v in kernels.items()]
    return ["| kernel | launches | FETCH KiB (raw) | WRITE KiB (raw) | HBM MB per launch (calibrated) |",
            "|---|---|---|---|---|"] + lines


def main(argv=None):
    ap = argparse.ArgumentParser()
    ap.add_argument("what", choices=("trace", "counters", "hbm"))
    ap.add_argument("dir", help="result directory, or (hbm) the workload")
    ap.add_argument("more", nargs="*", help="(hbm) the FETCH_SIZE and WRITE_SIZE result directories")
    ap.add_argument("--title", default="")
    ap.add_argument("--cmd", action="append", default=[])
    ap.add_argument("--out", default="")
    ap.add_argument("--by-grid", action="store_true", help="(trace) one row per kernel kind and grid")
    a = ap.parse_args(argv)
    lines = []
    if a.title:
        lines += [f"## {a.title}", ""]
    if a.cmd:
        lines += ["Command:" if len(a.cmd) == 1 else "Commands:", ""] + [f"    {c}" for c in a.cmd] + [""]
    if a.what == "hbm":
        if len(a.more) != 2 or not a.out:
            raise SystemExit("hbm WORKLOAD FETCH_DIR WRITE_DIR --out JSON")
        lines += hbm(a.dir, a.more[0], a.more[1], a.out, a.cmd)
    else:
        lines += trace(a.dir, a.by_grid) if a.what == "trace" else counters(a.dir)
    print("\n".join(lines))


if __name__ == "__main__":
    sys.exit(main())
