"""Phase timing of the GEMM kernel's workgroups (diagnostic; needs a GPU).

Runs the GEMMs of a benchmark workload through the diagnostic build
libjetfp8_phase.so (include/jetphase.h) and summarises, per GEMM call, what
its workgroups spent in each phase: tile set-up, the K loop (per K step, and
the shader clock it ran at, from the shader-clock counter over the wall
counter), the epilogue, the gap until the next workgroup starts on the same
CU, and how long CUs sat idle at the kernel's end.

    python -m fp8_blockwise_quantized_amd.phase_timing [--workload train|moe] [--out FILE]

(from the repository root: it builds its layers with bench.py's classes).
"""
from __future__ import annotations

import argparse
import ctypes
import os
import sys

import numpy as np

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
PHASE_LIB = os.path.join(PKG, "lib", "libjetfp8_phase.so")

# MFMA issue clocks per K step on each SIMD: the 256 x 256 tile (512 threads)
# runs 8 wavefronts, 2 per SIMD, of 32 MFMAs of 32 shader clocks; the 128 x
# 128 tile (256 threads, two workgroups per CU) 4 wavefronts, one per SIMD,
# of 16 such MFMAs.
MFMA_CLOCKS_PER_STEP = {512: 2 * 32 * 32, 256: 16 * 32}


class Phase:
    def __init__(self):
        self.lib = ctypes.CDLL(PHASE_LIB)
        self.hip = ctypes.CDLL("libamdhip64.so")
        self.rec, self.flag, cap = ctypes.c_void_p(), ctypes.c_void_p(), ctypes.c_int()
        if self.lib.jet_phase_buffers(ctypes.byref(self.rec), ctypes.byref(self.flag), ctypes.byref(cap)):
            raise RuntimeError("jet_phase_buffers failed")
        self.cap = cap.value
        self.wall_khz = float(self._wall_khz())

    def _wall_khz(self) -> int:
        # the wall counter's rate, as the roofline probes library reports it
        probe = ctypes.CDLL(os.path.join(PKG, "lib", "libjetprobe.so"))
        khz = probe.jet_probe_wall_clock_khz()
        if khz <= 0:
            raise RuntimeError("wall clock rate unavailable")
        return khz

    def _copy(self, dst, src, n, kind):
        if self.hip.hipMemcpy(dst, src, ctypes.c_size_t(n), kind) != 0:
            raise RuntimeError("hipMemcpy failed")

    def set_flag(self, v: int):
        x = ctypes.c_int(v)
        self._copy(self.flag, ctypes.byref(x), 4, 1)

    def clear(self):
        z = np.zeros(self.cap * 8, np.uint64)
        self._copy(self.rec, z.ctypes.data_as(ctypes.c_void_p), z.nbytes, 1)

    def records(self) -> np.ndarray:
        b = np.zeros(self.cap * 8, np.uint64)
        self._copy(b.ctypes.data_as(ctypes.c_void_p), self.rec, b.nbytes, 2)
        return b.reshape(self.cap, 8)

    def run(self, torch, fn):
        for _ in range(3):
            fn()
        torch.cuda.synchronize()
        self.clear()
        self.set_flag(1)
        torch.cuda.synchronize()
        fn()
        torch.cuda.synchronize()
        self.set_flag(0)
        return self.records()


def summarise(rec: np.ndarray, wall_khz: float, ksteps: int | None):
    """One row per launch (records grouped by grid size)."""
    rows = []
    rec = rec[rec[:, 0] > 0]
    us = lambda t: t * 1000.0 / wall_khz
    for launch in sorted(set(rec[:, 5].tolist()), reverse=True):
        r = rec[rec[:, 5] == launch].astype(np.int64)
        grid, threads = launch & 0xFFFFFFFF, launch >> 32
        t0, t1, t2, t3 = r[:, 0], r[:, 1], r[:, 2], r[:, 3]
        work = t1 > 0                        # workgroups that had a tile
        complete = len(r) == grid
        hw, xcc = r[:, 4] & 0xFFFFFFFF, r[:, 4] >> 32
        cu = (xcc & 0xF) * 1000 + ((hw >> 13) & 7) * 100 + ((hw >> 12) & 1) * 16 + ((hw >> 8) & 15)
        loop = us(t2 - t1)[work]
        mhz = ((r[:, 7] - r[:, 6])[work] / np.maximum((t2 - t1)[work], 1)) * wall_khz / 1000.0
        row = dict(grid=int(grid), threads=int(threads), recorded=int(len(r)), tiles=int(work.sum()), complete=complete,
                   setup=float(np.median(us(t1 - t0)[work])), loop=float(np.median(loop)),
                   epi=float(np.median(us(t3 - t2)[work])), mhz=float(np.median(mhz)))
        if ksteps:
            row["step"] = row["loop"] / ksteps
            row["clk_step"] = row["step"] * row["mhz"]
            if threads in MFMA_CLOCKS_PER_STEP:
                row["mfma_share"] = MFMA_CLOCKS_PER_STEP[threads] / row["clk_step"]
        if complete:
            span = us(t3.max() - t0.min())
            busy, gaps, tail = [], [], []
            for c in np.unique(cu):
                m = cu == c
                o = np.argsort(t0[m])
                s0, s3 = t0[m][o], t3[m][o]
                # time the CU held at least one of the launch's workgroups
                # (the small tile runs two at once)
                covered, end = 0, s0[0]
                for a, b in zip(s0, s3):
                    covered += max(0, b - max(a, end))
                    end = max(end, b)
                busy.append(us(covered))
                if threads == 512:      # one workgroup per CU: the gaps between them
                    gaps += list(us(s0[1:] - s3[:-1]))
                tail.append(us(t3.max() - s3.max()))
            row.update(span=span, busy=float(np.mean(busy)) / span,
                       gap=float(np.median(gaps)) if gaps else None, tail=float(np.mean(tail)),
                       cus=int(len(np.unique(cu))))
        rows.append(row)
    return rows


def fmt(v, d=2):
    return "" if v is None else f"{v:.{d}f}"


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--workload", choices=["train", "moe"], default="train")
    ap.add_argument("--out", default=None)
    args = ap.parse_args()
    os.environ["JET_LIB_PATH"] = PHASE_LIB          # before the binding loads a library
    sys.path.insert(0, ROOT)
    import torch
    import bench
    from fp8_blockwise_quantized_amd import jetfp8 as J
    ph = Phase()
    out = []
    cmd = f"python -m fp8_blockwise_quantized_amd.phase_timing --workload {args.workload}"
    out.append(f"Command (from the repository root): `{cmd}`\n")
    out.append("Each GEMM call of the workload once, after three unrecorded calls; medians over its "
               "workgroups. MFMA issue share: the MFMA clocks one K step needs on a SIMD (2048 for the "
               "256 x 256 tile, 512 per workgroup for the 128 x 128 tile, two of which share a CU) over "
               "the clocks the K step took. Gap: from a workgroup's exit to the next one's entry on the "
               "same CU. Idle tail: mean over CUs of the time from their last workgroup's exit to the "
               "launch's end. A call that runs as two launches shows the records of both, the first "
               "partly overwritten by the second.\n")
    out.append("| GEMM | launch grid | tiles | span us | set-up us | K loop us | us per K step | shader MHz "
               "| clocks per K step | MFMA issue share | epilogue us | gap us | CU busy | idle tail us |")
    out.append("|---|---|---|---|---|---|---|---|---|---|---|---|---|---|")
    if args.workload == "train":
        layers = [bench.Layer(J, torch, n, N, K, bench.M_TOKENS, seed=0) for (n, N, K) in bench.LAYERS]
    else:
        seg = bench.moe_routing()
        layers = [bench.MoELayer(J, torch, n, N, K, seg, seed=0) for (n, N, K) in bench.MOE_LAYERS]
    for L in layers:
        ops = L.ops(J)
        for _, _, _, fn in ops:
            fn()
        torch.cuda.synchronize()
        for kind, _, _, fn in ops:
            if kind.startswith("quant"):
                continue
            ks = {"fwd": L.K // 128, "dgrad": L.N // 128}.get(kind.split("_")[-1])
            if kind.endswith("wgrad"):
                ks = None if kind.startswith("grouped") else -(-L.M // 128)
            rec = ph.run(torch, fn)
            for row in summarise(rec, ph.wall_khz, ks):
                name = f"{L.name} {kind}"
                out.append("| " + " | ".join([
                    name, f"{row['grid']} x {row['threads']}" + ("" if row["complete"] else " (partly overwritten)"),
                    str(row["tiles"]), fmt(row.get("span"), 1), fmt(row["setup"]), fmt(row["loop"], 1),
                    fmt(row.get("step"), 3), fmt(row["mhz"], 0), fmt(row.get("clk_step"), 0),
                    fmt(row.get("mfma_share")), fmt(row["epi"]), fmt(row.get("gap")),
                    fmt(row.get("busy")), fmt(row.get("tail"), 1)]) + " |")
                print(out[-1], flush=True)
        del L
        torch.cuda.synchronize()
    text = "\n".join(out) + "\n"
    if args.out:
        with open(args.out, "w") as f:
            f.write(text)
    else:
        print(text)


if __name__ == "__main__":
    main()
