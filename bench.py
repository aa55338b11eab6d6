"""Benchmark of the FP8 linear-layer hot path on one MI355X.

One step = the whole path over the four Llama-3.1-8B decoder linears at the
training batch of M = 8192 tokens (8 sequences x 1024):
  for each of QKV (4096->6144), O (4096->4096), gate+up (4096->28672), down (14336->4096):
    128x128 re-quantization of the BF16 master weight (+ transposed codes),
    X quantized 1x128 and re-quantized 128x1 from those codes (transposed) in
    one read, forward GEMM with the fused 1x128 quantization of Y, dY
    quantized 1x128 and 128x1 (transposed) in one read, dgrad GEMM, wgrad GEMM.
Inputs are seeded synthetic tensors resident in HBM before timing starts.
`value` = GEMM FLOPs of the step (3 x 2*M*N*K per linear) / step time.

`--workload fused` the fused producers of the linear inputs of one layer
(RMSNorm + 1x128 twice, SwiGLU + 1x128 once) at M = 8192;
`--workload kv` the FP8 KV cache of one layer (scale recalibration and append
of a 8192-token prefill, append of a 64-token decode step);
`--workload decode` times the rollout forward of the same linears at M = 64;
`--workload moe` the grouped (mixture-of-experts) layer of Qwen3-30B-A3B shape
(hidden 2048, expert intermediate 768, 128 experts, top-8 of 8192 tokens with
Zipf(1.1) expert load), fwd + dgrad + wgrad with every quantizer;
`--workload qwen` the train step over the six Qwen-14B/32B-shaped linears at
M = 16384 tokens.

Every line carries `measured_ceilings`: streaming rates for the quantizers'
read/write mixes and the FP8 MFMA rate with and without the per-step FP32
fold on this GPU (include/jetprobe.h), with the shader clock under that MFMA
load, next to the published peaks the roofline fractions use.

Prints ONE JSON line.  --gpus above 1 is refused: the benchmark measures one GPU.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
METRIC = "FP8 linear fwd+bwd TFLOP/s (% FP8 MFMA peak) + quantizer GB/s, Llama-8B shapes"
PEAK_FP8_TFLOPS = 5000.0       # MI355X dense OCP-FP8 MFMA
PEAK_HBM_GBS = 8000.0          # MI355X HBM3E
LAYERS = [("qkv", 6144, 4096), ("o", 4096, 4096), ("gate_up", 28672, 4096), ("down", 4096, 14336)]
M_TOKENS = 8192
# Qwen-14B/32B (hidden 5120): QKV with 40 query and 8 key/value heads of 128,
# O, the fused gate+up of the 14B (intermediate 17408) and 32B (27648)
# models, and their down projections.
QWEN_LAYERS = [("qkv", 7168, 5120), ("o", 5120, 5120), ("gate_up_14b", 34816, 5120),
               ("gate_up_32b", 55296, 5120), ("down_14b", 5120, 17408), ("down_32b", 5120, 27648)]
QWEN_TOKENS = 16384
CSRC = os.path.join(ROOT, "fp8_blockwise_quantized_amd", "csrc")


def counters_path(workload: str) -> str:
    """The committed HBM counter summary of a workload (profile_summary.py hbm)."""
    return os.path.join(ROOT, "profiles", f"counters_{workload}.json")


def log(msg):
    """Progress on stderr (stdout carries only the JSON line)."""
    print(f"bench.py: {msg}", file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--median-steps", type=int, default=50,
                    help="steps of the per-step distribution pass (at least --steps; 0 skips it, "
                         "so a profiled run covers exactly the warm-up and timed steps)")
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--no-ceilings", action="store_true",
                    help="skip the measured ceilings (streaming and MFMA probes)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-bf16-context", action="store_true",
                    help="train: skip timing hipBLASLt BF16 GEMMs on the same shapes (context only)")
    ap.add_argument("--copy-probe", action="store_true",
                    help="run 1 GiB device copies first (HBM counter calibration)")
    ap.add_argument("--events", type=int, default=1,
                    help="1: after the timed steps, as many steps again with HIP events around every "
                         "launch (per-kernel times); 0: skip that pass")
    ap.add_argument("--workload", choices=("train", "qwen", "decode", "moe", "fused", "kv"), default="train",
                    help="train: the M=8192 fwd+bwd step (the headline line); decode: the rollout "
                         "forward at M=64 over the same four linears; qwen: the train step over the six "
                         "Qwen-14B/32B linears at M=16384; moe: the grouped expert "
                         "layer (Qwen3-30B-A3B shapes) fwd+bwd; fused: the fused RMSNorm/SwiGLU "
                         "producers of the 1x128 inputs of one Llama-8B layer; kv: the FP8 KV cache "
                         "(recalibration and append) of one Llama-8B layer")
    ap.add_argument("--fused-m", type=int, default=8192, help="tokens for --workload fused")
    ap.add_argument("--pow2", action="store_true",
                    help="train, moe, decode: the power-of-two-scale variant (E8M0 scales applied by the MFMA)")
    ap.add_argument("--invariant", action="store_true",
                    help="decode: the batch-invariant forward (one K range, bit-identical to training)")
    ap.add_argument("--no-mismatch", action="store_true",
                    help="decode: skip the token-mult-prob-error against the training forward")
    ap.add_argument("--quant", choices=("both", "separate"), default="both",
                    help="activation quantizers: one read for both groupings (default), or the "
                         "separate 1x128 and 128x1 kernels")
    return ap.parse_args()


def q_bytes_1x128(M, K):      # BF16 in, E4M3 + FP32 scale per 128 out
    return M * K * 2 + M * K + M * K // 128 * 4


def q_bytes_w(N, K, transposed=True):
    return N * K * 2 + N * K * (2 if transposed else 1) + N * K // 16384 * 4


def q_bytes_128x1_bf16(M, K):
    return M * K * 2 + M * K + M * K // 128 * 4


def q_bytes_128x1_fp8(M, K):  # E4M3 + 1x128 scales in, E4M3 + 128x1 scales out
    return M * K + M * K // 128 * 4 + M * K + M * K // 128 * 4


def q_bytes_both(M, K):       # BF16 in; 1x128 and 128x1-transposed codes and scales out
    Mp = -(-M // 128) * 128
    return M * K * 2 + M * K + M * K // 128 * 4 + Mp * K + Mp // 128 * K * 4


def q_bytes_128x1_grouped(M, K, P, fp8_src):
    """Grouped 128x1-transposed quantizer: M rows in (BF16, or E4M3 + 1x128
    scales), P padded columns of codes and P/128 scale rows out."""
    src = M * K + M * K // 128 * 4 if fp8_src else M * K * 2
    return src + P * K + P // 128 * K * 4


MOE_TOKENS, MOE_EXPERTS, MOE_TOPK, MOE_ALPHA = 8192, 128, 8, 1.1
MOE_LAYERS = [("gate_up", 1536, 2048), ("down", 2048, 768)]   # per expert: (N, K)


class MoELayer:
    """One grouped expert layer: rows sorted by expert (seg), weights [E, N, K]."""

    def __init__(self, J, torch, name, N, K, seg, seed):
        from fp8_blockwise_quantized_amd import inputs
        E, M = len(seg) - 1, int(seg[-1])
        self.name, self.N, self.K, self.M, self.E = name, N, K, M, E
        dev = "cuda"
        bf = lambda a: torch.from_numpy(a).to(torch.bfloat16).to(dev)
        self.seg = torch.from_numpy(np.asarray(seg, np.int32)).to(dev)
        self.x = bf(inputs.activations_with_outliers(M, K, seed=seed))
        self.w = bf(inputs.normal_bf16((E * N, K), 0.02, seed=seed, tensor_id=inputs.ID_W))
        self.dy = bf(inputs.normal_bf16((M, N), 1e-3, seed=seed, tensor_id=inputs.ID_DY))
        u8, f32 = torch.uint8, torch.float32
        e = lambda shape, dt: torch.empty(shape, dtype=dt, device=dev)
        self.P = P = J.grouped_columns(M, E)
        self.wq, self.ws, self.wqT = e((E * N, K), u8), e((E * N // 128, K // 128), f32), e((K, E * N), u8)
        self.xq, self.xs = e((M, K), u8), e((K // 128, M), f32)
        self.y, self.yq, self.ys = e((M, N), torch.bfloat16), e((M, N), u8), e((N // 128, M), f32)
        self.dyq, self.dys = e((M, N), u8), e((N // 128, M), f32)
        self.dx = e((M, K), torch.bfloat16)
        self.dyqT, self.dysT = e((N, P), u8), e((P // 128, N), f32)
        self.xqT, self.xsT = e((K, P), u8), e((P // 128, K), f32)
        self.dw = e((E, N, K), f32)
        self.flops = 2.0 * M * N * K

    def gemm_bytes(self, kind):
        """Algorithmic HBM bytes of one grouped GEMM launch (as Layer.gemm_bytes;
        the wgrad operands in their padded layout of P columns)."""
        M, N, K, E, P = self.M, self.N, self.K, self.E, self.P
        w = E * (N * K + N * K // 16384 * 4)
        if kind == "grouped_fwd":
            return M * K + M * K // 128 * 4 + w + M * N * 2 + M * N + M * N // 128 * 4
        if kind == "grouped_dgrad":
            return M * N + M * N // 128 * 4 + w + M * K * 2
        return (N + K) * P + P // 128 * (N + K) * 4 + E * N * K * 4

    def ops(self, J, pow2=False):
        M, N, K, E, P = self.M, self.N, self.K, self.E, self.P
        wq3 = self.wq.view(E, N, K)
        ws3 = self.ws.view(E, N // 128, K // 128)
        sfx = "_pow2" if pow2 else ""
        f = lambda name: getattr(J, name + sfx)
        return [
            ("quant_w128x128", q_bytes_w(E * N, K), "B",
             lambda: f("jet_quant_weight_128x128")(self.w, q=self.wq, s=self.ws, qT=self.wqT)),
            ("quant_1x128", q_bytes_1x128(M, K), "B",
             lambda: f("jet_quant_act_1x128")(self.x, q=self.xq, s=self.xs)),
            ("quant_128x1_T_grouped_fp8", q_bytes_128x1_grouped(M, K, P, True), "B",
             lambda: f("jet_quant_act_128x1_T_grouped")(self.xq, self.seg, src_s=self.xs,
                                                        qT=self.xqT, sT=self.xsT)),
            ("grouped_fwd", self.flops, "F",
             lambda: f("jet_fp8_grouped_fwd")(self.xq, self.xs, wq3, ws3, self.seg, y=self.y,
                                              fuse_quant=True, yq=self.yq, ys=self.ys)),
            ("quant_1x128", q_bytes_1x128(M, N), "B",
             lambda: f("jet_quant_act_1x128")(self.dy, q=self.dyq, s=self.dys)),
            ("grouped_dgrad", self.flops, "F",
             lambda: f("jet_fp8_grouped_dgrad")(self.dyq, self.dys, self.wqT, ws3, self.seg, dx=self.dx)),
            ("quant_128x1_T_grouped_bf16", q_bytes_128x1_grouped(M, N, P, False), "B",
             lambda: f("jet_quant_act_128x1_T_grouped")(self.dy, self.seg, qT=self.dyqT, sT=self.dysT)),
            ("grouped_wgrad", self.flops, "F",
             lambda: f("jet_fp8_grouped_wgrad")(self.dyqT, self.dysT, self.xqT, self.xsT, self.seg, M,
                                                dw=self.dw)),
        ]


def moe_routing():
    from fp8_blockwise_quantized_amd import inputs
    ids = inputs.zipf_top8_routing(MOE_TOKENS, MOE_EXPERTS, MOE_TOPK, MOE_ALPHA, seed=0)
    return inputs.segment_offsets(ids, MOE_EXPERTS)


class Layer:
    def __init__(self, J, torch, name, N, K, M, seed):
        from fp8_blockwise_quantized_amd import inputs
        self.name, self.N, self.K, self.M = name, N, K, M
        dev = "cuda"
        bf = lambda a: torch.from_numpy(a).to(torch.bfloat16).to(dev)
        self.x = bf(inputs.activations_with_outliers(M, K, seed=seed))
        self.w = bf(inputs.normal_bf16((N, K), 0.02, seed=seed, tensor_id=inputs.ID_W))
        self.dy = bf(inputs.normal_bf16((M, N), 1e-3, seed=seed, tensor_id=inputs.ID_DY))
        u8, f32 = torch.uint8, torch.float32
        e = lambda shape, dt: torch.empty(shape, dtype=dt, device=dev)
        Mp = -(-M // 128) * 128
        self.wq, self.ws, self.wqT = e((N, K), u8), e((N // 128, K // 128), f32), e((K, N), u8)
        self.xq, self.xs = e((M, K), u8), e((K // 128, M), f32)
        self.y, self.yq, self.ys = e((M, N), torch.bfloat16), e((M, N), u8), e((N // 128, M), f32)
        self.dyq, self.dys = e((M, N), u8), e((N // 128, M), f32)
        self.dx = e((M, K), torch.bfloat16)
        self.dyqT, self.dysT = e((N, Mp), u8), e((Mp // 128, N), f32)
        self.xqT, self.xsT = e((K, Mp), u8), e((Mp // 128, K), f32)
        self.dw = e((N, K), f32)
        self.flops = 2.0 * M * N * K

    def gemm_bytes(self, kind):
        """Algorithmic HBM bytes of one GEMM launch: operand codes and scales
        read once, outputs written once."""
        M, N, K = self.M, self.N, self.K
        Mp = -(-M // 128) * 128
        w = N * K + N * K // 16384 * 4
        if kind == "gemm_fwd":
            return M * K + M * K // 128 * 4 + w + M * N * 2 + M * N + M * N // 128 * 4
        if kind == "gemm_dgrad":
            return M * N + M * N // 128 * 4 + w + M * K * 2
        return (N + K) * Mp + Mp // 128 * (N + K) * 4 + N * K * 4

    def ops(self, J, separate=False, pow2=False):
        """(kernel kind, algorithmic work, unit, callable) in path order."""
        M, N, K = self.M, self.N, self.K
        if separate:
            return self.ops_separate(J)
        if pow2:
            return self.ops_pow2(J)
        return [
            ("quant_w128x128", q_bytes_w(N, K), "B",
             lambda: J.jet_quant_weight_128x128(self.w, q=self.wq, s=self.ws, qT=self.wqT)),
            ("quant_1x128_128x1_T_requant", q_bytes_both(M, K), "B",
             lambda: J.jet_quant_act_1x128_128x1_T(self.x, True, q=self.xq, s=self.xs,
                                                   qT=self.xqT, sT=self.xsT)),
            ("gemm_fwd", self.flops, "F",
             lambda: J.jet_fp8_linear_fwd(self.xq, self.xs, self.wq, self.ws, y=self.y,
                                          fuse_quant=True, yq=self.yq, ys=self.ys)),
            ("quant_1x128_128x1_T_bf16", q_bytes_both(M, N), "B",
             lambda: J.jet_quant_act_1x128_128x1_T(self.dy, False, q=self.dyq, s=self.dys,
                                                   qT=self.dyqT, sT=self.dysT)),
            ("gemm_dgrad", self.flops, "F",
             lambda: J.jet_fp8_linear_dgrad(self.dyq, self.dys, self.wqT, self.ws, dx=self.dx)),
            ("gemm_wgrad", self.flops, "F",
             lambda: J.jet_fp8_linear_wgrad(self.dyqT, self.dysT, self.xqT, self.xsT, M, dw=self.dw)),
        ]


    def ops_pow2(self, J):
        """The same step with power-of-two scales (E8M0, applied by the MFMA)."""
        M = self.M
        return [
            ("quant_w128x128", q_bytes_w(self.N, self.K), "B",
             lambda: J.jet_quant_weight_128x128_pow2(self.w, q=self.wq, s=self.ws, qT=self.wqT)),
            ("quant_1x128_128x1_T_requant", q_bytes_both(M, self.K), "B",
             lambda: J.jet_quant_act_1x128_128x1_T_pow2(self.x, True, q=self.xq, s=self.xs,
                                                        qT=self.xqT, sT=self.xsT)),
            ("gemm_fwd", self.flops, "F",
             lambda: J.jet_fp8_linear_fwd_pow2(self.xq, self.xs, self.wq, self.ws, y=self.y,
                                               fuse_quant=True, yq=self.yq, ys=self.ys)),
            ("quant_1x128_128x1_T_bf16", q_bytes_both(M, self.N), "B",
             lambda: J.jet_quant_act_1x128_128x1_T_pow2(self.dy, False, q=self.dyq, s=self.dys,
                                                        qT=self.dyqT, sT=self.dysT)),
            ("gemm_dgrad", self.flops, "F",
             lambda: J.jet_fp8_linear_dgrad_pow2(self.dyq, self.dys, self.wqT, self.ws, dx=self.dx)),
            ("gemm_wgrad", self.flops, "F",
             lambda: J.jet_fp8_linear_wgrad_pow2(self.dyqT, self.dysT, self.xqT, self.xsT, M, dw=self.dw)),
        ]

    def ops_separate(self, J):
        """The same step with the separate 1x128 and 128x1 quantizers."""
        M, N, K = self.M, self.N, self.K
        return [
            ("quant_w128x128", q_bytes_w(N, K), "B",
             lambda: J.jet_quant_weight_128x128(self.w, q=self.wq, s=self.ws, qT=self.wqT)),
            ("quant_1x128", q_bytes_1x128(M, K), "B",
             lambda: J.jet_quant_act_1x128(self.x, q=self.xq, s=self.xs)),
            ("gemm_fwd", self.flops, "F",
             lambda: J.jet_fp8_linear_fwd(self.xq, self.xs, self.wq, self.ws, y=self.y,
                                          fuse_quant=True, yq=self.yq, ys=self.ys)),
            ("quant_1x128", q_bytes_1x128(M, N), "B",
             lambda: J.jet_quant_act_1x128(self.dy, q=self.dyq, s=self.dys)),
            ("gemm_dgrad", self.flops, "F",
             lambda: J.jet_fp8_linear_dgrad(self.dyq, self.dys, self.wqT, self.ws, dx=self.dx)),
            ("quant_128x1_T_bf16", q_bytes_128x1_bf16(M, N), "B",
             lambda: J.jet_quant_act_128x1_T(self.dy, qT=self.dyqT, sT=self.dysT)),
            ("quant_128x1_T_fp8", q_bytes_128x1_fp8(M, K), "B",
             lambda: J.jet_quant_act_128x1_T(self.xq, src_s=self.xs, qT=self.xqT, sT=self.xsT)),
            ("gemm_wgrad", self.flops, "F",
             lambda: J.jet_fp8_linear_wgrad(self.dyqT, self.dysT, self.xqT, self.xsT, M, dw=self.dw)),
        ]


def bf16_context(torch, layers, ms_step, fp8_gemm_ms, steps=10, warmup=3):
    """Context, not the product: the same linears' three GEMMs per layer as
    BF16 products through torch.mm (hipBLASLt), every operand contiguous
    (transposes materialised before timing), no quantizers.  Compared with
    the FP8 step and with the FP8 GEMMs alone; the pages report FP8 linear
    layers about 2x faster than BF16 and the FP8 training step 1.41x faster
    (end-to-end, other hardware)."""
    ops = []
    for l in layers:
        wT = l.w.t().contiguous()
        dyT = l.dy.t().contiguous()
        ops += [(lambda x=l.x, b=wT: torch.mm(x, b)),
                (lambda a=l.dy, b=l.w: torch.mm(a, b)),
                (lambda a=dyT, b=l.x: torch.mm(a, b))]
    for _ in range(warmup):
        for f in ops:
            f()
    E = torch.cuda.Event
    t0, t1 = E(enable_timing=True), E(enable_timing=True)
    torch.cuda.synchronize()
    t0.record()
    for _ in range(steps):
        for f in ops:
            f()
    t1.record()
    torch.cuda.synchronize()
    ms = t0.elapsed_time(t1) / steps
    flops = sum(3 * l.flops for l in layers)
    del ops
    torch.cuda.empty_cache()
    return {"kind": "third-party: hipBLASLt BF16 GEMMs via torch.mm on the same shapes (fwd, dgrad, "
                    "wgrad per linear; contiguous operands; no quantizers)",
            "ms_per_step": round(ms, 4), "tflops": round(flops / (ms * 1e-3) / 1e12, 1),
            "fp8_step_speedup": round(ms / ms_step, 3),
            "fp8_gemm_speedup": round(ms / fp8_gemm_ms, 3) if fp8_gemm_ms else None,
            "pages": "FP8 linear layers about 2x BF16; RL training step 1.41x, rollout 1.10-1.33x "
                     "(end-to-end, other hardware)"}


def fp8_library_context(torch, layers, fp8_gemm_ms, steps=10, warmup=3):
    """Context, not the product: the same twelve GEMMs as plain FP8 products
    through torch._scaled_mm (hipBLASLt), E4M3 operands with one scale per
    tensor (no per-block scaling, so no per-step fold), BF16 outputs, every
    operand in the layout the library wants (transposes made before timing).
    It shows what the vendor's FP8 GEMM reaches on these shapes on this GPU
    without block scales."""
    f8 = torch.float8_e4m3fn
    one = torch.ones((), dtype=torch.float32, device="cuda")
    ops, per = [], []
    try:
        for l in layers:
            x8 = l.x.to(f8)
            w8 = l.w.to(f8)
            dy8 = l.dy.mul(1000.0).to(f8)
            wT8 = w8.t().contiguous()
            dyT8 = dy8.t().contiguous()
            xT8 = x8.t().contiguous()
            trip = [(lambda a=x8, b=w8: torch._scaled_mm(a, b.t(), one, one, out_dtype=torch.bfloat16)),
                    (lambda a=dy8, b=wT8: torch._scaled_mm(a, b.t(), one, one, out_dtype=torch.bfloat16)),
                    (lambda a=dyT8, b=xT8: torch._scaled_mm(a, b.t(), one, one, out_dtype=torch.bfloat16))]
            ops += trip
            per.append((l.name, trip, l.flops))
        for _ in range(warmup):
            for f in ops:
                f()
        torch.cuda.synchronize()
    except Exception as e:   # a torch build without FP8 GEMMs for this GPU
        return {"kind": "third-party: hipBLASLt FP8 via torch._scaled_mm", "error": str(e)[:200]}
    E = torch.cuda.Event
    t0, t1 = E(enable_timing=True), E(enable_timing=True)
    t0.record()
    for _ in range(steps):
        for f in ops:
            f()
    t1.record()
    torch.cuda.synchronize()
    ms = t0.elapsed_time(t1) / steps
    layer_tflops = {}
    for name, trip, fl in per:
        a, b = E(enable_timing=True), E(enable_timing=True)
        a.record()
        for _ in range(steps):
            for f in trip:
                f()
        b.record()
        torch.cuda.synchronize()
        layer_tflops[name] = round(3 * fl * steps / (a.elapsed_time(b) * 1e-3) / 1e12, 1)
    flops = sum(3 * l.flops for l in layers)
    del ops, per
    torch.cuda.empty_cache()
    return {"kind": "third-party: hipBLASLt FP8 GEMMs via torch._scaled_mm on the same shapes (fwd, dgrad, "
                    "wgrad per linear; E4M3 operands with one scale per tensor, no block scaling; BF16 out)",
            "ms_per_step": round(ms, 4), "tflops": round(flops / (ms * 1e-3) / 1e12, 1),
            "tflops_per_layer": layer_tflops,
            "block_scaled_gemm_ratio": round(ms / fp8_gemm_ms, 3) if fp8_gemm_ms else None}


def copy_probe(torch):
    n = 1 << 30
    a = torch.empty(n, dtype=torch.uint8, device="cuda")
    b = torch.empty(n, dtype=torch.uint8, device="cuda")
    a.fill_(1)
    for _ in range(3):
        b.copy_(a)
    torch.cuda.synchronize()
    del a, b


PROBE_LIB = os.path.join(ROOT, "fp8_blockwise_quantized_amd", "lib", "libjetprobe.so")


def measured_ceilings(torch):
    """Ceilings measured on this GPU with the probes of include/jetprobe.h:
    streaming TB/s for the quantizers' read:write byte mixes over a 1 GiB
    source (past the 256 MB MALL; best of 5), the FP8 MFMA rate with
    register-resident operands, pure and with the per-step FP32 fold (best
    of 3), and the shader clock the MFMA probe ran at."""
    import ctypes
    if not os.path.exists(PROBE_LIB):
        raise RuntimeError(f"{PROBE_LIB} is not built; run `python -m fp8_blockwise_quantized_amd._build`")
    L = ctypes.CDLL(PROBE_LIB)
    vp, i64, i32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
    L.jet_probe_stream.argtypes = [vp, vp, i64, i32, i32, i32, vp]
    L.jet_probe_mfma.argtypes = [vp, vp, vp, i32, i32, i32, vp]
    st = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    E = torch.cuda.Event
    cus = int(L.jet_probe_cu_count()) or 256

    def timed(fn, reps):
        best = None
        for _ in range(reps):
            t0, t1 = E(enable_timing=True), E(enable_timing=True)
            t0.record()
            fn()
            t1.record()
            torch.cuda.synchronize()
            ms = t0.elapsed_time(t1)
            best = ms if best is None else min(best, ms)
        return best

    src = torch.empty(1 << 30, dtype=torch.uint8, device="cuda").fill_(0x3C)
    dst = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
    out = {}
    for name, lb, sb in (("copy_16r_16w", 16, 16), ("quant_16r_8w", 16, 8), ("swiglu_32r_8w", 32, 8),
                         ("read_16r", 16, 0)):
        units = (1 << 30) // lb

        def run(lb=lb, sb=sb, units=units):
            rc = L.jet_probe_stream(ctypes.c_void_p(src.data_ptr()), ctypes.c_void_p(dst.data_ptr()), units,
                                    lb, sb, 4 * cus, st)
            if rc:
                raise RuntimeError(f"jet_probe_stream failed ({rc})")
        run()
        ms = timed(run, 5)
        out[f"hbm_{name}_gbs"] = round(units * (lb + sb) / (ms * 1e-3) / 1e9, 1)
    del src, dst
    ops = torch.randint(-100, 100, (1025,), dtype=torch.int32, device="cuda")
    ops[1024] = 3
    res = torch.empty(cus * 512, dtype=torch.float32, device="cuda")
    clk = torch.zeros(2, dtype=torch.int64, device="cuda")
    iters = 1000
    for fold in (0, 1):
        def run(fold=fold):
            rc = L.jet_probe_mfma(ctypes.c_void_p(ops.data_ptr()), ctypes.c_void_p(res.data_ptr()),
                                  ctypes.c_void_p(clk.data_ptr()), iters, fold, cus, st)
            if rc:
                raise RuntimeError(f"jet_probe_mfma failed ({rc})")
        run()
        ms = timed(run, 3)
        flops = cus * 8 * iters * 32 * 2.0 * 16 * 16 * 128
        key = "mfma_fp8_fold" if fold else "mfma_fp8"
        out[f"{key}_tflops"] = round(flops / (ms * 1e-3) / 1e12, 1)
        c = clk.cpu().numpy()
        khz = int(L.jet_probe_wall_clock_khz())
        if c[1] > 0 and khz > 0:
            out[f"{key}_sclk_mhz"] = round(float(c[0]) / float(c[1]) * khz / 1e3, 0)
    # the GEMMs' K step on synthetic bytes, built up from its parts (one 8-wavefront block per CU)
    L.jet_probe_gemm_step.argtypes = [vp, vp, i32, i32, i32, vp]
    gsrc = torch.empty(cus * 262144, dtype=torch.uint8, device="cuda").fill_(0x3C)
    gout = torch.empty(cus * 512, dtype=torch.float32, device="cuda")
    steps = 512
    step = {}
    for name, parts in (("mfma", 0), ("lds", 1), ("lds_a_only", 17), ("pipe_l2", 3), ("fold", 4), ("pipe_l2_fold", 7),
                        ("pipe_mall", 11), ("pipe_mall_fold", 15)):
        def run(parts=parts):
            rc = L.jet_probe_gemm_step(ctypes.c_void_p(gsrc.data_ptr()), ctypes.c_void_p(gout.data_ptr()), steps,
                                       parts, cus, st)
            if rc:
                raise RuntimeError(f"jet_probe_gemm_step failed ({rc})")
        run()
        ms = timed(run, 3)
        step[f"{name}_tflops"] = round(cus * 8 * steps * 32 * 2.0 * 16 * 16 * 128 / (ms * 1e-3) / 1e12, 1)
    del gsrc, gout
    step["what"] = ("the GEMMs' K step (8 wavefronts of 128 x 64, two 64 KiB LDS stages, 32 MFMAs per "
                    "wavefront and step) on synthetic bytes: MFMA only; + the step's LDS fragment reads (or the A "
                    "fragments only); + the "
                    "pipeline (next stage's direct loads, their wait, one barrier); FP32 fold; with the loads "
                    "hitting L2 or all missing it (MALL); best of 3")
    out["gemm_step"] = step
    out["what"] = ("best of 5 (streams, 1 GiB source) / 3 (MFMA: the GEMMs' 8x4-fragment wave tile in "
                   "registers, one 8-wavefront block per CU) probe launches, with the shader clock wavefront 0 "
                   "saw; published peaks: 8000 GB/s HBM, 5000 TFLOP/s dense FP8 at 2.4 GHz")
    return out


def host_threads():
    """(host CPU count, BLAS threads NumPy runs with).  A cpu_baseline's
    `cores` is the threads its oracle run used: the BLAS threads where float64
    GEMMs dominate, 1 for the element-wise oracles; the host's CPU count is
    reported beside it."""
    try:
        from threadpoolctl import threadpool_info
        blas = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        blas = 1
    return os.cpu_count() or 1, int(blas)


def step_distribution(torch, step, n):
    """Per-step times (one event pair per step, no per-launch events) over n
    steps: median, min and max in ms."""
    E = torch.cuda.Event
    evs = [(E(enable_timing=True), E(enable_timing=True)) for _ in range(n)]
    torch.cuda.synchronize()
    for i in range(n):
        evs[i][0].record()
        step(i)
        evs[i][1].record()
    torch.cuda.synchronize()
    t = sorted(a.elapsed_time(b) for a, b in evs)
    return {"steps": n, "median_ms": round(t[n // 2] if n % 2 else 0.5 * (t[n // 2 - 1] + t[n // 2]), 4),
            "min_ms": round(t[0], 4), "max_ms": round(t[-1], 4)}


def cpu_baseline(pow2=False):
    """The oracle (untuned) on a bounded sample of the workload: the QKV
    linear (4096 -> 6144) with its full weight and all 8192 tokens (one of
    the four layers), through every step of the path; scaled to TFLOP/s of
    the sample's GEMMs.  pow2: with the power-of-two scale rule."""
    from oracle import jet_oracle as O
    from oracle import pow2_scales as P
    from fp8_blockwise_quantized_amd import inputs
    rule = P.scale_pair_pow2 if pow2 else None
    cores, blas = host_threads()
    Ms, N, K = M_TOKENS, 6144, 4096
    x = inputs.activations_with_outliers(Ms, K, seed=0)
    w = inputs.normal_bf16((N, K), 0.02, seed=0, tensor_id=inputs.ID_W)
    dy = inputs.normal_bf16((Ms, N), 1e-3, seed=0, tensor_id=inputs.ID_DY)
    t0 = time.perf_counter()
    wq, ws = O.quant_128x128(w, rule)
    xq, xs = O.quant_1x128(x, rule)
    y = O.bf16_rne(O.fl32(O.gemm_fwd(xq, xs, wq, ws)))
    O.quant_1x128(y, rule)
    dyq, dys = O.quant_1x128(dy, rule)
    O.gemm_dgrad(dyq, dys, wq, ws)
    dyqT, dysT = O.quant_128x1_T(dy, rule)
    xqT, xsT = O.requant_128x1_T_from_1x128(xq, xs, rule)
    O.gemm_wgrad(dyqT, dysT, xqT, xsT, Ms)
    dt = time.perf_counter() - t0
    flops = 3 * 2.0 * Ms * N * K
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": blas, "host_cpu_count": cores,
            "kind": "oracle", "seconds": round(dt, 3),
            "sample": f"QKV linear 4096->6144, full weight, {Ms} of {M_TOKENS} tokens, all path steps "
                      f"(weight/act quantizers, fwd+fused quant, dgrad, 128x1 quantizers, wgrad); NumPy "
                      f"element-wise steps on one thread, float64 BLAS on {blas}"}


QWEN_SAMPLE_TOKENS = 4096


def cpu_baseline_qwen():
    """The oracle (untuned) on a bounded sample of the Qwen workload: the QKV
    linear (5120 -> 7168) with its full weight and 4096 of the 16384 tokens,
    through every step of the path; TFLOP/s of the sample's GEMMs."""
    from oracle import jet_oracle as O
    from fp8_blockwise_quantized_amd import inputs
    cores, blas = host_threads()
    Ms, (_, N, K) = QWEN_SAMPLE_TOKENS, QWEN_LAYERS[0]
    x = inputs.activations_with_outliers(Ms, K, seed=0)
    w = inputs.normal_bf16((N, K), 0.02, seed=0, tensor_id=inputs.ID_W)
    dy = inputs.normal_bf16((Ms, N), 1e-3, seed=0, tensor_id=inputs.ID_DY)
    t0 = time.perf_counter()
    wq, ws = O.quant_128x128(w)
    xq, xs = O.quant_1x128(x)
    y = O.bf16_rne(O.fl32(O.gemm_fwd(xq, xs, wq, ws)))
    O.quant_1x128(y)
    dyq, dys = O.quant_1x128(dy)
    O.gemm_dgrad(dyq, dys, wq, ws)
    dyqT, dysT = O.quant_128x1_T(dy)
    xqT, xsT = O.requant_128x1_T_from_1x128(xq, xs)
    O.gemm_wgrad(dyqT, dysT, xqT, xsT, Ms)
    dt = time.perf_counter() - t0
    flops = 3 * 2.0 * Ms * N * K
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": blas, "host_cpu_count": cores,
            "kind": "oracle", "seconds": round(dt, 3),
            "sample": f"QKV linear 5120->7168, full weight, {Ms} of {QWEN_TOKENS} tokens, all path steps; "
                      f"NumPy element-wise steps on one thread, float64 BLAS on {blas}"}


MOE_SAMPLE_EXPERTS = 16


def cpu_baseline_moe():
    """The oracle (untuned) on a bounded sample of the MoE workload: the
    gate+up expert layer (2048 -> 1536) restricted to the first
    MOE_SAMPLE_EXPERTS experts' segments of the same routing (their full
    weights and routed rows), through every step of the path; scaled to
    TFLOP/s of the sample's GEMMs."""
    from oracle import jet_oracle as O
    from fp8_blockwise_quantized_amd import inputs
    cores, blas = host_threads()
    seg_all = moe_routing()
    E = MOE_SAMPLE_EXPERTS
    seg = seg_all[:E + 1].astype(np.int32)
    M = int(seg[-1])
    _, N, K = MOE_LAYERS[0]
    x = inputs.activations_with_outliers(M, K, seed=0)
    w = inputs.normal_bf16((E, N, K), 0.02, seed=0, tensor_id=inputs.ID_W)
    dy = inputs.normal_bf16((M, N), 1e-3, seed=0, tensor_id=inputs.ID_DY)
    t0 = time.perf_counter()
    wq = np.empty((E, N, K), np.uint8)
    ws = np.empty((E, N // 128, K // 128), np.float32)
    for e in range(E):
        wq[e], ws[e] = O.quant_128x128(w[e])
    xq, xs = O.quant_1x128(x)
    xqT, xsT = O.requant_128x1_T_grouped_from_1x128(xq, xs, seg)
    y = O.bf16_rne(O.fl32(O.gemm_grouped_fwd(xq, xs, wq, ws, seg)))
    O.quant_1x128(y)
    dyq, dys = O.quant_1x128(dy)
    O.gemm_grouped_dgrad(dyq, dys, wq, ws, seg)
    dyqT, dysT = O.quant_128x1_T_grouped(dy, seg)
    O.gemm_grouped_wgrad(dyqT, dysT, xqT, xsT, seg)
    dt = time.perf_counter() - t0
    flops = 3 * 2.0 * M * N * K
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": blas, "host_cpu_count": cores,
            "kind": "oracle", "seconds": round(dt, 3),
            "sample": f"gate+up expert layer 2048->1536, the first {E} of {MOE_EXPERTS} experts "
                      f"({M} of {int(seg_all[-1])} routed rows), full expert weights, all path steps "
                      f"(weight/act quantizers, grouped fwd+fused quant, dgrad, grouped 128x1 "
                      f"quantizers, wgrad); NumPy element-wise steps on one thread, float64 BLAS on {blas}"}


def counters_for(kernel: str, workload: str):
    """HBM bytes per launch of `kernel` from the workload's committed
    rocprofv3 FETCH_SIZE/WRITE_SIZE summary, or None if absent or taken on
    other kernel sources than the ones built now."""
    try:
        c = json.load(open(counters_path(workload)))
    except (OSError, ValueError):
        return None
    shas = c.get("sources_sha256") or {}
    if not shas:
        return None
    for f, h in shas.items():
        try:
            if hashlib.sha256(open(os.path.join(CSRC, f), "rb").read()).hexdigest() != h:
                return None
        except OSError:
            return None
    k = c.get("kernels", {}).get(kernel)
    return None if k is None else k.get("hbm_bytes_per_launch")


DECODE_M = 64


def decode_traffic(kernel, args):
    """HBM bytes per call of the decode forward `kernel` (fwd_<layer>: the
    weight-streaming kernel plus its finishing pass) from the committed
    counter summary of the same forward variant, or None."""
    variant, wl = (("pow2", "decode_pow2") if args.pow2 else ("batch_invariant", "decode_invariant")
                   if args.invariant else ("split_k", "decode"))
    return counters_for(f"{kernel}_{variant}", wl)
DECODE_COPIES = 4      # weight copies cycled per step: 4 x 218 MB exceeds the 256 MB MALL


MISMATCH_VOCAB, MISMATCH_ROW0 = 32768, 1000


def token_mult_prob_error(logits_train, logits_infer, ids):
    """The multiplicative probability error of the NeMo-RL FP8 page (section
    on numerical divergence): the mean over the scored tokens of
    exp(|log p_train - log p_infer|), each log-probability the log-softmax of
    its row's logits at the token's id (float64 on the host)."""
    def logp(z):
        zmax = z.max(axis=1, keepdims=True)
        return z[np.arange(z.shape[0]), ids] - (zmax[:, 0] + np.log(np.exp(z - zmax).sum(axis=1)))
    return float(np.mean(np.exp(np.abs(logp(logits_train) - logp(logits_infer)))))


def decode_mismatch(torch, J, pow2=False):
    """Train/rollout mismatch of the rollout forward that the decode line
    times, on synthetic logits: the Llama-3.1-8B down projection (14336 ->
    4096) computed for 64 rows inside a training batch of 8192 rows (the tiled
    forward) and as a 64-row rollout batch (split-K, batch-invariant, and
    power-of-two forwards); each BF16 output projected to logits by a fixed
    BF16 output projection (vocabulary 32768, N(0, 0.02^2)) in float64 on the
    host, the token of each row sampled from the rollout's logits (seeded
    Gumbel-max)."""
    from fp8_blockwise_quantized_amd import inputs
    N, K = 4096, 14336
    bf = lambda a: torch.from_numpy(a).to(torch.bfloat16).cuda()
    x = bf(inputs.activations_with_outliers(M_TOKENS, K, seed=21))
    w = bf(inputs.normal_bf16((N, K), 0.02, seed=21, tensor_id=inputs.ID_W))
    head = inputs.normal_bf16((MISMATCH_VOCAB, N), 0.02, seed=22, tensor_id=inputs.ID_W).astype(np.float64)
    rows = slice(MISMATCH_ROW0, MISMATCH_ROW0 + DECODE_M)
    logits = lambda y: y.float().cpu().numpy().astype(np.float64) @ head.T
    out = {}
    variants = ((("pow2", J.jet_quant_act_1x128_pow2, J.jet_quant_weight_128x128_pow2, J.jet_fp8_linear_fwd_pow2),)
                if pow2 else
                (("split_k", J.jet_quant_act_1x128, J.jet_quant_weight_128x128, J.jet_fp8_linear_fwd),
                 ("batch_invariant", J.jet_quant_act_1x128, J.jet_quant_weight_128x128,
                  J.jet_fp8_linear_fwd_batch_invariant)))
    for name, qa, qw, fwd in variants:
        xq, xs = qa(x)
        wq, ws, _ = qw(w, transposed=False)
        train_fwd = J.jet_fp8_linear_fwd_pow2 if pow2 else J.jet_fp8_linear_fwd
        y_train = train_fwd(xq, xs, wq, ws)
        y_roll = fwd(xq[rows].contiguous(), xs[:, rows].contiguous(), wq, ws)
        torch.cuda.synchronize()
        lr = logits(y_roll)
        ids = np.argmax(lr + np.random.default_rng(23).gumbel(size=lr.shape), axis=1)
        out[name] = token_mult_prob_error(logits(y_train[rows]), lr, ids)
    return {"token_mult_prob_error": out,
            "what": "rollout (M=64) vs training-batch (M=8192) forward of the same rows, Llama-3.1-8B down "
                    "projection, synthetic logits (BF16 output projection, vocabulary 32768); 1 = identical; "
                    "the page quotes 1.03-1.05 as the usual range"}


def cpu_baseline_decode():
    """The oracle (untuned) on the decode workload itself: the four linears'
    forward at M = 64 (1x128 quantization of X, the float64 GEMM from the
    dequantized operands, BF16 output and its fused 1x128 quantization), from
    codes made once; GB/s of weight bytes streamed, as the line's value."""
    from oracle import jet_oracle as O
    from fp8_blockwise_quantized_amd import inputs
    cores, blas = host_threads()
    qs = []
    for (name, N, K) in LAYERS:
        x = inputs.activations_with_outliers(DECODE_M, K, seed=0)
        w = inputs.normal_bf16((N, K), 0.02, seed=0, tensor_id=inputs.ID_W)
        qs.append((x, O.quant_128x128(w)))
    t0 = time.perf_counter()
    for x, (wq, ws) in qs:
        xq, xs = O.quant_1x128(x)
        y = O.bf16_rne(O.fl32(O.gemm_fwd(xq, xs, wq, ws)))
        O.quant_1x128(y)
    dt = time.perf_counter() - t0
    wbytes = sum(N * K + N * K // 16384 * 4 for (_, N, K) in LAYERS)
    return {"value": wbytes / dt / 1e9, "unit": "GB/s", "cores": blas, "host_cpu_count": cores,
            "kind": "oracle", "seconds": round(dt, 3),
            "sample": f"the whole decode step: the four linears' forward at M={DECODE_M} with the fused "
                      f"1x128 output (weights quantized beforehand, untimed); NumPy element-wise steps on "
                      f"one thread, float64 BLAS on {blas}"}


def decode_bench(args, torch, J, ceilings=None):
    """Rollout decode: forward of the four linears at M=64, one weight copy per
    step (cycling DECODE_COPIES copies, so weights stream from HBM), with the
    fused 1x128 output.  value = weight bytes streamed / time."""
    from fp8_blockwise_quantized_amd import inputs
    bf = lambda a: torch.from_numpy(a).to(torch.bfloat16).cuda()
    M = DECODE_M
    copies = []
    for c in range(DECODE_COPIES):
        layer = []
        for (name, N, K) in LAYERS:
            x = bf(inputs.activations_with_outliers(M, K, seed=c))
            w = bf(inputs.normal_bf16((N, K), 0.02, seed=c, tensor_id=inputs.ID_W))
            if args.pow2:
                xq, xs = J.jet_quant_act_1x128_pow2(x)
                wq, ws, _ = J.jet_quant_weight_128x128_pow2(w, transposed=False)
            else:
                xq, xs = J.jet_quant_act_1x128(x)
                wq, ws, _ = J.jet_quant_weight_128x128(w, transposed=False)
            del x, w
            y = torch.empty(M, N, dtype=torch.bfloat16, device="cuda")
            yq = torch.empty(M, N, dtype=torch.uint8, device="cuda")
            ys = torch.empty(N // 128, M, dtype=torch.float32, device="cuda")
            wsp = torch.empty(max(J.jet_workspace_bytes(J.JET_OP_FWD, M, N, K), 16), dtype=torch.uint8,
                              device="cuda")
            if args.pow2:
                fn = (lambda xq=xq, xs=xs, wq=wq, ws=ws, y=y, yq=yq, ys=ys:
                      J.jet_fp8_linear_fwd_pow2(xq, xs, wq, ws, y=y, fuse_quant=True, yq=yq, ys=ys))
            elif args.invariant:
                fn = (lambda xq=xq, xs=xs, wq=wq, ws=ws, y=y, yq=yq, ys=ys:
                      J.jet_fp8_linear_fwd_batch_invariant(xq, xs, wq, ws, y=y, fuse_quant=True, yq=yq, ys=ys))
            else:
                fn = (lambda xq=xq, xs=xs, wq=wq, ws=ws, y=y, yq=yq, ys=ys, wsp=wsp:
                      J.jet_fp8_linear_fwd(xq, xs, wq, ws, y=y, fuse_quant=True, yq=yq, ys=ys, workspace=wsp))
            layer.append((name, N, K, fn))
        copies.append(layer)
    torch.cuda.synchronize()
    E = torch.cuda.Event
    def step(s):
        for (_, _, _, fn) in copies[s % DECODE_COPIES]:
            fn()
    for s in range(args.warmup):
        step(s)
    torch.cuda.synchronize()
    # the timed steps run without per-call events (at ~10 us per call the host
    # cost of recording them would show); the per-layer breakdown comes from
    # back-to-back calls of each layer below
    t0, t1 = E(enable_timing=True), E(enable_timing=True)
    t0.record()
    for s in range(args.steps):
        step(s)
    t1.record()
    torch.cuda.synchronize()
    ms = t0.elapsed_time(t1) / args.steps
    dist = step_distribution(torch, step, max(args.steps, args.median_steps)) if args.median_steps else None
    # Per layer: args.steps back-to-back calls of that layer (one weight copy
    # after another, so still from HBM) between two events.  An event pair
    # around each call of the mixed step would also time the host's argument
    # checks whenever the GPU drains its queue between calls (10-40 us calls).
    wbytes = sum(N * K + N * K // 16384 * 4 for (_, N, K) in LAYERS)
    flops = sum(2.0 * M * N * K for (_, N, K) in LAYERS)
    kernels = {}
    if args.events:
        for i, (name, N, K) in enumerate(LAYERS):
            for c in range(DECODE_COPIES):
                copies[c][i][3]()
            a, b = E(enable_timing=True), E(enable_timing=True)
            torch.cuda.synchronize()
            a.record()
            for s in range(args.steps):
                copies[s % DECODE_COPIES][i][3]()
            b.record()
            torch.cuda.synchronize()
            us = a.elapsed_time(b) / args.steps * 1e3
            kernels[f"fwd_{name}"] = {"avg_us": round(us, 2), "weight_gbs": round((N * K) / (us * 1e-6) / 1e9, 1),
                                      "what": "back-to-back calls of the layer (weight-streaming kernel and, "
                                              "split-K, its finishing pass)"}
    dom = max(kernels, key=lambda k: kernels[k]["avg_us"]) if kernels else None
    out = {
        "metric": "FP8 linear decode forward weight-stream GB/s, Llama-8B shapes, M=64",
        "value": round(wbytes / (ms * 1e-3) / 1e9, 1), "unit": "GB/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "e4m3",
        "data": "synthetic",
        "config": {"workload": "Llama-3.1-8B decoder linears (QKV, O, gate+up, down) at rollout decode "
                               "batch M=64, forward with the fused 1x128 output, weights cycled over "
                               f"{DECODE_COPIES} copies", "M": M, "parallelism": "none (1 GPU)",
                   "forward": ("power-of-two scales (E8M0, applied by the MFMA), one K range" if args.pow2
                               else "batch-invariant (one K range)" if args.invariant else "split-K")},
        "tflops": round(flops / (ms * 1e-3) / 1e12, 1),
        "step_distribution": dist,
        "roofline": None if dom is None else {
            "bound": "hbm", "kernel": dom, "achieved": kernels[dom]["weight_gbs"], "peak": PEAK_HBM_GBS,
            "unit": "GB/s", "frac": round(kernels[dom]["weight_gbs"] / PEAK_HBM_GBS, 4),
            "traffic": decode_traffic(dom, args)},
        "kernels": kernels,
        "measured_ceilings": ceilings,
    }
    if not args.no_mismatch:
        log("token-mult-prob-error of the rollout forward against the training forward")
        out["mismatch"] = decode_mismatch(torch, J, pow2=args.pow2)
    if not args.no_cpu_baseline:
        log("timing the oracle on its bounded sample")
        out["cpu_baseline"] = cpu_baseline_decode()
    print(json.dumps(out), flush=True)


FUSED_H, FUSED_I, FUSED_EPS = 4096, 14336, 1e-5


def cpu_baseline_fused():
    """The oracle (untuned) on a bounded sample of the fused workload: 2048
    rows through RMSNorm + 1x128 (H=4096) and through SwiGLU + 1x128
    (I=14336); scaled to GB/s of the sample's algorithmic bytes."""
    from oracle import fused_producers as F
    from fp8_blockwise_quantized_amd import inputs
    rows = 2048
    x = inputs.activations_with_outliers(rows, FUSED_H, seed=0)
    g = inputs.normal_bf16((FUSED_H,), 0.1, seed=0, tensor_id=inputs.ID_W) + np.float32(1.0)
    gu = inputs.normal_bf16((rows, 2 * FUSED_I), 1.3, seed=0, tensor_id=inputs.ID_X)
    t0 = time.perf_counter()
    F.rmsnorm_quant_1x128(x, g, FUSED_EPS)
    F.swiglu_quant_1x128(gu, FUSED_I)
    dt = time.perf_counter() - t0
    nbytes = fused_bytes_rms(rows, FUSED_H) + fused_bytes_swiglu(rows, FUSED_I)
    cores, blas = host_threads()
    return {"value": nbytes / dt / 1e9, "unit": "GB/s", "cores": 1, "host_cpu_count": cores,
            "kind": "oracle", "seconds": round(dt, 3),
            "sample": f"{rows} rows: RMSNorm+1x128 at H={FUSED_H} and SwiGLU+1x128 at I={FUSED_I} "
                      f"(element-wise NumPy, one thread)"}


def fused_bytes_rms(M, H):      # x and gamma in; codes and scales out
    return M * H * 2 + H * 2 + M * H + M * H // 128 * 4


def fused_bytes_swiglu(M, I):   # gate and up in; codes and scales out
    return M * 2 * I * 2 + M * I + M * I // 128 * 4


def fused_bench(args, torch, J, ceilings=None):
    """Fused producers of one Llama-3.1-8B layer's linear inputs at M tokens:
    RMSNorm + 1x128 for the attention and MLP inputs (H=4096), SwiGLU + 1x128
    for the down projection's input (I=14336).  value = algorithmic bytes /
    time.  For context, the unfused sequence (torch's BF16 operator, then the
    1x128 quantizer) is timed on the same inputs."""
    from fp8_blockwise_quantized_amd import inputs
    M, H, I = args.fused_m, FUSED_H, FUSED_I
    bf = lambda a: torch.from_numpy(a).to(torch.bfloat16).cuda()
    log(f"building the fused-producer inputs (M={M})")
    xs = [bf(inputs.activations_with_outliers(M, H, seed=i)) for i in range(2)]
    gs = [bf(inputs.normal_bf16((H,), 0.1, seed=i, tensor_id=inputs.ID_W) + np.float32(1.0)) for i in range(2)]
    gu = bf(inputs.normal_bf16((M, 2 * I), 1.3, seed=0, tensor_id=inputs.ID_X))
    e = lambda shape, dt: torch.empty(shape, dtype=dt, device="cuda")
    qx = [e((M, H), torch.uint8) for _ in range(2)]
    sx = [e((H // 128, M), torch.float32) for _ in range(2)]
    qh, sh = e((M, I), torch.uint8), e((I // 128, M), torch.float32)
    plan = [("rmsnorm_quant_1x128", fused_bytes_rms(M, H),
             lambda i=i: J.jet_rmsnorm_quant_1x128(xs[i], gs[i], FUSED_EPS, q=qx[i], s=sx[i])) for i in range(2)]
    plan.append(("swiglu_quant_1x128", fused_bytes_swiglu(M, I),
                 lambda: J.jet_swiglu_quant_1x128(gu, q=qh, s=sh)))
    yb, hb = e((M, H), torch.bfloat16), e((M, I), torch.bfloat16)
    def unfused():
        for i in range(2):
            yb.copy_(torch.nn.functional.rms_norm(xs[i], (H,), weight=gs[i], eps=FUSED_EPS))
            J.jet_quant_act_1x128(yb, q=qx[i], s=sx[i])
        hb.copy_(torch.nn.functional.silu(gu[:, :I]) * gu[:, I:])
        J.jet_quant_act_1x128(hb, q=qh, s=sh)
    E = torch.cuda.Event
    def step(evs=None):
        for i, (_, _, fn) in enumerate(plan):
            if evs is not None:
                evs[i][0].record()
            fn()
            if evs is not None:
                evs[i][1].record()
    for _ in range(args.warmup):
        step()
        unfused()
    torch.cuda.synchronize()
    log(f"{args.warmup} warm-up steps, then {args.steps} timed steps")
    per = [[[E(enable_timing=True), E(enable_timing=True)] for _ in plan] for _ in range(args.steps)]
    t0, t1 = E(enable_timing=True), E(enable_timing=True)
    t0.record()
    for st in range(args.steps):
        step()
    t1.record()
    torch.cuda.synchronize()
    ms = t0.elapsed_time(t1) / args.steps
    if args.events:     # per-kernel times from a second pass with events
        for st in range(args.steps):
            step(per[st])
        torch.cuda.synchronize()
    u0, u1 = E(enable_timing=True), E(enable_timing=True)
    u0.record()
    for _ in range(args.steps):
        unfused()
    u1.record()
    torch.cuda.synchronize()
    ms_unfused = u0.elapsed_time(u1) / args.steps
    total = sum(b for (_, b, _) in plan)
    kernels = {}
    if args.events:
        for i, (kind, b, _) in enumerate(plan):
            us = sum(per[st][i][0].elapsed_time(per[st][i][1]) for st in range(args.steps)) / args.steps * 1e3
            k = kernels.setdefault(kind, {"avg_us": 0.0, "launches_per_step": 0, "bytes": 0})
            k["avg_us"] += us
            k["launches_per_step"] += 1
            k["bytes"] += b
        for k in kernels.values():
            k["gbs"] = round(k["bytes"] / (k["avg_us"] * 1e-6) / 1e9, 1)
            k["avg_us"] = round(k["avg_us"] / k["launches_per_step"], 2)
            k["frac_hbm_peak"] = round(k["gbs"] / PEAK_HBM_GBS, 4)
    dom = max(kernels, key=lambda k: kernels[k]["avg_us"] * kernels[k]["launches_per_step"]) if kernels else None
    out = {
        "metric": "Fused RMSNorm/SwiGLU + 1x128 FP8 producers GB/s, Llama-8B layer inputs",
        "value": round(total / (ms * 1e-3) / 1e9, 1), "unit": "GB/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": f"Llama-3.1-8B layer, M={M} tokens: RMSNorm+1x128 of the attention and "
                               f"MLP inputs (H={H}), SwiGLU+1x128 of the down projection's input "
                               f"(I={I}, from the fused gate+up output)", "M": M,
                   "parallelism": "none (1 GPU)"},
        "roofline": None if dom is None else {
            "bound": "hbm", "kernel": dom, "achieved": kernels[dom]["gbs"], "peak": PEAK_HBM_GBS,
            "unit": "GB/s", "frac": round(kernels[dom]["gbs"] / PEAK_HBM_GBS, 4),
            "traffic": counters_for(dom, "fused"),
            "bytes_per_launch": kernels[dom]["bytes"] // kernels[dom]["launches_per_step"]},
        "kernels": kernels,
        "measured_ceilings": ceilings,
        "unfused_context": {"ms_per_step": round(ms_unfused, 4),
                            "what": "torch BF16 rms_norm / silu*mul, then jet_quant_act_1x128",
                            "speedup_of_fused": round(ms_unfused / ms, 2)},
    }
    if not args.no_cpu_baseline:
        log("timing the oracle on its bounded sample")
        out["cpu_baseline"] = cpu_baseline_fused()
    print(json.dumps(out), flush=True)


KV_Q, KV_D, KV_T, KV_DECODE = 4096, 1024, 8192, 64


def kv_bytes_calibrate(T, D):     # K and V read
    return 2 * T * D * 2


def kv_bytes_append(T, D):        # K and V read, slots read, codes written
    return 2 * T * D * 2 + T * 8 + 2 * T * D


def cpu_baseline_kv():
    """The oracle (untuned) on the KV workload's prefill: all 8192 tokens
    recalibrated and appended (a few seconds); GB/s of its bytes."""
    from oracle import kv_cache as KV
    from fp8_blockwise_quantized_amd import inputs
    T = KV_T
    y = inputs.normal_bf16((T, KV_Q + 2 * KV_D), 1.3, seed=0, tensor_id=inputs.ID_X)
    k, v = y[:, KV_Q:KV_Q + KV_D], y[:, KV_Q + KV_D:]
    cache = np.zeros((T, KV_D), np.uint8)
    t0 = time.perf_counter()
    (sk, rk), (sv, rv) = KV.kv_calibrate(k, v)
    KV.kv_append(cache, k, np.arange(T), rk)
    KV.kv_append(cache, v, np.arange(T), rv)
    dt = time.perf_counter() - t0
    nbytes = kv_bytes_calibrate(T, KV_D) + kv_bytes_append(T, KV_D)
    cores, blas = host_threads()
    return {"value": nbytes / dt / 1e9, "unit": "GB/s", "cores": 1, "host_cpu_count": cores,
            "kind": "oracle", "seconds": round(dt, 3),
            "sample": f"the whole prefill, {T} tokens (D={KV_D}): recalibration and append of K and V "
                      f"(NumPy, one thread)"}


def kv_bench(args, torch, J, ceilings=None):
    """FP8 KV cache of one Llama-3.1-8B layer (8 KV heads x 128): after a
    weight update, recalibrate the K and V scales on a 8192-token prefill and
    append it; then append one 64-token decode step.  value = algorithmic
    bytes of recalibration + prefill append / their time."""
    from fp8_blockwise_quantized_amd import inputs
    log("building the KV-cache inputs")
    y = torch.from_numpy(inputs.normal_bf16((KV_T, KV_Q + 2 * KV_D), 1.3, seed=0,
                                            tensor_id=inputs.ID_X)).to(torch.bfloat16).cuda()
    k, v = y[:, KV_Q:KV_Q + KV_D], y[:, KV_Q + KV_D:]
    yd = y[:KV_DECODE]
    kd, vd = yd[:, KV_Q:KV_Q + KV_D], yd[:, KV_Q + KV_D:]
    rows = KV_T + 4096
    kc = torch.zeros((rows, KV_D), dtype=torch.uint8, device="cuda")
    vc = torch.zeros((rows, KV_D), dtype=torch.uint8, device="cuda")
    slots = torch.randperm(KV_T, device="cuda", generator=torch.Generator(device="cuda").manual_seed(0))
    slots_d = torch.arange(KV_T, KV_T + KV_DECODE, dtype=torch.int64, device="cuda")
    sc = torch.empty(6, dtype=torch.float32, device="cuda")
    plan = [("kv_calibrate", kv_bytes_calibrate(KV_T, KV_D), lambda: J.jet_kv_calibrate(k, v, kv_scales=sc)),
            ("kv_append_prefill", kv_bytes_append(KV_T, KV_D), lambda: J.jet_kv_append(k, v, slots, sc, kc, vc)),
            ("kv_append_decode", kv_bytes_append(KV_DECODE, KV_D),
             lambda: J.jet_kv_append(kd, vd, slots_d, sc, kc, vc))]
    E = torch.cuda.Event
    for _ in range(args.warmup):
        for _, _, fn in plan:
            fn()
    torch.cuda.synchronize()
    log(f"{args.warmup} warm-up steps, then {args.steps} timed steps")
    per = [[[E(enable_timing=True), E(enable_timing=True)] for _ in plan] for _ in range(args.steps)]
    t0, t1 = E(enable_timing=True), E(enable_timing=True)
    t0.record()
    for st in range(args.steps):
        for i, (_, _, fn) in enumerate(plan):
            per[st][i][0].record()
            fn()
            per[st][i][1].record()
    t1.record()
    torch.cuda.synchronize()
    ms = t0.elapsed_time(t1) / args.steps
    kernels = {}
    for i, (kind, b, _) in enumerate(plan):
        us = sum(per[st][i][0].elapsed_time(per[st][i][1]) for st in range(args.steps)) / args.steps * 1e3
        kernels[kind] = {"avg_us": round(us, 2), "bytes": b, "gbs": round(b / (us * 1e-6) / 1e9, 1),
                         "frac_hbm_peak": round(b / (us * 1e-6) / 1e9 / PEAK_HBM_GBS, 4)}
    main_bytes = kernels["kv_calibrate"]["bytes"] + kernels["kv_append_prefill"]["bytes"]
    main_us = kernels["kv_calibrate"]["avg_us"] + kernels["kv_append_prefill"]["avg_us"]
    dom = "kv_append_prefill"
    out = {
        "metric": "FP8 KV-cache recalibration + append GB/s, Llama-8B layer (8 KV heads x 128)",
        "value": round(main_bytes / (main_us * 1e-6) / 1e9, 1), "unit": "GB/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f32", "data": "synthetic",
        "config": {"workload": f"Llama-3.1-8B layer KV cache: per-tensor scale recalibration on a {KV_T}-token "
                               f"prefill and its append (K and V column slices of the QKV output, D={KV_D}), "
                               f"then a {KV_DECODE}-token decode append", "T": KV_T,
                   "parallelism": "none (1 GPU)"},
        "roofline": {"bound": "hbm", "kernel": dom, "achieved": kernels[dom]["gbs"], "peak": PEAK_HBM_GBS,
                     "unit": "GB/s", "frac": kernels[dom]["frac_hbm_peak"],
                     "traffic": counters_for(dom, "kv"), "bytes_per_launch": kernels[dom]["bytes"]},
        "kernels": kernels,
        "measured_ceilings": ceilings,
    }
    if not args.no_cpu_baseline:
        log("timing the oracle on its bounded sample")
        out["cpu_baseline"] = cpu_baseline_kv()
    print(json.dumps(out), flush=True)


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py: --gpus {args.gpus} is not supported: the benchmark measures exactly one GPU "
              f"(the path shards by tokens; a multi-GPU run is not part of it).", file=sys.stderr)
        sys.exit(2)
    import torch
    if not torch.cuda.is_available():
        print("bench.py: no GPU visible", file=sys.stderr)
        sys.exit(1)
    from fp8_blockwise_quantized_amd import jetfp8 as J

    ceilings = None
    if not args.no_ceilings:
        log("measuring the ceilings (streaming and MFMA probes)")
        ceilings = measured_ceilings(torch)
    if args.copy_probe:
        copy_probe(torch)
        torch.cuda.empty_cache()
    if args.workload == "decode":
        decode_bench(args, torch, J, ceilings)
        return
    if args.workload == "fused":
        fused_bench(args, torch, J, ceilings)
        return
    if args.workload == "kv":
        kv_bench(args, torch, J, ceilings)
        return
    moe = args.workload == "moe"
    qwen = args.workload == "qwen"
    log(f"building the {args.workload} inputs")
    if moe:
        seg = moe_routing()
        layers = [MoELayer(J, torch, n, N, K, seg, seed=0) for (n, N, K) in MOE_LAYERS]
        plan = [(l.name, kind, work, unit, fn) for l in layers for (kind, work, unit, fn) in l.ops(J, pow2=args.pow2)]
    else:
        shapes, tokens = (QWEN_LAYERS, QWEN_TOKENS) if qwen else (LAYERS, M_TOKENS)
        layers = [Layer(J, torch, n, N, K, tokens, seed=0) for (n, N, K) in shapes]
        plan = [(l.name, kind, work, unit, fn) for l in layers
                for (kind, work, unit, fn) in l.ops(J, separate=args.quant == "separate", pow2=args.pow2)]
    torch.cuda.synchronize()

    def step(evs=None):
        for i, (_, _, _, _, fn) in enumerate(plan):
            if evs is not None:
                evs[i][0].record()
            fn()
            if evs is not None:
                evs[i][1].record()

    log(f"{args.warmup} warm-up steps, then {args.steps} timed steps")
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    E = torch.cuda.Event
    # The timed steps run without per-launch events: recording two events
    # around each of the step's launches adds about 3 % to the step.  The
    # per-kernel breakdown (and the roofline) comes from a second pass of the
    # same number of steps with an event pair around every launch.
    per = [[[E(enable_timing=True), E(enable_timing=True)] for _ in plan] for _ in range(args.steps)]
    t_start, t_end = E(enable_timing=True), E(enable_timing=True)
    torch.cuda.synchronize()
    t_start.record()
    for s in range(args.steps):
        step()
    t_end.record()
    torch.cuda.synchronize()
    ms_step = t_start.elapsed_time(t_end) / args.steps
    log(f"{max(args.steps, 50)} more steps with one event pair per step (median step time)")
    dist = (step_distribution(torch, lambda i: step(), max(args.steps, args.median_steps))
            if args.median_steps else None)
    if args.events:
        log(f"{args.steps} steps with an event pair around every launch (per-kernel times)")
        for s in range(args.steps):
            step(per[s])
        torch.cuda.synchronize()

    # per-kernel-kind aggregates over the timed region
    agg = {}
    for s in range(args.steps):
        for i, (lname, kind, work, unit, _) in enumerate(plan):
            if not args.events:
                continue
            ms = per[s][i][0].elapsed_time(per[s][i][1])
            a = agg.setdefault(kind, {"ms": 0.0, "work": 0.0, "launches": 0, "unit": unit})
            a["ms"] += ms
            a["work"] += work
            a["launches"] += 1
    flops_step = sum(3 * l.flops for l in layers)
    value = flops_step / (ms_step * 1e-3) / 1e12

    kernels = {}
    for kind, a in agg.items():
        sec = a["ms"] * 1e-3
        rate = a["work"] / sec
        d = {"avg_us": round(a["ms"] / a["launches"] * 1e3, 2), "launches_per_step": a["launches"] // args.steps,
             "share_of_step": round(a["ms"] / args.steps / ms_step, 4)}
        if a["unit"] == "F":
            d.update(tflops=round(rate / 1e12, 1), frac_fp8_peak=round(rate / 1e12 / PEAK_FP8_TFLOPS, 4))
        else:
            d.update(gbs=round(rate / 1e9, 1), frac_hbm_peak=round(rate / 1e9 / PEAK_HBM_GBS, 4))
        kernels[kind] = d

    gemm_kinds = [k for k in agg if agg[k]["unit"] == "F"]
    roofline = None
    if gemm_kinds:
        # The dominant GEMM kind, priced against the roofline its arithmetic
        # intensity (FLOP per algorithmic byte) puts it under: MFMA above the
        # ridge (5.0 PF / 8 TB/s = 625 FLOP/B), HBM below it.
        dom = max(gemm_kinds, key=lambda k: agg[k]["ms"])
        a = agg[dom]
        sec = a["ms"] / a["launches"] * 1e-3
        flops = a["work"] / a["launches"]
        nbytes = sum(l.gemm_bytes(dom) for l in layers) / len(layers)
        intensity = flops / nbytes
        common = {"kernel": dom,
                  "traffic": counters_for(dom + ("_pow2" if args.pow2 and not (moe or qwen) else ""),
                                          "moe" if moe else "qwen" if qwen else "pow2" if args.pow2 else "train"),
                  "flops_per_launch": flops, "bytes_per_launch": nbytes,
                  "intensity_flop_per_byte": round(intensity, 1)}
        if intensity >= PEAK_FP8_TFLOPS * 1e12 / (PEAK_HBM_GBS * 1e9):
            achieved = flops / sec / 1e12
            roofline = {"bound": "mfma", "achieved": round(achieved, 1), "peak": PEAK_FP8_TFLOPS,
                        "unit": "TFLOP/s", "frac": round(achieved / PEAK_FP8_TFLOPS, 4), **common}
        else:
            achieved = nbytes / sec / 1e9
            roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBS,
                        "unit": "GB/s", "frac": round(achieved / PEAK_HBM_GBS, 4), **common}

    quant_bytes = sum(agg[k]["work"] for k in agg if agg[k]["unit"] == "B") / args.steps
    quant_ms = sum(agg[k]["ms"] for k in agg if agg[k]["unit"] == "B") / args.steps
    if moe:
        metric = "FP8 grouped MoE expert layers fwd+bwd TFLOP/s, Qwen3-30B-A3B shapes"
        config = {"workload": f"Qwen3-30B-A3B-shaped MoE expert layers (gate+up 2048->1536 and down "
                              f"768->2048 per expert), {MOE_EXPERTS} experts, top-{MOE_TOPK} of "
                              f"{MOE_TOKENS} tokens with Zipf({MOE_ALPHA}) expert load, grouped fwd + "
                              f"dgrad + wgrad with every quantizer and the weight re-quantization per step",
                  "routed_rows": int(seg[-1]), "experts": MOE_EXPERTS,
                  "largest_segment": int(np.diff(seg).max()), "smallest_segment": int(np.diff(seg).min()),
                  "scales": "power of two (E8M0, applied by the MFMA)" if args.pow2 else "FP32 amax/448",
                  "parallelism": "none (1 GPU)"}
    elif qwen:
        metric = "FP8 linear fwd+bwd TFLOP/s (% FP8 MFMA peak) + quantizer GB/s, Qwen-14B/32B shapes"
        config = {"workload": "Qwen-14B/32B-shaped linears (hidden 5120: QKV 5120->7168, O 5120->5120, "
                              "gate+up 5120->34816 and 5120->55296, down 17408->5120 and 27648->5120), "
                              f"training batch M={QWEN_TOKENS} tokens, fwd + dgrad + wgrad with every "
                              "quantizer and the BF16-master weight re-quantization per step",
                  "M": QWEN_TOKENS, "activation_quantizers": args.quant,
                  "scales": "power of two (E8M0, applied by the MFMA)" if args.pow2 else "FP32 amax/448",
                  "parallelism": "none (1 GPU)"}
    else:
        metric = METRIC
        config = {"workload": "Llama-3.1-8B decoder linears (QKV 4096->6144, O 4096->4096, "
                              "gate+up 4096->28672, down 14336->4096), training batch M=8192 tokens, "
                              "fwd + dgrad + wgrad with every quantizer and the BF16-master weight "
                              "re-quantization per step",
                  "M": M_TOKENS, "activation_quantizers": args.quant,
                  "scales": "power of two (E8M0, applied by the MFMA)" if args.pow2 else "FP32 amax/448",
                  "parallelism": "none (1 GPU)"}
    out = {
        "metric": metric, "value": round(value, 2), "unit": "TFLOP/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "e4m3",
        "data": "synthetic",
        "config": config,
        "frac_fp8_peak_step": round(value / PEAK_FP8_TFLOPS, 4),
        "step_distribution": dist,
        "quantizer_gbs_step": round(quant_bytes / (quant_ms * 1e-3) / 1e9, 1) if quant_ms else None,
        "roofline": roofline,
        "kernels": kernels,
        "measured_ceilings": ceilings,
    }
    if not moe and not args.no_bf16_context:
        log("timing hipBLASLt BF16 GEMMs on the same shapes (context)")
        gemm_ms = sum(agg[k]["ms"] for k in gemm_kinds) / args.steps if args.events else None
        out["bf16_context"] = bf16_context(torch, layers, ms_step, gemm_ms)
        log("timing hipBLASLt FP8 (tensor-wise scales) GEMMs on the same shapes (context)")
        out["fp8_library_context"] = fp8_library_context(torch, layers, gemm_ms)
    if not args.no_cpu_baseline:
        log("timing the oracle on its bounded sample")
        out["cpu_baseline"] = (cpu_baseline_moe() if moe else cpu_baseline_qwen() if qwen
                               else cpu_baseline(pow2=args.pow2))
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
