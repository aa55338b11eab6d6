"""Plain CPU oracle for the fused producers of the 1x128-quantized input.

TEST INFRASTRUCTURE ONLY. Imported by tests/, by __graft_entry__.smoke() and
by the cpu_baseline leg of bench.py, and by nothing else. The GPU library
never calls it and shares no code with it.

Source: [JET-DE] "Jet-RL: Enabling On-Policy FP8 Reinforcement Learning with
Unified Training and Rollout Precision Flow" (gist.science explainer), section
"Implementierung": besides the FP8 GEMMs the system has its own kernels for
quantization, transposition and fused activation/RMSNorm operations; section
"Quantisierungsschema": activations are kept in FP8, quantized together with
the operator that produces them.  [JET-ZH] (163.com write-up), section 五:
every quantization can run fused with the computation before it.

The pages name the operators but give no formula, so the plainest readings,
those of the Llama decoder the pages' models use, are taken:

R12 RMSNorm of one token's hidden vector x (length H) with weight gamma:
    y = x / sqrt(mean(x^2) + eps) * gamma, computed exactly (float64) and
    rounded once: BF16 round-to-nearest-even of the FP32 rounding (the same
    output convention as the GEMMs, reading R6 of jet_oracle).
R13 The gated activation of the MLP (SwiGLU): the fused gate+up projection
    gives [M, 2I]; gate = columns 0..I-1, up = columns I..2I-1;
    h = silu(gate) * up with silu(g) = g / (1 + exp(-g)), computed exactly
    and rounded once as in R12.
R14 The fused producer's FP8 output is the 1x128 quantization (jet_oracle
    steps 3-5) of that BF16 tensor: fusing changes where the quantization
    runs, not what it computes.
"""
from __future__ import annotations

import numpy as np

from oracle.jet_oracle import bf16_rne, fl32, quant_1x128


def rmsnorm_bf16(x, gamma, eps: float) -> np.ndarray:
    """R12: BF16 RMSNorm of each row of x [M, H] (float32 holding BF16 values)
    with weight gamma [H]; float32 holding BF16 values out."""
    x64 = np.asarray(x, dtype=np.float64)
    g64 = np.asarray(gamma, dtype=np.float64)
    ms = np.mean(x64 * x64, axis=1, keepdims=True)
    y = x64 / np.sqrt(ms + float(eps)) * g64[None, :]
    return bf16_rne(fl32(y))


def silu(g) -> np.ndarray:
    """silu(g) = g / (1 + exp(-g)) in float64 (g -> -inf gives -0)."""
    g64 = np.asarray(g, dtype=np.float64)
    with np.errstate(over="ignore"):
        return g64 / (1.0 + np.exp(-g64))


def swiglu_bf16(gu, inter: int) -> np.ndarray:
    """R13: BF16 h = silu(gate) * up from the fused gate+up output gu [M, 2*inter]."""
    gu64 = np.asarray(gu, dtype=np.float64)
    if gu64.shape[1] < 2 * inter:
        raise ValueError("gu must hold gate and up: at least 2*inter columns")
    h = silu(gu64[:, :inter]) * gu64[:, inter:2 * inter]
    return bf16_rne(fl32(h))


def rmsnorm_quant_1x128(x, gamma, eps: float):
    """R12 + R14: (BF16 y, codes [M, H], scales [H/128, M])."""
    y = rmsnorm_bf16(x, gamma, eps)
    q, s = quant_1x128(y)
    return y, q, s


def swiglu_quant_1x128(gu, inter: int):
    """R13 + R14: (BF16 h, codes [M, inter], scales [inter/128, M])."""
    h = swiglu_bf16(gu, inter)
    q, s = quant_1x128(h)
    return h, q, s


def bf16_ulp(v) -> np.ndarray:
    """Spacing of BF16 values at magnitude |v| (float64): 2^(e-7) for
    |v| in [2^e, 2^(e+1)), and the subnormal spacing 2^-133 below 2^-126."""
    a = np.abs(np.asarray(v, dtype=np.float64))
    e = np.floor(np.log2(np.maximum(a, 2.0 ** -126)))
    return np.exp2(e - 7)
