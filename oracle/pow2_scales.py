"""Plain CPU oracle for the power-of-two-scale variant of the FP8 linear layer.

TEST INFRASTRUCTURE ONLY. Imported by tests/, by __graft_entry__.smoke() and
by the cpu_baseline leg of bench.py, and by nothing else. The GPU library
never calls it and shares no code with it.

This variant is not on the pages.  The pages' group scale is an FP32 number
(jet_oracle, reading R2: s = amax/448, from the data, [JET-ZH] section 七).
gfx950's block-scaled MFMA takes its operand scales as 8-bit powers of two
(E8M0: 2^(b-127)), so when every group scale is a power of two the scales can
be applied inside the MFMA and the sum over the contraction steps can stay
there as well.  Readings for the variant:

R18 Group scale s = 2^e, e the smallest integer with 448 * 2^e >= amax_c,
    amax_c = max(max|x|, 2^-96) as in R2; quantization multiplier r = 2^-e
    (exactly 1/s).  Rounding the scale up to a power of two keeps every
    |x * r| <= 448 (nothing saturates) and puts the group's largest magnitude
    in (224, 448].  With the floor, e >= -104; for BF16 data e <= 120: every
    scale is an E8M0 value.
R19 All other steps as in jet_oracle: codes enc(fl32(x * r)) (R3; x * r is
    exact here unless it falls below FP32's subnormal range), the weight's
    128x128 blocks, the 128x1 re-quantization of the activations from their
    dequantized 1x128 values (R4; with power-of-two scales the dequantization
    is exact), the zero-padded token tail (R5), the expert segments of the
    grouped layer (R7), and the GEMM reference (R6):
    the float64 product of the exactly dequantized operands, so jet_oracle's
    GEMM functions apply unchanged.  The forward's fused output quantization
    is quant_1x128_pow2 of the BF16 output.
"""
from __future__ import annotations

import numpy as np

from oracle import jet_oracle as J

E8M0_BIAS = 127


def pow2_exponent(amax) -> np.ndarray:
    """R18: int64 e, the smallest integer with 448 * 2^e >= max(amax, 2^-96).

    A float64 estimate of log2(amax_c / 448), then exact comparisons (448 * 2^e
    and amax_c are both exact in float64) move it to the smallest such e.
    """
    a = np.maximum(np.asarray(amax, dtype=np.float32), J.AMAX_FLOOR).astype(np.float64)
    e = np.ceil(np.log2(a / J.E4M3_MAX)).astype(np.int64)
    for _ in range(3):
        e = np.where(J.E4M3_MAX * np.exp2(e.astype(np.float64)) < a, e + 1, e)
        e = np.where(J.E4M3_MAX * np.exp2((e - 1).astype(np.float64)) >= a, e - 1, e)
    return e


def scale_pair_pow2(amax) -> tuple[np.ndarray, np.ndarray]:
    """R18: (s, r) = (2^e, 2^-e) as float32 arrays."""
    e = pow2_exponent(amax).astype(np.float64)
    return np.exp2(e).astype(np.float32), np.exp2(-e).astype(np.float32)


def e8m0(scales) -> np.ndarray:
    """The E8M0 byte of each power-of-two scale: log2(s) + 127 (uint8)."""
    m, ex = np.frexp(np.asarray(scales, dtype=np.float64))
    if np.any(m != 0.5):
        raise ValueError("e8m0: a scale is not a power of two")
    return (ex - 1 + E8M0_BIAS).astype(np.uint8)


def quant_1x128_pow2(x):
    """R18-R19: 1x128 groups (activations, output gradients, the forward's
    fused output): codes [R, C] and scales [C/128, R]."""
    return J.quant_1x128(x, scale_rule=scale_pair_pow2)


def quant_128x128_pow2(w):
    """R18-R19: 128x128 weight blocks: codes [N, K] and scales [N/128, K/128]."""
    return J.quant_128x128(w, scale_rule=scale_pair_pow2)


def quant_128x1_T_pow2(a):
    """R18-R19: 128x1 groups along the token axis, transposed: codesT [C, Mp]
    and scales [ceil(M/128), C]."""
    return J.quant_128x1_T(a, scale_rule=scale_pair_pow2)


def requant_128x1_T_from_1x128_pow2(codes, scales):
    """R18-R19: the saved 1x128 activation re-quantized as 128x1 (transposed)."""
    return J.requant_128x1_T_from_1x128(codes, scales, scale_rule=scale_pair_pow2)


def quant_128x1_T_grouped_pow2(a, seg_off):
    """R18-R19 with R7: 128x1 groups restarting at each expert segment,
    in the padded transposed layout."""
    return J.quant_128x1_T_grouped(a, seg_off, scale_rule=scale_pair_pow2)


def requant_128x1_T_grouped_from_1x128_pow2(codes, scales, seg_off):
    """R18-R19 with R7: the grouped 128x1 re-quantization of the 1x128 activation."""
    return J.requant_128x1_T_grouped_from_1x128(codes, scales, seg_off, scale_rule=scale_pair_pow2)


def rmsnorm_quant_1x128_pow2(x, gamma, eps: float):
    """R12 + R14 with R18: the BF16 RMSNorm output and its power-of-two 1x128
    quantization."""
    from oracle.fused_producers import rmsnorm_bf16
    y = rmsnorm_bf16(x, gamma, eps)
    q, s = quant_1x128_pow2(y)
    return y, q, s


def swiglu_quant_1x128_pow2(gu, inter: int):
    """R13 + R14 with R18: the BF16 SwiGLU output and its power-of-two 1x128
    quantization."""
    from oracle.fused_producers import swiglu_bf16
    h = swiglu_bf16(gu, inter)
    q, s = quant_1x128_pow2(h)
    return h, q, s
