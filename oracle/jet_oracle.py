"""Plain CPU oracle for the unified-precision FP8 linear layer.

TEST INFRASTRUCTURE ONLY. This module is imported by tests/, by
__graft_entry__.smoke() and by the cpu_baseline leg of bench.py, and by
nothing else. The GPU library never calls it and shares no code with it.

It is deliberately slow and direct: each function restates one step of the
method in NumPy, with no blocking, fusion or reordering beyond what the
definition states, so that it can be checked against the pages by eye.

Sources, cited by page title and section:

[JET-DE]  "Jet-RL: Enabling On-Policy FP8 Reinforcement Learning with Unified
          Training and Rollout Precision Flow" (gist.science explainer of
          arXiv:2601.14243), section "Quantisierungsschema": linear layers
          (GEMMs) quantize activations per 1x128 group and weights per 128x128
          block; activations saved for backward are kept in FP8; gradients
          passed between operators stay BF16; DGrad and WGrad run in FP8, with
          1x128 and 128x1 groupings for WGrad.  Section "Kernarchitektur":
          BF16 master weights; the rollout graph is a subgraph of the training
          forward graph with the same granularity and precision.
[NV-RL]   "NVIDIA强化学习加速实操：10分钟提升2倍训练效率" (nmedialink.com
          repost of the NeMo-RL FP8 blog), quantization table in section
          "为什么FP8适配线性层？": weights E4M3 in [128,128] blocks, input
          activations and output gradients E4M3 in [1,128] groups, each with
          an FP32 block scale.
[JET-ZH]  "英伟达破解AI训练效率难题：让强化学习训练速度飞升40%的技术"
          (163.com write-up), section 五: forward = 1x128 input times 128x128
          weight; activations quantized 1x128 in forward are re-quantized as
          128x1 for backward; BF16 master copy of the weights.  Section 七:
          scales follow the data dynamically (no calibration).
[FP8-RL]  66260.cn news item on NVIDIA's FP8-RL, weight-synchronisation
          paragraph: updated parameters are re-converted to the compressed
          format on every weight sync, block-wise.
[OCP]     OCP 8-bit Floating Point Specification (OFP8), format E4M3: bias 7,
          subnormals, no infinities, NaN = S.1111.111, largest finite 448.
          The pages name the format only as "E4M3"; the +-448 range is the
          OCP E4M3 range.

Readings taken where the pages are silent:

R1  E4M3 is OCP E4M3FN ([OCP]); not the FNUZ variant (max 240).
R2  Scale per group: amax_c = max(max|x|, 2^-96); stored scale
    s = fl32(amax_c / 448) (the dequantisation multiplier); codes are
    enc(fl32(x * r)) with r = fl32(448 / amax_c).
R3  enc = round to nearest, ties to even, saturating at +-448; the sign of
    zero is kept; E4M3 subnormals are used; FP32 denormals are not flushed.
R4  WGrad contracts over tokens, so both of its operands are grouped 128x1
    along the token axis: X is re-quantized 128x1 from its saved FP8 1x128
    codes and scales, and dY (kept in BF16 between operators) is quantized
    a second time as 128x1.  Both are written transposed (token axis
    contiguous).
R5  A partial 128x1 group at the token tail uses only its valid rows; the
    transposed code rows are padded with zero codes up to a multiple of 128.
R6  GEMM reference = float64 product of the exactly dequantized operands;
    BF16 outputs are the round-to-nearest-even BF16 of the FP32 rounding of
    that product.
R7  Mixture-of-experts layers ([FP8-RL]: expert layers run in the compressed
    format; [NV-RL] section on the Qwen3-30B MoE experiment: the same FP8
    recipe on an MoE model).  The pages give no grouped layout, so: the rows
    routed to expert e form the contiguous segment seg_off[e]..seg_off[e+1]-1
    of the token matrix; every step of the dense layer applies to each
    segment with expert e's weights; 128x1 groups restart at each segment
    start; the transposed 128x1 outputs give segment e the column range
    starting at 128 * sum_{e'<e} ceil(len_e'/128), zero-padded to a multiple
    of 128 columns.  An empty segment contributes nothing (dW_e = 0).
"""
from __future__ import annotations

import numpy as np

GROUP = 128
E4M3_MAX = 448.0
AMAX_FLOOR = np.float32(2.0 ** -96)
_F32_448 = np.float32(448.0)


# ---------------------------------------------------------------------------
# E4M3 codec  ([OCP] E4M3; [NV-RL] table: all three tensors are E4M3)
# ---------------------------------------------------------------------------

def _build_decode_table() -> np.ndarray:
    """Value of each of the 256 E4M3 codes, as float64 (NaN for S.1111.111)."""
    t = np.empty(256, dtype=np.float64)
    for code in range(256):
        sign = -1.0 if code & 0x80 else 1.0
        e = (code >> 3) & 0xF
        m = code & 0x7
        if e == 0xF and m == 0x7:
            t[code] = np.nan
        elif e == 0:
            t[code] = sign * m * 2.0 ** -9          # subnormal: m/8 * 2^(1-7)
        else:
            t[code] = sign * (1.0 + m / 8.0) * 2.0 ** (e - 7)
    return t


DECODE = _build_decode_table()
# Non-negative finite codes 0x00..0x7E in increasing order of value.
_POS_VALUES = DECODE[:0x7F].copy()
assert np.all(np.diff(_POS_VALUES) > 0)


def e4m3_decode(codes: np.ndarray) -> np.ndarray:
    """E4M3 codes (uint8) -> float64 values."""
    return DECODE[np.asarray(codes, dtype=np.uint8)]


def e4m3_encode(v) -> np.ndarray:
    """Encode finite float32 values to E4M3 codes (reading R3).

    Round to nearest with ties to even, saturate to +-448, keep the sign of
    zero.  The spacing of E4M3 values below 2^-6 is 2^-9 (subnormals); in a
    binade [2^e, 2^(e+1)) it is 2^(e-3) (three mantissa bits).
    """
    v = np.asarray(v, dtype=np.float32)
    if not np.all(np.isfinite(v)):
        raise ValueError("e4m3_encode: input must be finite")
    a = np.minimum(np.abs(v.astype(np.float64)), E4M3_MAX)
    _, e = np.frexp(a)                       # a = f * 2^e, f in [0.5, 1)
    spacing_exp = np.where(a < 2.0 ** -6, -9, (e - 1) - 3)
    spacing = np.ldexp(1.0, spacing_exp.astype(np.int32))
    n = np.rint(a / spacing)                 # exact quotient; rint = ties-to-even
    value = n * spacing                      # exactly representable in E4M3
    idx = np.searchsorted(_POS_VALUES, value)
    if not np.all(_POS_VALUES[np.minimum(idx, 0x7E)] == value):
        raise AssertionError("e4m3_encode: rounded value not representable")
    code = idx.astype(np.uint8)
    code = code | (np.signbit(v).astype(np.uint8) << 7)
    return code.astype(np.uint8)


# ---------------------------------------------------------------------------
# Group scale  ([NV-RL] table: one FP32 scale per group/block;
#               [JET-ZH] 七: scales are dynamic, from the data; reading R2)
# ---------------------------------------------------------------------------

def scale_pair(amax) -> tuple[np.ndarray, np.ndarray]:
    """(stored scale s, quantize multiplier r) for float32 group maxima."""
    amax = np.asarray(amax, dtype=np.float32)
    amax_c = np.maximum(amax, AMAX_FLOOR)
    s = (amax_c / _F32_448).astype(np.float32)
    r = (_F32_448 / amax_c).astype(np.float32)
    return s, r


def _quantize_with(x32: np.ndarray, r32: np.ndarray) -> np.ndarray:
    """codes = enc(fl32(x * r)); x and r already broadcast to the same shape."""
    prod = (x32.astype(np.float32) * r32.astype(np.float32)).astype(np.float32)
    return e4m3_encode(prod)


# ---------------------------------------------------------------------------
# Quantizers
# ---------------------------------------------------------------------------

def quant_1x128(x, scale_rule=None) -> tuple[np.ndarray, np.ndarray]:
    """1x128 per-group quantization of an activation or output gradient.

    [JET-DE] Quantisierungsschema (activations 1x128); [NV-RL] table (input
    activations and output gradients [1,128], FP32 scale).

    x : [R, C] float32 holding BF16 values, C a multiple of 128.
    returns codes [R, C] uint8 and scales [C/128, R] float32, the scale of
    (row m, columns 128j..128j+127) at [j, m].  scale_rule (default
    scale_pair, reading R2) maps group maxima to (s, r).
    """
    scale_rule = scale_pair if scale_rule is None else scale_rule
    x = np.asarray(x, dtype=np.float32)
    R, C = x.shape
    if C % GROUP:
        raise ValueError("quant_1x128: columns must be a multiple of 128")
    groups = x.reshape(R, C // GROUP, GROUP)
    amax = np.max(np.abs(groups), axis=2) if R else np.zeros((0, C // GROUP), np.float32)
    s, r = scale_rule(amax)                              # [R, C/128]
    codes = _quantize_with(groups, np.broadcast_to(r[:, :, None], groups.shape))
    return codes.reshape(R, C), np.ascontiguousarray(s.T)


def quant_128x128(w, scale_rule=None) -> tuple[np.ndarray, np.ndarray]:
    """128x128 per-block quantization of a (BF16 master) weight.

    [JET-DE] Quantisierungsschema (weights 128x128); [NV-RL] table;
    [FP8-RL] weight sync re-converts the updated parameters block-wise.

    w : [N, K] float32 holding BF16 values, N and K multiples of 128.
    returns codes [N, K] uint8 and scales [N/128, K/128] float32.
    The transposed codes used by the data-gradient GEMM are codes.T.
    scale_rule as for quant_1x128.
    """
    scale_rule = scale_pair if scale_rule is None else scale_rule
    w = np.asarray(w, dtype=np.float32)
    N, K = w.shape
    if N % GROUP or K % GROUP:
        raise ValueError("quant_128x128: both dims must be multiples of 128")
    blocks = w.reshape(N // GROUP, GROUP, K // GROUP, GROUP)
    amax = np.max(np.abs(blocks), axis=(1, 3))          # [N/128, K/128]
    s, r = scale_rule(amax)
    codes = _quantize_with(blocks, np.broadcast_to(r[:, None, :, None], blocks.shape))
    return codes.reshape(N, K), s


def quant_128x1_T(a, scale_rule=None) -> tuple[np.ndarray, np.ndarray]:
    """128x1 per-group quantization along the row (token) axis, written transposed.

    [JET-DE] Quantisierungsschema (128x1 grouping for WGrad); [JET-ZH] 五
    (128x1 re-quantization for backward); readings R4, R5.

    a : [M, C] float32.  Groups are rows 128g..min(128g+127, M-1) of one
    column.  returns codesT [C, Mp] uint8 with Mp = ceil(M/128)*128 (columns
    M..Mp-1 hold zero codes) and scales [ceil(M/128), C] float32.
    scale_rule as for quant_1x128.
    """
    scale_rule = scale_pair if scale_rule is None else scale_rule
    a = np.asarray(a, dtype=np.float32)
    M, C = a.shape
    G = -(-M // GROUP)
    Mp = G * GROUP
    codesT = np.zeros((C, Mp), dtype=np.uint8)
    scales = np.empty((G, C), dtype=np.float32)
    for g in range(G):
        rows = a[g * GROUP: min((g + 1) * GROUP, M)]        # valid rows only (R5)
        amax = np.max(np.abs(rows), axis=0)                 # per column
        s, r = scale_rule(amax)
        scales[g] = s
        q = _quantize_with(rows, np.broadcast_to(r[None, :], rows.shape))
        codesT[:, g * GROUP: g * GROUP + rows.shape[0]] = q.T
    return codesT, scales


def dequant_1x128_fl32(codes, scales) -> np.ndarray:
    """fl32(D[q] * s) for 1x128 codes [R, C] with scales [C/128, R] (reading R4:
    the FP32 activation the 128x1 re-quantization starts from)."""
    vals = e4m3_decode(codes).astype(np.float32)
    s_full = np.repeat(np.asarray(scales, np.float32).T, GROUP, axis=1)   # [R, C]
    return (vals * s_full).astype(np.float32)


def requant_128x1_T_from_1x128(codes, scales, scale_rule=None) -> tuple[np.ndarray, np.ndarray]:
    """Re-quantize saved 1x128 FP8 activations into transposed 128x1 groups.

    [JET-ZH] 五: activations quantized 1x128 in forward are re-quantized
    128x1 for backward; [JET-DE]: activations saved for backward are FP8.
    """
    return quant_128x1_T(dequant_1x128_fl32(codes, scales), scale_rule)


# ---------------------------------------------------------------------------
# Exact dequantization (float64) and the three GEMMs  (reading R6)
# ---------------------------------------------------------------------------

def dequant_1x128(codes, scales) -> np.ndarray:
    """float64 D[q] * s for codes [R, C], scales [C/128, R] (exact)."""
    s_full = np.repeat(np.asarray(scales, np.float64).T, GROUP, axis=1)
    return e4m3_decode(codes) * s_full


def dequant_128x128(codes, scales) -> np.ndarray:
    """float64 D[q] * s for codes [N, K], scales [N/128, K/128] (exact)."""
    s_full = np.kron(np.asarray(scales, np.float64), np.ones((GROUP, GROUP)))
    return e4m3_decode(codes) * s_full


def dequant_128x1_T(codesT, scales, M) -> np.ndarray:
    """float64 [C, M] from transposed 128x1 codes [C, Mp] and scales [G, C]."""
    s_full = np.repeat(np.asarray(scales, np.float64), GROUP, axis=0)[:M].T   # [C, M]
    return e4m3_decode(np.asarray(codesT)[:, :M]) * s_full


def gemm_fwd(xq, xs, wq, ws) -> np.ndarray:
    """Forward Y = X W^T on dequantized operands, float64 [M, N].

    [JET-ZH] 五: 1x128 input times 128x128 weight; [JET-DE] Quantisierungsschema.
    """
    return dequant_1x128(xq, xs) @ dequant_128x128(wq, ws).T


def gemm_dgrad(dyq, dys, wq, ws) -> np.ndarray:
    """Data gradient dX = dY W on dequantized operands, float64 [M, K].

    [JET-DE] Quantisierungsschema (DGrad in FP8); [NV-RL] table (output
    gradients 1x128).  The weight is the forward's 128x128-quantized copy.
    """
    return dequant_1x128(dyq, dys) @ dequant_128x128(wq, ws)


def gemm_wgrad(dyqT, dysT, xqT, xsT, M) -> np.ndarray:
    """Weight gradient dW = dY^T X on dequantized operands, float64 [N, K].

    [JET-DE] Quantisierungsschema (WGrad in FP8 with 128x1 groupings);
    reading R4: both operands grouped 128x1 along the M tokens.
    """
    return dequant_128x1_T(dyqT, dysT, M) @ dequant_128x1_T(xqT, xsT, M).T


# ---------------------------------------------------------------------------
# Grouped (mixture-of-experts) layer, reading R7: the dense steps per segment
# ---------------------------------------------------------------------------

def segment_columns(seg_off) -> np.ndarray:
    """Start column of each segment in the transposed 128x1 layout, int64 [E+1]
    (entry E = the padded total)."""
    seg_off = np.asarray(seg_off, dtype=np.int64)
    lens = seg_off[1:] - seg_off[:-1]
    col = np.zeros(len(lens) + 1, dtype=np.int64)
    col[1:] = np.cumsum(-(-lens // GROUP) * GROUP)
    return col


def quant_128x1_T_grouped(a, seg_off, scale_rule=None) -> tuple[np.ndarray, np.ndarray]:
    """128x1 transposed quantization with groups restarting at each segment.

    a : [M, C] float32, seg_off : [E+1].  returns codesT [C, P] and scales
    [P/128, C], P = segment_columns(seg_off)[E]; segment e occupies columns
    col[e] .. col[e+1]-1 (its own quant_128x1_T output).  scale_rule as for
    quant_1x128.
    """
    a = np.asarray(a, dtype=np.float32)
    col = segment_columns(seg_off)
    C = a.shape[1]
    codesT = np.zeros((C, int(col[-1])), dtype=np.uint8)
    scales = np.zeros((int(col[-1]) // GROUP, C), dtype=np.float32)
    for e in range(len(col) - 1):
        lo, hi = int(seg_off[e]), int(seg_off[e + 1])
        if hi == lo:
            continue
        qT, sT = quant_128x1_T(a[lo:hi], scale_rule)
        codesT[:, col[e]:col[e + 1]] = qT
        scales[col[e] // GROUP: col[e + 1] // GROUP] = sT
    return codesT, scales


def requant_128x1_T_grouped_from_1x128(codes, scales, seg_off, scale_rule=None) -> tuple[np.ndarray, np.ndarray]:
    """Grouped form of requant_128x1_T_from_1x128 (readings R4, R7)."""
    return quant_128x1_T_grouped(dequant_1x128_fl32(codes, scales), seg_off, scale_rule)


def gemm_grouped_fwd(xq, xs, wq, ws, seg_off) -> np.ndarray:
    """Y rows of segment e = X_e W_e^T (float64 [M, N]); wq [E, N, K], ws [E, N/128, K/128]."""
    a = dequant_1x128(xq, xs)
    y = np.zeros((a.shape[0], wq.shape[1]))
    for e in range(wq.shape[0]):
        lo, hi = int(seg_off[e]), int(seg_off[e + 1])
        y[lo:hi] = a[lo:hi] @ dequant_128x128(wq[e], ws[e]).T
    return y


def gemm_grouped_dgrad(dyq, dys, wq, ws, seg_off) -> np.ndarray:
    """dX rows of segment e = dY_e W_e (float64 [M, K])."""
    a = dequant_1x128(dyq, dys)
    dx = np.zeros((a.shape[0], wq.shape[2]))
    for e in range(wq.shape[0]):
        lo, hi = int(seg_off[e]), int(seg_off[e + 1])
        dx[lo:hi] = a[lo:hi] @ dequant_128x128(wq[e], ws[e])
    return dx


def gemm_grouped_wgrad(dyqT, dysT, xqT, xsT, seg_off) -> np.ndarray:
    """dW_e = dY_e^T X_e (float64 [E, N, K]) from the grouped transposed operands."""
    col = segment_columns(seg_off)
    E = len(col) - 1
    dw = np.zeros((E, dyqT.shape[0], xqT.shape[0]))
    for e in range(E):
        n = int(seg_off[e + 1] - seg_off[e])
        if n == 0:
            continue
        c0, c1 = int(col[e]), int(col[e + 1])
        g0, g1 = c0 // GROUP, c1 // GROUP
        dw[e] = gemm_wgrad(dyqT[:, c0:c1], dysT[g0:g1], xqT[:, c0:c1], xsT[g0:g1], n)
    return dw


# ---------------------------------------------------------------------------
# Output roundings (reading R6)
# ---------------------------------------------------------------------------

def fl32(x) -> np.ndarray:
    return np.asarray(x, dtype=np.float64).astype(np.float32)


def bf16_rne(x) -> np.ndarray:
    """Round finite float32 values to BF16 (nearest, ties to even); the
    result is returned as float32 holding the BF16 value."""
    u = np.asarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    lsb = (u >> 16) & 1
    u = ((u + 0x7FFF + lsb) >> 16) << 16
    return u.astype(np.uint32).view(np.float32)


def bf16_bits(x) -> np.ndarray:
    """BF16 bit patterns (uint16) of float32 values that are BF16-representable."""
    u = np.asarray(x, dtype=np.float32).view(np.uint32)
    if np.any(u & 0xFFFF):
        raise ValueError("bf16_bits: value not representable in BF16")
    return (u >> 16).astype(np.uint16)


# ---------------------------------------------------------------------------
# Error bounds (used to pin the quantized GEMMs against unquantized products)
# ---------------------------------------------------------------------------

def _enc_half_spacing(a) -> np.ndarray:
    """Largest rounding error of enc at magnitude a (float64): half the E4M3
    spacing, at most a*2^-4 in a normal binade and 2^-10 in the subnormals."""
    a = np.asarray(a, np.float64)
    return np.where(a >= 2.0 ** -6, a * 2.0 ** -4, 2.0 ** -10)


def quant_error_bound(x, s_full) -> np.ndarray:
    """Per-element bound on |D[q]*s - x| for a value x quantized with scale s.

    x*r lies within 2^-24 relative of x/s; enc moves it by at most half an
    E4M3 spacing; s*r is within 2^-23 of 1.  Hence
    |D[q]*s - x| <= s * half_spacing(|x|/s * (1+2^-24)) + |x| * 2^-22.
    """
    x = np.abs(np.asarray(x, np.float64))
    s_full = np.asarray(s_full, np.float64)
    return s_full * _enc_half_spacing(x / s_full * (1 + 2.0 ** -24)) + x * 2.0 ** -22


def gemm_error_bound(a, ea, b, eb) -> np.ndarray:
    """Bound on |A^ B^T - A B^T| given |A^-A| <= ea and |B^-B| <= eb
    elementwise (float64 rounding slack included)."""
    a, b = np.abs(np.asarray(a, np.float64)), np.abs(np.asarray(b, np.float64))
    ea, eb = np.asarray(ea, np.float64), np.asarray(eb, np.float64)
    bound = ea @ b.T + a @ eb.T + ea @ eb.T
    k = a.shape[1]
    slack = 4.0 * k * 2.0 ** -53 * ((a + ea) @ (b + eb).T)
    return bound + slack
