"""Pins of the power-of-two-scale oracle (readings R18-R19 of
oracle/pow2_scales.py): hand-worked exponents and codes, closed forms at the
power-of-two boundaries, invariants the rounding-up of the scale implies, a
brute-force GEMM, and planted mistakes.  CPU only.

Hand-worked codes use the OCP E4M3 grid: in [256, 448] the spacing is 32
(256 = 0x78, 288 = 0x79, 384 = 0x7C, 448 = 0x7E); in [128, 256) it is 16
(192 = 0x74, 240 = 0x77); in [0.25, 0.5) it is 2^-5 (0.40625 = 0x2D);
1.0 = 0x38, 0.75 = 0x34, 0.5 = 0x30; the sign bit is 0x80.
"""
import math

import numpy as np
import pytest

from oracle import jet_oracle as J
from oracle import pow2_scales as P
from fp8_blockwise_quantized_amd import inputs


def test_hand_exponents():
    # 448 * 2^e >= amax, smallest e
    cases = {448.0: 0, 449.0: 1, 224.0: -1, 300.0: 0, 1000.0: 2, 100.0: -2, 1.0: -8, 1.75: -8,
             0.0: -104, 3.3895313892515355e38: 120}
    for a, e in cases.items():
        assert int(P.pow2_exponent(np.float32(a))) == e, a
    just_above = np.nextafter(np.float32(1.75), np.float32(2.0))
    assert int(P.pow2_exponent(just_above)) == -7
    # below the 2^-96 floor: 448 * 2^-104 = 1.75 * 2^-96 >= 2^-96 > 448 * 2^-105
    assert int(P.pow2_exponent(np.float32(2.0 ** -120))) == -104


def test_boundaries_closed_form():
    for j in range(-100, 111):
        a = np.float32(448.0 * 2.0 ** j)
        assert int(P.pow2_exponent(a)) == j
        assert int(P.pow2_exponent(np.nextafter(a, np.float32(np.inf)))) == j + 1
        assert int(P.pow2_exponent(np.nextafter(a, np.float32(0)))) == j
    s, r = P.scale_pair_pow2(np.array([448.0, 449.0, 0.0], np.float32))
    assert s.tolist() == [1.0, 2.0, 2.0 ** -104] and r.tolist() == [1.0, 0.5, 2.0 ** 104]
    assert P.e8m0(s).tolist() == [127, 128, 23]


def test_hand_codes_1x128_and_128x128():
    x = np.zeros((2, 128), np.float32)
    x[0, :3] = [300.0, 1.0, -0.5]           # amax 300 -> s = 1: the values' own codes
    x[1, :2] = [1000.0, 3.0]                # amax 1000 -> s = 4: 250 -> 256, 0.75
    q, s = P.quant_1x128_pow2(x)
    assert s.tolist() == [[1.0, 4.0]]
    assert q[0, :4].tolist() == [0x79, 0x38, 0xB0, 0x00]
    assert q[1, :3].tolist() == [0x78, 0x34, 0x00]
    w = np.zeros((128, 256), np.float32)
    w[5, 7], w[100, 3] = -1000.0, 3.0       # block (0, 0): amax 1000 -> s = 4
    w[0, 200] = 448.0                       # block (0, 1): s = 1
    wq, ws = P.quant_128x128_pow2(w)
    assert ws.tolist() == [[4.0, 1.0]]
    assert (wq[5, 7], wq[100, 3], wq[0, 200]) == (0xF8, 0x34, 0x7E)


def test_hand_codes_128x1_T():
    a = np.zeros((3, 128), np.float32)
    a[:, 0] = [100.0, -50.0, 0.1]           # amax 100 -> s = 1/4, r = 4: 400 -> 384 (tie to even),
    qT, sT = P.quant_128x1_T_pow2(a)        # -200 -> -192 (tie to even), 0.4 -> 0.40625
    assert qT.shape == (128, 128) and sT.shape == (1, 128)
    assert qT[0, :4].tolist() == [0x7C, 0xF4, 0x2D, 0x00]
    assert sT[0, 0] == 0.25 and sT[0, 1] == np.float32(2.0 ** -104)


@pytest.mark.parametrize("seed", [0, 1])
def test_invariants_of_rounding_the_scale_up(seed):
    x = inputs.activations_with_outliers(96, 512, seed=seed)
    q, s = P.quant_1x128_pow2(x)
    _, s_fp32 = J.quant_1x128(x)
    P.e8m0(s)                                          # every scale a power of two
    ratio = s.astype(np.float64) / s_fp32.astype(np.float64)
    assert np.all(ratio >= 1.0) and np.all(ratio <= 2.0)
    s_full = np.repeat(s.T, 128, axis=1)
    assert np.all(np.abs(x.astype(np.float64) / s_full) <= 448.0), "nothing saturates"
    mag = (q & 0x7F).reshape(96, 4, 128).max(axis=2)
    assert np.all((mag >= 0x76) & (mag <= 0x7E)), "group maximum in (224, 448] before rounding"
    # dequantization with a power-of-two scale is exact in FP32
    assert np.array_equal(J.dequant_1x128_fl32(q, s).astype(np.float64), J.dequant_1x128(q, s))
    assert np.all(np.abs(J.dequant_1x128(q, s) - x) <= J.quant_error_bound(x, s_full))
    # x * 2^j -> the same codes, scales * 2^j
    for j in (-20, 9):
        q2, s2 = P.quant_1x128_pow2(x * np.float32(2.0 ** j))
        assert np.array_equal(q2, q) and np.array_equal(s2, s * np.float32(2.0 ** j))


def test_requant_128x1_from_pow2_1x128():
    x = inputs.activations_with_outliers(200, 256, seed=3)
    q, s = P.quant_1x128_pow2(x)
    qT, sT = P.requant_128x1_T_from_1x128_pow2(q, s)
    # the re-quantized operand starts from the exact dequantized values
    ref_qT, ref_sT = P.quant_128x1_T_pow2(J.dequant_1x128(q, s).astype(np.float32))
    assert np.array_equal(qT, ref_qT) and np.array_equal(sT, ref_sT)
    assert qT.shape == (256, 256) and not np.any(qT[:, 200:])


def test_gemm_on_pow2_operands_brute_force():
    rng = np.random.default_rng(4)
    x = (rng.standard_normal((3, 256)) * 5).astype(np.float32)
    w = (rng.standard_normal((128, 256)) * 0.02).astype(np.float32)
    xq, xs = P.quant_1x128_pow2(x)
    wq, ws = P.quant_128x128_pow2(w)
    y = J.gemm_fwd(xq, xs, wq, ws)
    dv = J.e4m3_decode
    for m in range(3):
        for n in (0, 1, 77, 127):
            terms = [float(dv(xq[m, k])) * float(xs[k // 128, m]) * float(dv(wq[n, k])) * float(ws[0, k // 128])
                     for k in range(256)]
            want = math.fsum(terms)
            assert abs(y[m, n] - want) <= 1e-12 * math.fsum(abs(t) for t in terms) + 1e-300


# --- planted mistakes ----------------------------------------------------------

_EXP = P.pow2_exponent


def _exp_floor(amax):
    a = np.maximum(np.asarray(amax, np.float32), J.AMAX_FLOOR).astype(np.float64)
    return np.floor(np.log2(a / 448.0)).astype(np.int64)


def _exp_float32_log2(amax):
    a = np.maximum(np.asarray(amax, np.float32), J.AMAX_FLOOR)
    return np.ceil(np.log2(a / np.float32(448.0))).astype(np.int64)


def _exp_no_floor(amax):
    a = np.asarray(amax, np.float32).astype(np.float64)
    with np.errstate(divide="ignore"):
        return _EXP(a) + np.where(a == 0, 1, 0)


def _exp_off_by_one(amax):
    return _EXP(amax) + 1


_PINS = (test_hand_exponents, test_boundaries_closed_form, test_hand_codes_1x128_and_128x128,
         test_hand_codes_128x1_T)


@pytest.mark.parametrize("bad", [_exp_floor, _exp_float32_log2, _exp_no_floor, _exp_off_by_one])
def test_planted_exponent_mistakes_are_caught(bad, monkeypatch):
    monkeypatch.setattr(P, "pow2_exponent", bad)
    failed = 0
    for pin in _PINS:
        try:
            pin()
        except AssertionError:
            failed += 1
    assert failed >= 1, f"{bad.__name__} passed every pin"


def _pair_r_is_s(amax):
    e = _EXP(amax).astype(np.float64)
    return np.exp2(e).astype(np.float32), np.exp2(e).astype(np.float32)


def test_planted_multiplier_mistake_is_caught(monkeypatch):
    monkeypatch.setattr(P, "scale_pair_pow2", _pair_r_is_s)
    with pytest.raises(AssertionError):
        test_hand_codes_1x128_and_128x128()


def test_grouped_restarts_per_segment():
    """R7 with R18: the grouped 128x1 groups restart at every expert segment,
    each segment's columns equal to its own power-of-two 128x1 quantization."""
    lens = [5, 0, 200, 128, 1, 130]
    seg = np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)
    a = inputs.activations_with_outliers(int(seg[-1]), 256, seed=9)
    qT, sT = P.quant_128x1_T_grouped_pow2(a, seg)
    col = J.segment_columns(seg)
    for e in range(len(lens)):
        lo, hi = int(seg[e]), int(seg[e + 1])
        if hi == lo:
            assert col[e] == col[e + 1]
            continue
        q1, s1 = P.quant_128x1_T_pow2(a[lo:hi])
        assert np.array_equal(qT[:, col[e]:col[e + 1]], q1)
        assert np.array_equal(sT[col[e] // 128:col[e + 1] // 128], s1)
    P.e8m0(sT)
    xq, xs = P.quant_1x128_pow2(a)
    rq, rs = P.requant_128x1_T_grouped_from_1x128_pow2(xq, xs, seg)
    assert np.array_equal(rq, P.quant_128x1_T_grouped_pow2(J.dequant_1x128(xq, xs).astype(np.float32), seg)[0])


def test_fused_producers_compose():
    """R14 with R18: the fused producers' FP8 output is the power-of-two 1x128
    quantization of their BF16 output (hand case: RMSNorm of [3, 4, 0...] with
    gamma 1 has its maximum 4/sqrt(25/128) = 9.0509... in BF16 9.0625, so
    e = -5 (448 * 2^-6 = 7 < 9.0625 <= 14) and the code of 9.0625 * 32 = 290
    is 288 = 0x79)."""
    from oracle import fused_producers as F
    x = np.zeros((1, 128), np.float32)
    x[0, :2] = [3.0, 4.0]
    y, q, s = P.rmsnorm_quant_1x128_pow2(x, np.ones(128, np.float32), 0.0)
    assert y[0, 1] == np.float32(9.0625) and s[0, 0] == np.float32(2.0 ** -5)
    assert q[0, 1] == 0x79
    gu = inputs.normal_bf16((3, 256), 2.0, seed=1, tensor_id=inputs.ID_X)
    h, hq, hs = P.swiglu_quant_1x128_pow2(gu, 128)
    assert np.array_equal(h, F.swiglu_bf16(gu, 128))
    assert all(np.array_equal(a, b) for a, b in zip((hq, hs), P.quant_1x128_pow2(h)))
