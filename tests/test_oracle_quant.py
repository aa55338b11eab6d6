"""Pins of the oracle's quantizers (1x128, 128x128, 128x1 transposed, and the
128x1 re-quantization from saved FP8) to facts the pages and the mathematics
fix, independent of the oracle's own formulas:

* group shapes and scale dtypes from the pages' quantization table
  (tests/golden/nvrl_quant_table.txt);
* hand-worked groups; exact round trips of E4M3-representable groups whose
  amax is 448*2^j; scale invariance under 2^j; sign symmetry; permutation
  equivariance inside a group; group locality; tail == zero padding; the
  transpose relation between 1x128 and 128x1; block == row groups when every
  row group holds the block maximum; the per-element quantization error bound;
* planted mistakes in a copy of the oracle that these checks must reject.
"""
import os

import numpy as np
import pytest

from oracle import jet_oracle as O
from fp8_blockwise_quantized_amd import inputs

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "nvrl_quant_table.txt")


def load_table():
    rows = {}
    for line in open(GOLDEN):
        line = line.strip()
        if not line or line.startswith("#"):
            continue
        name, fmt, gr, gc, sdt, _src = line.split()
        rows[name] = (fmt, int(gr), int(gc), sdt)
    return rows


def rnd(shape, seed, std=1.0):
    return inputs.normal_bf16(shape, std, seed, 1)


# ---------------------------------------------------------------------------
def test_group_shapes_follow_pages_table():
    t = load_table()
    M, K, N = 256, 384, 256
    x = rnd((M, K), 0)
    q, s = O.quant_1x128(x)
    fmt, gr, gc, sdt = t["input_activation"]
    assert (fmt, sdt) == ("E4M3", "float32") and q.dtype == np.uint8 and s.dtype == np.float32
    assert q.shape == (M, K) and s.shape == (K // gc, M // gr)
    assert t["output_gradient"][1:3] == (1, 128)
    w = rnd((N, K), 1)
    qw, sw = O.quant_128x128(w)
    _, gr, gc, _ = t["weight"]
    assert qw.shape == (N, K) and sw.shape == (N // gr, K // gc)
    _, gr, gc, _ = t["wgrad_operand"]
    qt, st = O.quant_128x1_T(x)
    assert qt.shape == (K, M) and st.shape == (M // gr, K // gc)


def test_hand_examples():
    # E1: amax 448 -> s = 1, r = 1: codes are the plain encodings
    g = np.zeros((1, 128), np.float32)
    g[0, :4] = [448.0, 1.0, -0.5, -0.0]
    q, s = O.quant_1x128(g)
    assert s[0, 0] == 1.0
    assert list(q[0, :5]) == [0x7E, 0x38, 0xB0, 0x80, 0x00]
    # E2: amax 1 -> r = 448; 0.375*448 = 168 is a tie between 160 and 176 -> 160 (0x72);
    #     2^-12*448 = 0.109375 = 1.75*2^-4 -> biased exponent 3, mantissa 6 -> 0x1E
    g = np.zeros((1, 128), np.float32)
    g[0, :3] = [1.0, 0.375, 2.0 ** -12]
    q2, s2 = O.quant_1x128(g)
    assert s2[0, 0] == np.float32(1.0 / 448.0)
    assert list(q2[0, :3]) == [0x7E, 0x72, 0x1E]
    # E3: all-zero group: codes 0, scale = fl32(2^-96 / 448)
    q, s = O.quant_1x128(np.zeros((2, 128), np.float32))
    assert not q.any() and s[0, 0] == np.float32(2.0 ** -96) / np.float32(448.0)
    # E4: E2 * 2^10 -> same codes, scale * 2^10
    q4, s4 = O.quant_1x128(g * np.float32(1024.0))
    assert np.array_equal(q4, q2) and s4[0, 0] == np.float32(1024.0 / 448.0)


def representable_groups(rng, rows, j):
    """Rows of E4M3 values times 2^j, each row holding +-448*2^j somewhere."""
    codes = rng.integers(0, 0x7F, size=(rows, 128)).astype(np.uint8)
    codes |= (rng.integers(0, 2, size=(rows, 128)) << 7).astype(np.uint8)
    v = O.DECODE[codes]
    anchor = rng.integers(0, 128, size=rows)
    v[np.arange(rows), anchor] = np.where(rng.integers(0, 2, rows) == 1, 448.0, -448.0)
    return (v * 2.0 ** j).astype(np.float32)


def check_round_trip(quant1x128):
    rng = np.random.default_rng(7)
    for j in (-20, -3, 0, 5, 30):
        x = representable_groups(rng, 16, j).reshape(8, 256)
        q, s = quant1x128(x)
        assert np.all(s == np.float32(2.0 ** j)), "scale of a 448*2^j group must be 2^j"
        assert np.array_equal(O.dequant_1x128(q, s), x.astype(np.float64)), "lossless round trip"


def check_scale_invariance(quant1x128):
    x = rnd((64, 512), 3)
    q0, s0 = quant1x128(x)
    for j in (-13, -1, 1, 9):
        q1, s1 = quant1x128((x * np.float32(2.0 ** j)).astype(np.float32))
        assert np.array_equal(q0, q1)
        assert np.array_equal(s1, (s0 * np.float32(2.0 ** j)).astype(np.float32))


def check_structure(quant1x128):
    x = rnd((32, 512), 4)
    q, s = quant1x128(x)
    vals = O.e4m3_decode(q)
    assert np.all(np.isfinite(vals)) and np.all(np.abs(vals) <= 448.0)
    # the element holding the group maximum encodes to +-448
    g = np.abs(x.reshape(32, 4, 128))
    arg = np.argmax(g, axis=2)
    qq = q.reshape(32, 4, 128)
    at = np.take_along_axis(qq, arg[:, :, None], axis=2)[..., 0]
    assert np.all((at & 0x7F) == 0x7E)
    # sign symmetry
    qn, sn = quant1x128(-x)
    assert np.array_equal(sn, s) and np.array_equal(qn, q ^ 0x80)
    # permutation inside every group
    perm = np.random.default_rng(5).permutation(128)
    xp = x.reshape(32, 4, 128)[:, :, perm].reshape(32, 512)
    qp, sp = quant1x128(xp)
    assert np.array_equal(sp, s)
    assert np.array_equal(qp, q.reshape(32, 4, 128)[:, :, perm].reshape(32, 512))
    # group locality: changing one group leaves the others bit-identical
    x2 = x.copy()
    x2[5, 128:256] *= np.float32(3.0)
    q2, s2 = quant1x128(x2)
    mask = np.ones_like(q, bool)
    mask[5, 128:256] = False
    assert np.array_equal(q2[mask], q[mask])
    smask = np.ones_like(s, bool)
    smask[1, 5] = False
    assert np.array_equal(s2[smask], s[smask])
    # error bound per element
    s_full = np.repeat(s.T, 128, axis=1)
    err = np.abs(O.dequant_1x128(q, s) - x)
    assert np.all(err <= O.quant_error_bound(x, s_full))


def test_1x128_pins():
    check_round_trip(O.quant_1x128)
    check_scale_invariance(O.quant_1x128)
    check_structure(O.quant_1x128)


def test_quant_outlier_and_subnormal_groups():
    # BF16 subnormals and an amax below the 2^-96 floor still give finite scales
    x = np.zeros((4, 128), np.float32)
    x[0, :4] = inputs.to_bf16_values(np.float32([1e-39, -3e-40, 5e-41, 0.0]))
    x[1, :] = inputs.to_bf16_values(np.linspace(-1e-30, 1e-30, 128, dtype=np.float32))
    x[2, :] = 1e30
    x[3, 0] = -3.0e38
    q, s = O.quant_1x128(x)
    assert np.all(np.isfinite(s)) and np.all(s > 0)
    assert q[2, 0] == 0x7E and q[3, 0] == 0xFE
    assert np.all(np.abs(O.dequant_1x128(q, s) - x) <= O.quant_error_bound(x, np.repeat(s.T, 128, axis=1)))


def test_128x128_equals_row_groups_holding_block_max():
    rng = np.random.default_rng(11)
    N, K = 256, 384
    w = rnd((N, K), 12, std=0.02)
    # give every block a distinct magnitude so a wrong block index shows
    for bi in range(N // 128):
        for bj in range(K // 128):
            w[bi * 128:(bi + 1) * 128, bj * 128:(bj + 1) * 128] *= np.float32(2.0 ** rng.integers(-6, 7))
    # put the block maximum (same sign pattern irrelevant) into column 0 of each row group
    blocks = w.reshape(N // 128, 128, K // 128, 128)
    bmax = np.max(np.abs(blocks), axis=(1, 3))
    for bi in range(N // 128):
        for bj in range(K // 128):
            blocks[bi, :, bj, 0] = bmax[bi, bj]
    w = blocks.reshape(N, K)
    qb, sb = O.quant_128x128(w)
    qr, sr = O.quant_1x128(w)
    assert np.array_equal(qb, qr)
    assert np.array_equal(np.repeat(sb, 128, axis=0), sr.T)


def test_128x128_bound_and_round_trip():
    rng = np.random.default_rng(13)
    # [128, 256]: every row of both blocks holds +-448*2^-2, so each block amax is 112
    v = np.concatenate([representable_groups(rng, 128, -2) for _ in range(2)], axis=1)
    q, s = O.quant_128x128(v)
    assert np.all(s == np.float32(0.25))
    assert np.array_equal(O.dequant_128x128(q, s), v.astype(np.float64))
    w = rnd((256, 256), 14, std=0.02)
    q, s = O.quant_128x128(w)
    s_full = np.kron(s, np.ones((128, 128)))
    assert np.all(np.abs(O.dequant_128x128(q, s) - w) <= O.quant_error_bound(w, s_full))


@pytest.mark.parametrize("M", [1, 63, 128, 200, 256])
def test_128x1_T_is_1x128_of_transpose_and_tail_is_zero_padding(M):
    K = 256
    a = rnd((M, K), 20 + M)
    qT, sT = O.quant_128x1_T(a)
    G = -(-M // 128)
    Mp = G * 128
    assert qT.shape == (K, Mp) and sT.shape == (G, K)
    # zero padding of the tail group gives the same groups
    ap = np.zeros((Mp, K), np.float32)
    ap[:M] = a
    q1, s1 = O.quant_1x128(ap.T.copy())          # 1x128 of the transpose
    assert np.array_equal(qT, q1)
    assert np.array_equal(sT, s1)
    assert not qT[:, M:].any()
    # error bound
    s_full = np.repeat(sT, 128, axis=0)[:M].T
    assert np.all(np.abs(O.dequant_128x1_T(qT, sT, M) - a.T) <= O.quant_error_bound(a.T, s_full))


def test_requant_from_fp8_is_lossless_on_power_of_two_scales():
    # If the 1x128 scales are powers of two, fl32(D[q]*s) is exact, and the
    # 128x1 re-quantization equals the direct 128x1 quantization of those values.
    rng = np.random.default_rng(21)
    x = representable_groups(rng, 256, -1).reshape(256, 128)
    q, s = O.quant_1x128(x)
    a = O.dequant_1x128_fl32(q, s)
    assert np.array_equal(a, x)
    qT, sT = O.requant_128x1_T_from_1x128(q, s)
    qT2, sT2 = O.quant_128x1_T(x)
    assert np.array_equal(qT, qT2) and np.array_equal(sT, sT2)


def test_requant_error_bound_composes():
    M, K = 300, 256
    x = inputs.activations_with_outliers(M, K, seed=0)
    q, s = O.quant_1x128(x)
    a = O.dequant_1x128_fl32(q, s)
    e1 = O.quant_error_bound(x, np.repeat(s.T, 128, axis=1))
    qT, sT = O.requant_128x1_T_from_1x128(q, s)
    s2 = np.repeat(sT, 128, axis=0)[:M]
    e2 = O.quant_error_bound(a, s2) + np.abs(a) * 2.0 ** -23
    err = np.abs(O.dequant_128x1_T(qT, sT, M).T - x)
    assert np.all(err <= e1 + e2)


# --- planted mistakes ------------------------------------------------------

def _mut_1x128(kind):
    def quant(x):
        x = np.asarray(x, np.float32)
        R, C = x.shape
        g = x.reshape(R, C // 128, 128)
        amax = np.max(np.abs(g), axis=2)
        if kind == "max_not_abs":
            amax = np.max(g, axis=2)
        s, r = O.scale_pair(amax)
        if kind == "swap_s_r":
            s, r = r, s
        if kind == "divide_instead":
            v = (g / np.float32(448.0) * amax[:, :, None]).astype(np.float32)
        else:
            v = (g * r[:, :, None]).astype(np.float32)
        if kind == "e4m3_240":
            v = v * np.float32(240.0 / 448.0)
        q = O.e4m3_encode(v).reshape(R, C)
        st = s.T.copy()
        if kind == "scale_row_major":
            st = s.copy().reshape(st.shape)
        return q, st
    return quant


@pytest.mark.parametrize("kind", ["max_not_abs", "swap_s_r", "divide_instead", "e4m3_240",
                                  "scale_row_major"])
def test_quant_pins_reject_planted_mistakes(kind):
    mut = _mut_1x128(kind)
    failed = 0
    for check in (check_round_trip, check_scale_invariance, check_structure):
        try:
            check(mut)
        except (AssertionError, ValueError):
            failed += 1
    assert failed > 0, f"planted mistake {kind} went undetected"
