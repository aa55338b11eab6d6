"""Pins of the oracle's grouped (mixture-of-experts) functions, reading R7,
to facts independent of their own code:

* one segment covering every row reduces each grouped function to the dense
  one (pinned in test_oracle_quant.py / test_oracle_gemm.py);
* the transpose relation per segment: the grouped 128x1 output of segment e
  equals the 1x128 quantization of that segment's rows transposed, with the
  segment's rows zero-padded to a multiple of 128 (pinned dense 1x128);
* locality: changing one segment's rows leaves every other segment's codes
  and scales bit-identical; an empty segment owns no columns;
* an exact integer case: integer operands with a +-448 anchor in every group
  *of every segment* make every scale 1, so each grouped GEMM must equal the
  per-segment integer matrix products (numpy int64 matmul);
* expert relabelling: permuting the experts together with their segments
  permutes the outputs and nothing else;
* planted mistakes (groups not restarting at a segment, the neighbouring
  expert's weights, a segment bound off by one) that these checks reject.
"""
import numpy as np
import pytest

from oracle import jet_oracle as O
from fp8_blockwise_quantized_amd import inputs

GROUP = 128


def seg_from_lens(lens):
    off = np.zeros(len(lens) + 1, dtype=np.int32)
    off[1:] = np.cumsum(lens)
    return off


LENS = [5, 0, 200, 128, 1, 130]          # empty, short, ragged, exact and long segments


def rows(M, C, seed):
    return inputs.normal_bf16((M, C), 1.0, seed, inputs.ID_X)


def anchored_segments(rng, lens, cols):
    """Integers in [-16, 16] with +-448 anchors: inside each 128-row group of
    a segment (counted from the segment start; nr <= 128 rows), row r holds
    +-448 at the columns c with c % nr == r.  Every column then has one
    anchor in each 128x1 group and every row at least one in each 1x128
    group, so every scale is exactly 1 and every code equals its value."""
    out = []
    for n in lens:
        v = rng.integers(-16, 17, size=(n, cols)).astype(np.float32)
        for g0 in range(0, n, GROUP):
            nr = min(GROUP, n - g0)
            anchor = (np.arange(nr)[:, None]) == (np.arange(cols)[None, :] % nr)
            blk = v[g0:g0 + nr]
            blk[anchor] = np.where(rng.integers(0, 2, size=int(anchor.sum())) == 1, 448.0, -448.0)
        out.append(v)
    return np.concatenate(out, axis=0)


def anchored_weights(rng, E, N, K):
    w = rng.integers(-16, 17, size=(E, N, K)).astype(np.float32)
    diag = (np.arange(N)[:, None] % GROUP) == (np.arange(K)[None, :] % GROUP)
    for e in range(E):
        w[e][diag] = np.where(rng.integers(0, 2, size=int(diag.sum())) == 1, 448.0, -448.0)
    return w


# --- planted mistakes -------------------------------------------------------

def mutant_no_restart(a, seg_off):
    """Groups of 128 rows counted from row 0 of the whole matrix."""
    qT, sT = O.quant_128x1_T(a)
    col = O.segment_columns(seg_off)
    out_q = np.zeros((a.shape[1], int(col[-1])), np.uint8)
    out_s = np.zeros((int(col[-1]) // GROUP, a.shape[1]), np.float32)
    for e in range(len(seg_off) - 1):
        lo, hi = int(seg_off[e]), int(seg_off[e + 1])
        out_q[:, col[e]:col[e] + hi - lo] = qT[:, lo:hi]
        g = -(-(hi - lo) // GROUP)
        out_s[col[e] // GROUP: col[e] // GROUP + g] = sT[lo // GROUP: lo // GROUP + g]
    return out_q, out_s


def mutant_fwd_next_expert(xq, xs, wq, ws, seg_off):
    E = wq.shape[0]
    return O.gemm_grouped_fwd(xq, xs, wq[(np.arange(E) + 1) % E], ws[(np.arange(E) + 1) % E], seg_off)


def mutant_fwd_bound_shift(xq, xs, wq, ws, seg_off):
    off = np.array(seg_off, np.int64)
    off[1:-1] += 1
    return O.gemm_grouped_fwd(xq, xs, wq, ws, off)


# --- pins -------------------------------------------------------------------

def test_single_segment_reduces_to_dense():
    M, K, N = 300, 256, 256
    a = rows(M, K, 0)
    one = np.array([0, M], np.int32)
    qT, sT = O.quant_128x1_T_grouped(a, one)
    qd, sd = O.quant_128x1_T(a)
    assert np.array_equal(qT, qd) and np.array_equal(sT.view(np.uint32), sd.view(np.uint32))
    xq, xs = O.quant_1x128(a)
    w = inputs.normal_bf16((N, K), 0.02, 0, inputs.ID_W)
    wq, ws = O.quant_128x128(w)
    assert np.array_equal(O.gemm_grouped_fwd(xq, xs, wq[None], ws[None], one), O.gemm_fwd(xq, xs, wq, ws))
    dy = inputs.normal_bf16((M, N), 1e-3, 0, inputs.ID_DY)
    dyq, dys = O.quant_1x128(dy)
    assert np.array_equal(O.gemm_grouped_dgrad(dyq, dys, wq[None], ws[None], one),
                          O.gemm_dgrad(dyq, dys, wq, ws))
    dyqT, dysT = O.quant_128x1_T(dy)
    xqT, xsT = O.requant_128x1_T_from_1x128(xq, xs)
    gqT, gsT = O.requant_128x1_T_grouped_from_1x128(xq, xs, one)
    assert np.array_equal(gqT, xqT) and np.array_equal(gsT, xsT)
    assert np.array_equal(O.gemm_grouped_wgrad(dyqT, dysT, xqT, xsT, one)[0],
                          O.gemm_wgrad(dyqT, dysT, xqT, xsT, M))


def test_segment_transpose_relation():
    seg = seg_from_lens(LENS)
    a = rows(int(seg[-1]), 256, 1)
    qT, sT = O.quant_128x1_T_grouped(a, seg)
    col = O.segment_columns(seg)
    assert qT.shape == (256, int(col[-1]))
    for e in range(len(LENS)):
        lo, hi = int(seg[e]), int(seg[e + 1])
        assert col[e + 1] - col[e] == -(-(hi - lo) // GROUP) * GROUP
        if hi == lo:
            continue
        padded = np.zeros((col[e + 1] - col[e], 256), np.float32)
        padded[:hi - lo] = a[lo:hi]
        q1, s1 = O.quant_1x128(padded.T)              # 1x128 of the transposed, padded segment
        assert np.array_equal(qT[:, col[e]:col[e + 1]], q1)
        assert np.array_equal(sT[col[e] // GROUP: col[e + 1] // GROUP], s1)


def test_segment_locality_and_empty_segment():
    seg = seg_from_lens(LENS)
    a = rows(int(seg[-1]), 128, 2)
    b = a.copy()
    b[seg[2]:seg[3]] *= 3.0                            # change segment 2 only
    qa, sa = O.quant_128x1_T_grouped(a, seg)
    qb, sb = O.quant_128x1_T_grouped(b, seg)
    col = O.segment_columns(seg)
    for e in range(len(LENS)):
        sl = slice(col[e], col[e + 1])
        same = np.array_equal(qa[:, sl], qb[:, sl]) and np.array_equal(
            sa[col[e] // GROUP: col[e + 1] // GROUP], sb[col[e] // GROUP: col[e + 1] // GROUP])
        assert same == (e != 2) or LENS[e] == 0
    assert col[2] == col[1]                             # the empty segment owns no columns


def grouped_int_case(seed):
    rng = np.random.default_rng(seed)
    E, N, K = len(LENS), 256, 256
    seg = seg_from_lens(LENS)
    x = anchored_segments(rng, LENS, K)
    dy = anchored_segments(rng, LENS, N)
    w = anchored_weights(rng, E, N, K)
    return seg, x, dy, w


def test_grouped_gemms_integer_case():
    seg, x, dy, w = grouped_int_case(0)
    E = w.shape[0]
    xq, xs = O.quant_1x128(x)
    dyq, dys = O.quant_1x128(dy)
    wq = np.empty(w.shape, np.uint8)
    ws = np.empty((E, w.shape[1] // GROUP, w.shape[2] // GROUP), np.float32)
    for e in range(E):
        wq[e], ws[e] = O.quant_128x128(w[e])
    xqT, xsT = O.requant_128x1_T_grouped_from_1x128(xq, xs, seg)
    dyqT, dysT = O.quant_128x1_T_grouped(dy, seg)
    for arr in (xs, dys, ws, xsT, dysT):
        used = arr[arr != 0]
        assert np.all(used == 1.0)
    xi, dyi, wi = x.astype(np.int64), dy.astype(np.int64), w.astype(np.int64)
    y = O.gemm_grouped_fwd(xq, xs, wq, ws, seg)
    dx = O.gemm_grouped_dgrad(dyq, dys, wq, ws, seg)
    dw = O.gemm_grouped_wgrad(dyqT, dysT, xqT, xsT, seg)
    for e in range(E):
        lo, hi = int(seg[e]), int(seg[e + 1])
        assert np.array_equal(y[lo:hi], (xi[lo:hi] @ wi[e].T).astype(np.float64))
        assert np.array_equal(dx[lo:hi], (dyi[lo:hi] @ wi[e]).astype(np.float64))
        assert np.array_equal(dw[e], (dyi[lo:hi].T @ xi[lo:hi]).astype(np.float64))
    assert not dw[1].any()                              # empty segment


def test_expert_relabelling_permutes_outputs():
    seg, x, dy, w = grouped_int_case(1)
    E = w.shape[0]
    perm = np.array([3, 5, 0, 2, 1, 4])
    lens = np.diff(seg)
    seg_p = seg_from_lens(lens[perm])
    x_p = np.concatenate([x[seg[e]:seg[e + 1]] for e in perm])
    xq, xs = O.quant_1x128(x)
    xq_p, xs_p = O.quant_1x128(x_p)
    wq = np.empty(w.shape, np.uint8)
    ws = np.empty((E, 2, 2), np.float32)
    for e in range(E):
        wq[e], ws[e] = O.quant_128x128(w[e])
    y = O.gemm_grouped_fwd(xq, xs, wq, ws, seg)
    y_p = O.gemm_grouped_fwd(xq_p, xs_p, wq[perm], ws[perm], seg_p)
    assert np.array_equal(y_p, np.concatenate([y[seg[e]:seg[e + 1]] for e in perm]))


def test_planted_no_restart_rejected():
    seg = seg_from_lens(LENS)
    a = rows(int(seg[-1]), 256, 3)
    qT, sT = mutant_no_restart(a, seg)
    col = O.segment_columns(seg)
    bad = False
    for e in range(len(LENS)):
        lo, hi = int(seg[e]), int(seg[e + 1])
        if hi == lo:
            continue
        padded = np.zeros((col[e + 1] - col[e], 256), np.float32)
        padded[:hi - lo] = a[lo:hi]
        q1, s1 = O.quant_1x128(padded.T)
        bad |= not (np.array_equal(qT[:, col[e]:col[e + 1]], q1)
                    and np.array_equal(sT[col[e] // GROUP: col[e + 1] // GROUP], s1))
    assert bad


@pytest.mark.parametrize("mutant", [mutant_fwd_next_expert, mutant_fwd_bound_shift])
def test_planted_fwd_mistakes_rejected(mutant):
    seg, x, dy, w = grouped_int_case(2)
    E = w.shape[0]
    xq, xs = O.quant_1x128(x)
    wq = np.empty(w.shape, np.uint8)
    ws = np.empty((E, 2, 2), np.float32)
    for e in range(E):
        wq[e], ws[e] = O.quant_128x128(w[e])
    y = mutant(xq, xs, wq, ws, seg)
    xi, wi = x.astype(np.int64), w.astype(np.int64)
    ok = all(np.array_equal(y[int(seg[e]):int(seg[e + 1])],
                            (xi[int(seg[e]):int(seg[e + 1])] @ wi[e].T).astype(np.float64))
             for e in range(E))
    assert not ok
