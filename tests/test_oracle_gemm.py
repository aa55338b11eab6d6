"""Pins of the oracle's three block-scaled GEMMs (forward, data gradient,
weight gradient) to facts independent of its formulas:

* an exact special case: integer operands with a +-448 anchor in every
  group make every scale exactly 1 and every product exact, so each GEMM
  must equal the integer matrix product (numpy int64 matmul);
* brute force: the float64 product of the *unquantized* BF16 inputs lies
  within the propagated quantization error bound of the oracle's result,
  on inputs whose groups carry very different magnitudes (so a wrong scale
  index, a transposed operand or a dropped scale breaks the bound);
* linearity under 2^j (bit-exact);
* planted mistakes in copies of the GEMMs that these checks must reject.
"""
import numpy as np
import pytest

from oracle import jet_oracle as O
from fp8_blockwise_quantized_amd import inputs


def anchored_int(rng, rows, cols, group_axis):
    """Integers in [-16, 16] with +-448 on the diagonal rows == cols (mod 128),
    so every 1x128 group along `group_axis`=1, every 128x1 group along axis 0,
    and every 128x128 block holds a +-448."""
    v = rng.integers(-16, 17, size=(rows, cols)).astype(np.float32)
    r = np.arange(rows)[:, None]
    c = np.arange(cols)[None, :]
    diag = (r % 128) == (c % 128)
    v[diag] = np.where(rng.integers(0, 2, size=diag.sum()) == 1, 448.0, -448.0)
    return v


def graded(shape, seed, std, gsize=(1, 128)):
    """BF16 normals whose 128-groups are scaled by distinct powers of two."""
    x = inputs.normal_bf16(shape, std, seed, 1)
    rng = np.random.default_rng(seed + 100)
    gr, gc = gsize
    f = 2.0 ** rng.integers(-8, 9, size=(-(-shape[0] // gr), shape[1] // gc))
    f = np.repeat(np.repeat(f, gr, axis=0)[:shape[0]], gc, axis=1)
    return (x * f).astype(np.float32)


def fwd_case(M, N, K, seed):
    x = graded((M, K), seed, 1.0)
    w = graded((N, K), seed + 1, 0.02, (128, 128))
    return x, w


def check_fwd(gemm_fwd, quant1, quant_w):
    rng = np.random.default_rng(3)
    # exact integer case
    xi = anchored_int(rng, 256, 384, 1)
    wi = anchored_int(rng, 256, 384, 1)
    xq, xs = quant1(xi)
    wq, ws = quant_w(wi)
    exact = (xi.astype(np.int64) @ wi.astype(np.int64).T).astype(np.float64)
    assert np.array_equal(gemm_fwd(xq, xs, wq, ws), exact)
    # brute force bound
    for (M, N, K) in [(200, 256, 384), (64, 128, 512)]:
        x, w = fwd_case(M, N, K, 10 + M)
        xq, xs = quant1(x)
        wq, ws = quant_w(w)
        got = gemm_fwd(xq, xs, wq, ws)
        ex = np.repeat(np.asarray(xs, np.float64).T, 128, axis=1)
        ew = np.kron(np.asarray(ws, np.float64), np.ones((128, 128)))
        bound = O.gemm_error_bound(x, O.quant_error_bound(x, ex), w, O.quant_error_bound(w, ew))
        ref = x.astype(np.float64) @ w.astype(np.float64).T
        assert np.all(np.abs(got - ref) <= bound), "forward outside quantization bound"
    # linearity in 2^j
    y0 = gemm_fwd(xq, xs, wq, ws)
    xq2, xs2 = quant1((x * np.float32(8.0)).astype(np.float32))
    assert np.array_equal(gemm_fwd(xq2, xs2, wq, ws), 8.0 * y0)


def check_dgrad(gemm_dgrad, quant1, quant_w):
    rng = np.random.default_rng(4)
    dyi = anchored_int(rng, 256, 384, 1)        # [M, N]
    wi = anchored_int(rng, 384, 256, 1)         # [N, K]
    dq, ds = quant1(dyi)
    wq, ws = quant_w(wi)
    exact = (dyi.astype(np.int64) @ wi.astype(np.int64)).astype(np.float64)
    assert np.array_equal(gemm_dgrad(dq, ds, wq, ws), exact)
    M, N, K = 136, 256, 384
    dy = graded((M, N), 31, 1e-3)
    w = graded((N, K), 32, 0.02, (128, 128))
    dq, ds = quant1(dy)
    wq, ws = quant_w(w)
    got = gemm_dgrad(dq, ds, wq, ws)
    edy = O.quant_error_bound(dy, np.repeat(np.asarray(ds, np.float64).T, 128, axis=1))
    ew = O.quant_error_bound(w, np.kron(np.asarray(ws, np.float64), np.ones((128, 128))))
    bound = O.gemm_error_bound(dy, edy, w.T, ew.T)
    ref = dy.astype(np.float64) @ w.astype(np.float64)
    assert np.all(np.abs(got - ref) <= bound), "dgrad outside quantization bound"


def check_wgrad(gemm_wgrad, quant1, quantT):
    rng = np.random.default_rng(5)
    M = 256
    dyi = anchored_int(rng, M, 256, 0)          # [M, N]; 128x1 groups along M hold anchors
    xi = anchored_int(rng, M, 384, 0)           # [M, K]
    dqT, dsT = quantT(dyi)
    xqT, xsT = quantT(xi)
    exact = (dyi.astype(np.int64).T @ xi.astype(np.int64)).astype(np.float64)
    assert np.array_equal(gemm_wgrad(dqT, dsT, xqT, xsT, M), exact)
    # brute force, X through the 1x128 -> 128x1 re-quantization
    for M in (200, 256):
        N, K = 256, 384
        dy = graded((M, N), 41 + M, 1e-3, (128, 1))
        x = graded((M, K), 42 + M, 1.0, (128, 1))
        dqT, dsT = quantT(dy)
        xq, xs = quant1(x)
        a = O.dequant_1x128_fl32(xq, xs)
        xqT, xsT = quantT(a)
        got = gemm_wgrad(dqT, dsT, xqT, xsT, M)
        edy = O.quant_error_bound(dy.T, np.repeat(dsT, 128, axis=0)[:M].T)
        e1 = O.quant_error_bound(x, np.repeat(np.asarray(xs, np.float64).T, 128, axis=1))
        e2 = O.quant_error_bound(a, np.repeat(xsT, 128, axis=0)[:M]) + np.abs(a) * 2.0 ** -23
        bound = O.gemm_error_bound(dy.T, edy, x.T, (e1 + e2).T)
        ref = dy.astype(np.float64).T @ x.astype(np.float64)
        assert np.all(np.abs(got - ref) <= bound), "wgrad outside quantization bound"


def test_fwd_pins():
    check_fwd(O.gemm_fwd, O.quant_1x128, O.quant_128x128)


def test_dgrad_pins():
    check_dgrad(O.gemm_dgrad, O.quant_1x128, O.quant_128x128)


def test_wgrad_pins():
    check_wgrad(O.gemm_wgrad, O.quant_1x128, O.quant_128x1_T)


def test_bf16_rne_matches_library():
    import torch
    rng = np.random.default_rng(9)
    v = np.concatenate([rng.standard_normal(200_000).astype(np.float32) * 1e3,
                        rng.integers(0, 0x7F000000, 200_000, dtype=np.uint32).view(np.float32)])
    v = np.concatenate([v, -v])
    ref = torch.from_numpy(v).to(torch.bfloat16).to(torch.float32).numpy()
    assert np.array_equal(O.bf16_rne(v), ref)


# --- planted mistakes ------------------------------------------------------

def _mut_fwd(kind):
    def f(xq, xs, wq, ws):
        a = O.dequant_1x128(xq, xs)
        ws = np.asarray(ws, np.float64)
        if kind == "weight_block_rows_swapped":
            ws = ws[::-1]
        b = O.e4m3_decode(wq) * np.kron(ws, np.ones((128, 128)))
        if kind == "dropped_act_scale":
            a = O.e4m3_decode(xq)
        if kind == "weight_columns_reversed":
            return a @ b[:, ::-1].T
        return a @ b.T
    return f


def _mut_wgrad(kind):
    def f(dqT, dsT, xqT, xsT, M):
        a = O.dequant_128x1_T(dqT, dsT, M)
        b = O.dequant_128x1_T(xqT, xsT, M)
        if kind == "dy_scale_dropped":
            a = O.e4m3_decode(np.asarray(dqT)[:, :M])
        if kind == "scale_group_shift":
            sx = np.repeat(np.roll(np.asarray(xsT, np.float64), 1, axis=0), 128, axis=0)[:M].T
            b = O.e4m3_decode(np.asarray(xqT)[:, :M]) * sx
        return a @ b.T
    return f


@pytest.mark.parametrize("kind", ["weight_block_rows_swapped", "dropped_act_scale", "weight_columns_reversed"])
def test_fwd_pins_reject_planted_mistakes(kind):
    with pytest.raises(AssertionError):
        check_fwd(_mut_fwd(kind), O.quant_1x128, O.quant_128x128)


@pytest.mark.parametrize("kind", ["dy_scale_dropped", "scale_group_shift"])
def test_wgrad_pins_reject_planted_mistakes(kind):
    with pytest.raises(AssertionError):
        check_wgrad(_mut_wgrad(kind), O.quant_1x128, O.quant_128x1_T)
