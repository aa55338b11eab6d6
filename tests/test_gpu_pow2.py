"""GPU parity of the power-of-two-scale variant (oracle/pow2_scales.py,
readings R18-R19).  The _pow2 quantizers must match the oracle bit for bit.
The _pow2 GEMMs, which hand each scale to the MFMA as its E8M0 operand scale
and accumulate across K inside it, must meet the GEMM rules of gpu_helpers on
the GPU's own oracle-checked codes.  The integer case must be exact, and
the fused output quantization must be bit-exact against the GPU's own BF16 Y.
Rows, columns and weight blocks whose scales differ by large powers of two
check that each lane's scale reaches the rows it belongs to.
"""
import numpy as np
import pytest
import torch

from oracle import jet_oracle as O
from oracle import pow2_scales as P
from fp8_blockwise_quantized_amd import inputs
from tests.gpu_helpers import (assert_bits_equal, check_bf16_output, check_f32_output, dev_bf16,
                               edge_matrix, host, oracle_absprod)

pytestmark = pytest.mark.gpu


def quantize_all_pow2(J, x, w, dy, fused_quantizer=False):
    """GPU power-of-two quantization of one layer's tensors, checked bit-exact."""
    xd, wd, dyd = dev_bf16(x), dev_bf16(w), dev_bf16(dy)
    if fused_quantizer:
        xq, xs, xqT, xsT = J.jet_quant_act_1x128_128x1_T_pow2(xd, True)
        dyq, dys, dyqT, dysT = J.jet_quant_act_1x128_128x1_T_pow2(dyd, False)
    else:
        xq, xs = J.jet_quant_act_1x128_pow2(xd)
        dyq, dys = J.jet_quant_act_1x128_pow2(dyd)
        dyqT, dysT = J.jet_quant_act_128x1_T_pow2(dyd)
        xqT, xsT = J.jet_quant_act_128x1_T_pow2(xq, src_s=xs)
    wq, ws, wqT = J.jet_quant_weight_128x128_pow2(wd)
    torch.cuda.synchronize()
    ref = {}
    ref["xq"], ref["xs"] = P.quant_1x128_pow2(x)
    ref["wq"], ref["ws"] = P.quant_128x128_pow2(w)
    ref["dyq"], ref["dys"] = P.quant_1x128_pow2(dy)
    ref["dyqT"], ref["dysT"] = P.quant_128x1_T_pow2(dy)
    ref["xqT"], ref["xsT"] = P.requant_128x1_T_from_1x128_pow2(ref["xq"], ref["xs"])
    dev = dict(xq=xq, xs=xs, wq=wq, ws=ws, wqT=wqT, dyq=dyq, dys=dys, dyqT=dyqT, dysT=dysT,
               xqT=xqT, xsT=xsT)
    for k in ref:
        assert_bits_equal(host(dev[k]), ref[k], f"pow2 {k}")
    assert_bits_equal(host(wqT), ref["wq"].T, "pow2 wqT")
    return dev, ref


def layer_inputs(M, N, K, seed):
    x = inputs.activations_with_outliers(M, K, seed=seed)
    w = inputs.normal_bf16((N, K), 0.02, seed=seed, tensor_id=inputs.ID_W)
    dy = inputs.normal_bf16((M, N), 1e-3, seed=seed, tensor_id=inputs.ID_DY)
    return x, w, dy


def check_gemms(J, d, r, M, tag, out_f32=True):
    a_x = O.dequant_1x128(r["xq"], r["xs"])
    b_w = O.dequant_128x128(r["wq"], r["ws"])
    a_dy = O.dequant_1x128(r["dyq"], r["dys"])
    a_dyT = O.dequant_128x1_T(r["dyqT"], r["dysT"], M)
    a_xT = O.dequant_128x1_T(r["xqT"], r["xsT"], M)
    y16, yq, ys = J.jet_fp8_linear_fwd_pow2(d["xq"], d["xs"], d["wq"], d["ws"], fuse_quant=True)
    dx16 = J.jet_fp8_linear_dgrad_pow2(d["dyq"], d["dys"], d["wqT"], d["ws"])
    dw32 = J.jet_fp8_linear_wgrad_pow2(d["dyqT"], d["dysT"], d["xqT"], d["xsT"], M)
    torch.cuda.synchronize()
    y_ref, dx_ref, dw_ref = a_x @ b_w.T, a_dy @ b_w, a_dyT @ a_xT.T
    check_bf16_output(host(y16), y_ref, oracle_absprod(a_x, b_w), f"pow2 fwd bf16 {tag}")
    qo, so = P.quant_1x128_pow2(host(y16))
    assert_bits_equal(host(yq), qo, f"pow2 fused codes {tag}")
    assert_bits_equal(host(ys), so, f"pow2 fused scales {tag}")
    check_bf16_output(host(dx16), dx_ref, oracle_absprod(a_dy, b_w.T), f"pow2 dgrad bf16 {tag}")
    check_f32_output(host(dw32), dw_ref, oracle_absprod(a_dyT, a_xT), f"pow2 wgrad f32 {tag}")
    if out_f32:
        y32 = J.jet_fp8_linear_fwd_pow2(d["xq"], d["xs"], d["wq"], d["ws"], out_dtype=torch.float32)
        dx32 = J.jet_fp8_linear_dgrad_pow2(d["dyq"], d["dys"], d["wqT"], d["ws"], out_dtype=torch.float32)
        dw16 = J.jet_fp8_linear_wgrad_pow2(d["dyqT"], d["dysT"], d["xqT"], d["xsT"], M,
                                           out_dtype=torch.bfloat16)
        torch.cuda.synchronize()
        check_f32_output(host(y32), y_ref, oracle_absprod(a_x, b_w), f"pow2 fwd f32 {tag}")
        check_f32_output(host(dx32), dx_ref, oracle_absprod(a_dy, b_w.T), f"pow2 dgrad f32 {tag}")
        check_bf16_output(host(dw16), dw_ref, oracle_absprod(a_dyT, a_xT), f"pow2 wgrad bf16 {tag}")


def boundary_rows(K=512):
    """Groups whose maximum sits exactly on, or one BF16 step above, a
    power-of-two boundary 448 * 2^j (the scale's rounding-up decision)."""
    rng = np.random.default_rng(8)
    rows = []
    for j in (-100, -30, -7, 0, 5, 60, 119):
        for bump in (1.0, 450.0 / 448.0):                # 450 = next BF16 above 448
            v = inputs.to_bf16_values((rng.standard_normal(K) * 40.0).astype(np.float32))
            v = np.clip(v, -440, 440).astype(np.float32)
            for g in range(K // 128):
                v[g * 128 + (g * 53) % 128] = 448.0 * bump * (1 if g % 2 else -1)
            rows.append((v.astype(np.float64) * 2.0 ** j).astype(np.float32))
    return np.stack(rows)


def test_quantizers_edge_and_boundary_rows(gpu_lib):
    J = gpu_lib
    e = np.concatenate([edge_matrix(512), boundary_rows(512)])
    ed = dev_bf16(e)
    q, s = J.jet_quant_act_1x128_pow2(ed)
    qT, sT = J.jet_quant_act_128x1_T_pow2(ed)
    q2, s2, qT2, sT2 = J.jet_quant_act_1x128_128x1_T_pow2(ed, True)
    q3, s3, qT3, sT3 = J.jet_quant_act_1x128_128x1_T_pow2(ed, False)
    torch.cuda.synchronize()
    rq, rs = P.quant_1x128_pow2(e)
    assert_bits_equal(host(q), rq, "edge 1x128 codes")
    assert_bits_equal(host(s), rs, "edge 1x128 scales")
    tq, ts = P.quant_128x1_T_pow2(e)
    assert_bits_equal(host(qT), tq, "edge 128x1 codes")
    assert_bits_equal(host(sT), ts, "edge 128x1 scales")
    for a, b, c, dd, what, (wq, ws) in ((q2, s2, qT2, sT2, "requant", P.requant_128x1_T_from_1x128_pow2(rq, rs)),
                                        (q3, s3, qT3, sT3, "bf16", (tq, ts))):
        assert_bits_equal(host(a), rq, f"both groupings ({what}) 1x128 codes")
        assert_bits_equal(host(b), rs, f"both groupings ({what}) 1x128 scales")
        assert_bits_equal(host(c), wq, f"both groupings ({what}) 128x1 codes")
        assert_bits_equal(host(dd), ws, f"both groupings ({what}) 128x1 scales")
    # every scale is a power of two and the boundary groups land on both sides
    P.e8m0(host(s))
    assert {int(v) for v in P.e8m0(rs[:, len(edge_matrix(512)):]).ravel()} >= {27, 28, 127, 128, 246, 247}


def test_weight_quantizer_boundaries(gpu_lib):
    w = np.concatenate([boundary_rows(384)] * 10)[:128 * 1]          # 128 x 384: three blocks
    w = np.concatenate([w, inputs.normal_bf16((128, 384), 0.02, seed=4, tensor_id=inputs.ID_W)])
    q, s, qT = gpu_lib.jet_quant_weight_128x128_pow2(dev_bf16(w))
    torch.cuda.synchronize()
    rq, rs = P.quant_128x128_pow2(w)
    assert_bits_equal(host(q), rq, "weight codes")
    assert_bits_equal(host(s), rs, "weight scales")
    assert_bits_equal(host(qT), rq.T, "weight codes transposed")


@pytest.mark.parametrize("M,N,K", [(1, 128, 128), (64, 256, 384), (65, 384, 256), (200, 256, 512),
                                   (129, 128, 1024), (384, 640, 384)])
def test_ragged_shapes_all_gemms(gpu_lib, M, N, K):
    x, w, dy = layer_inputs(M, N, K, seed=M + 2 * N + K)
    d, r = quantize_all_pow2(gpu_lib, x, w, dy, fused_quantizer=(M % 2 == 1))
    check_gemms(gpu_lib, d, r, M, f"M={M} N={N} K={K}")


def test_ragged_big_tile_all_gemms(gpu_lib):
    """3969 x 3840 x 3968: the 256x256-tile kernel in every GEMM, ragged tail."""
    M, N, K = 3969, 3840, 3968
    x, w, dy = layer_inputs(M, N, K, 12)
    d, r = quantize_all_pow2(gpu_lib, x, w, dy, fused_quantizer=True)
    check_gemms(gpu_lib, d, r, M, "big tile", out_f32=False)


def anchored_small_int(rng, rows, cols):
    v = rng.integers(-7, 8, size=(rows, cols)).astype(np.float32)
    diag = (np.arange(rows)[:, None] % 128) == (np.arange(cols)[None, :] % 128)
    v[diag] = np.where(rng.integers(0, 2, size=int(diag.sum())) == 1, 7.0, -7.0)
    return v


@pytest.mark.parametrize("M,N,K", [(256, 384, 1024), (3968, 3840, 3968)])
def test_integer_case_bit_exact(gpu_lib, M, N, K):
    """Integers in [-7, 7] with a +-7 in every group: every power-of-two scale
    is 2^-6 (448 * 2^-6 = 7), every code exact, every sum an integer below
    2^24, so the MFMA's in-place accumulation must give the integer products
    exactly, in both tile configurations."""
    rng = np.random.default_rng(2)
    x, w, dy = anchored_small_int(rng, M, K), anchored_small_int(rng, N, K), anchored_small_int(rng, M, N)
    d, r = quantize_all_pow2(gpu_lib, x, w, dy)
    for key in ("xs", "ws", "dys", "dysT", "xsT"):
        assert np.all(r[key] == np.float32(2.0 ** -6))
    J = gpu_lib
    y = J.jet_fp8_linear_fwd_pow2(d["xq"], d["xs"], d["wq"], d["ws"], out_dtype=torch.float32)
    dx = J.jet_fp8_linear_dgrad_pow2(d["dyq"], d["dys"], d["wqT"], d["ws"], out_dtype=torch.float32)
    dw = J.jet_fp8_linear_wgrad_pow2(d["dyqT"], d["dysT"], d["xqT"], d["xsT"], M)
    torch.cuda.synchronize()
    xf, wf, dyf = x.astype(np.float64), w.astype(np.float64), dy.astype(np.float64)
    assert_bits_equal(host(y), (xf @ wf.T).astype(np.float32), "pow2 fwd integer")
    assert_bits_equal(host(dx), (dyf @ wf).astype(np.float32), "pow2 dgrad integer")
    assert_bits_equal(host(dw), (dyf.T @ xf).astype(np.float32), "pow2 wgrad integer")


def test_scales_reach_their_rows_and_columns(gpu_lib):
    """Row m of X and dY scaled by 2^(3*(m%7)-9), weight block (i, j) by
    2^(2*((i+3j)%5)-4), column n of dY and k of X (for WGrad) by further
    factors: scales differ by up to 2^18 between neighbouring rows, so a scale
    applied to the wrong row, column or block is off by powers of two."""
    M, N, K = 320, 384, 640
    x, w, dy = layer_inputs(M, N, K, 21)
    rf = np.exp2(3.0 * (np.arange(M) % 7) - 9.0)
    x = inputs.to_bf16_values((x * rf[:, None] * np.exp2((np.arange(K) % 5) - 2.0)[None, :]).astype(np.float32))
    dy = inputs.to_bf16_values((dy * rf[::-1, None] * np.exp2(2.0 * (np.arange(N) % 3) - 2.0)[None, :])
                               .astype(np.float32))
    bi, bj = np.arange(N)[:, None] // 128, np.arange(K)[None, :] // 128
    w = inputs.to_bf16_values((w * np.exp2(2.0 * ((bi + 3 * bj) % 5) - 4.0)).astype(np.float32))
    d, r = quantize_all_pow2(gpu_lib, x, w, dy)
    assert len(np.unique(r["xs"])) > 10 and len(np.unique(r["ws"])) >= 5
    check_gemms(gpu_lib, d, r, M, "scale mapping")


def test_wgrad_accumulate_and_empty_tokens(gpu_lib):
    M, N, K = 200, 256, 384
    x, w, dy = layer_inputs(M, N, K, 9)
    d, r = quantize_all_pow2(gpu_lib, x, w, dy)
    c0 = torch.randn(N, K, device="cuda")
    dw = c0.clone()
    gpu_lib.jet_fp8_linear_wgrad_pow2(d["dyqT"], d["dysT"], d["xqT"], d["xsT"], M, dw=dw, accumulate=True)
    z = torch.full((N, K), 7.0, device="cuda")
    gpu_lib.jet_fp8_linear_wgrad_pow2(d["dyqT"][:, :0], d["dysT"][:0], d["xqT"][:, :0], d["xsT"][:0], 0, dw=z)
    torch.cuda.synchronize()
    a_dyT = O.dequant_128x1_T(r["dyqT"], r["dysT"], M)
    a_xT = O.dequant_128x1_T(r["xqT"], r["xsT"], M)
    absprod = oracle_absprod(a_dyT, a_xT) + np.abs(host(c0))
    check_f32_output(host(dw), host(c0).astype(np.float64) + a_dyT @ a_xT.T, absprod, "pow2 wgrad accumulate")
    assert not host(z).any()


def test_forward_is_batch_invariant(gpu_lib):
    """The pow2 forward runs the tiled kernel at every M: a token's output row
    is bit-identical alone, in a decode batch and in a training batch."""
    N, K = 1024, 1536
    x = inputs.activations_with_outliers(1000, K, seed=6)
    w = inputs.normal_bf16((N, K), 0.02, seed=6, tensor_id=inputs.ID_W)
    J = gpu_lib
    xq, xs = J.jet_quant_act_1x128_pow2(dev_bf16(x))
    wq, ws, _ = J.jet_quant_weight_128x128_pow2(dev_bf16(w), transposed=False)
    full = J.jet_fp8_linear_fwd_pow2(xq, xs, wq, ws)
    part = J.jet_fp8_linear_fwd_pow2(xq[:64].contiguous(), xs[:, :64].contiguous(), wq, ws)
    one = J.jet_fp8_linear_fwd_pow2(xq[5:6].contiguous(), xs[:, 5:6].contiguous(), wq, ws)
    torch.cuda.synchronize()
    assert_bits_equal(host(part).view(np.uint32), host(full)[:64].view(np.uint32), "decode rows")
    assert_bits_equal(host(one).view(np.uint32), host(full)[5:6].view(np.uint32), "single row")


LLAMA = {"qkv": (6144, 4096), "down": (4096, 14336)}


@pytest.mark.parametrize("name", list(LLAMA))
def test_training_shapes_sampled(gpu_lib, name):
    """Llama-3.1-8B linears at M=8192: the step's pow2 quantizers and GEMMs at
    full size, checked on sampled rows and columns."""
    N, K = LLAMA[name]
    M = 8192
    x, w, dy = layer_inputs(M, N, K, 0)
    xd, wd, dyd = dev_bf16(x), dev_bf16(w), dev_bf16(dy)
    J = gpu_lib
    xq, xs, xqT, xsT = J.jet_quant_act_1x128_128x1_T_pow2(xd, True)
    dyq, dys, dyqT, dysT = J.jet_quant_act_1x128_128x1_T_pow2(dyd, False)
    wq, ws, wqT = J.jet_quant_weight_128x128_pow2(wd)
    y, yq, ys = J.jet_fp8_linear_fwd_pow2(xq, xs, wq, ws, fuse_quant=True)
    dx = J.jet_fp8_linear_dgrad_pow2(dyq, dys, wqT, ws)
    dw = J.jet_fp8_linear_wgrad_pow2(dyqT, dysT, xqT, xsT, M)
    torch.cuda.synchronize()
    del xd, wd, dyd
    rng = np.random.default_rng(7)
    rows = np.sort(rng.choice(M, 48, replace=False))
    ridx = torch.from_numpy(rows).cuda()
    qx, sx = P.quant_1x128_pow2(x[rows])
    assert_bits_equal(host(xq[ridx]), qx, "x codes")
    assert_bits_equal(host(xs[:, ridx]), sx, "x scales")
    qd, sd = P.quant_1x128_pow2(dy[rows])
    assert_bits_equal(host(dyq[ridx]), qd, "dy codes")
    g = int(rng.integers(0, M // 128))
    gs = slice(g * 128, g * 128 + 128)
    cq, cs = P.quant_1x128_pow2(x[gs])
    rq, rs = P.requant_128x1_T_from_1x128_pow2(cq, cs)
    assert_bits_equal(host(xqT[:, gs]), rq, "x 128x1 codes")
    assert_bits_equal(host(xsT[g]), rs[0], "x 128x1 scales")
    tq, ts = P.quant_128x1_T_pow2(dy[gs])
    assert_bits_equal(host(dyqT[:, gs]), tq, "dy 128x1 codes")
    assert_bits_equal(host(dysT[g]), ts[0], "dy 128x1 scales")
    wq_h, ws_h = host(wq), host(ws)
    wqo, wso = P.quant_128x128_pow2(w[:128])
    assert_bits_equal(wq_h[:128], wqo, "w codes, first block row")
    assert_bits_equal(ws_h[:1], wso, "w scales, first block row")
    del x, w, dy
    bw = O.dequant_128x128(wq_h, ws_h)
    ax = O.dequant_1x128(qx, sx)
    check_bf16_output(host(y[ridx]), ax @ bw.T, oracle_absprod(ax, bw), f"pow2 fwd {name}")
    qo, so = P.quant_1x128_pow2(host(y[ridx]))
    assert_bits_equal(host(yq[ridx]), qo, "fused codes")
    assert_bits_equal(host(ys[:, ridx]), so, "fused scales")
    ad = O.dequant_1x128(qd, sd)
    check_bf16_output(host(dx[ridx]), ad @ bw, oracle_absprod(ad, bw.T), f"pow2 dgrad {name}")
    del bw
    nrows = np.sort(rng.choice(N, 48, replace=False))
    nidx = torch.from_numpy(nrows).cuda()
    a = O.dequant_128x1_T(host(dyqT[nidx]), host(dysT[:, nidx]), M)
    b = O.dequant_128x1_T(host(xqT), host(xsT), M)
    check_f32_output(host(dw[nidx]), a @ b.T, oracle_absprod(a, b), f"pow2 wgrad {name}")


# --- grouped (mixture-of-experts) layer --------------------------------------

LENS = [5, 0, 200, 128, 1, 130, 0, 257]


def test_grouped_all_steps(gpu_lib):
    """Every step of the grouped layer with power-of-two scales: the dense
    _pow2 1x128 and stacked 128x128 quantizers, the grouped 128x1 quantizer
    (bit-exact on the padded layout), the grouped GEMMs per expert to the
    GEMM tolerance, the fused codes by composition, empty experts' dW zero."""
    J = gpu_lib
    seg = np.concatenate([[0], np.cumsum(LENS)]).astype(np.int32)
    E, N, K = len(LENS), 256, 384
    M = int(seg[-1])
    x = inputs.activations_with_outliers(M, K, seed=31)
    w = inputs.normal_bf16((E, N, K), 0.02, seed=31, tensor_id=inputs.ID_W)
    dy = inputs.normal_bf16((M, N), 1e-3, seed=31, tensor_id=inputs.ID_DY)
    segd = torch.from_numpy(seg).cuda()
    xq, xs = J.jet_quant_act_1x128_pow2(dev_bf16(x))
    dyq, dys = J.jet_quant_act_1x128_pow2(dev_bf16(dy))
    wq, ws, wqT = J.jet_quant_weight_128x128_pow2(dev_bf16(w.reshape(E * N, K)))
    dyqT, dysT = J.jet_quant_act_128x1_T_grouped_pow2(dev_bf16(dy), segd)
    xqT, xsT = J.jet_quant_act_128x1_T_grouped_pow2(xq, segd, src_s=xs)
    y16, yq, ys = J.jet_fp8_grouped_fwd_pow2(xq, xs, wq.view(E, N, K), ws.view(E, N // 128, K // 128), segd,
                                             fuse_quant=True)
    dx16 = J.jet_fp8_grouped_dgrad_pow2(dyq, dys, wqT, ws.view(E, N // 128, K // 128), segd)
    dw32 = J.jet_fp8_grouped_wgrad_pow2(dyqT, dysT, xqT, xsT, segd, M)
    torch.cuda.synchronize()
    rxq, rxs = P.quant_1x128_pow2(x)
    rdq, rds = P.quant_1x128_pow2(dy)
    assert_bits_equal(host(xq), rxq, "grouped x codes")
    assert_bits_equal(host(dys), rds, "grouped dy scales")
    rdqT, rdsT = P.quant_128x1_T_grouped_pow2(dy, seg)
    rxqT, rxsT = P.requant_128x1_T_grouped_from_1x128_pow2(rxq, rxs, seg)
    Pc = rdqT.shape[1]
    assert_bits_equal(host(dyqT)[:, :Pc], rdqT, "grouped dyqT")
    assert_bits_equal(host(dysT)[:Pc // 128], rdsT, "grouped dysT")
    assert_bits_equal(host(xqT)[:, :Pc], rxqT, "grouped xqT")
    assert_bits_equal(host(xsT)[:Pc // 128], rxsT, "grouped xsT")
    hwq, hws = host(wq).reshape(E, N, K), host(ws).reshape(E, N // 128, K // 128)
    y16h, dx16h, dw32h, yqh, ysh = host(y16), host(dx16), host(dw32), host(yq), host(ys)
    col = O.segment_columns(seg)
    for e in range(E):
        lo, hi = int(seg[e]), int(seg[e + 1])
        tag = f"pow2 expert {e} rows {lo}:{hi}"
        if hi == lo:
            assert not dw32h[e].any(), f"empty {tag}: dW must be zero"
            continue
        owq, ows = P.quant_128x128_pow2(w[e])
        assert_bits_equal(hwq[e], owq, f"w codes {tag}")
        assert_bits_equal(hws[e], ows, f"w scales {tag}")
        qo, so = P.quant_1x128_pow2(y16h[lo:hi])
        assert_bits_equal(yqh[lo:hi], qo, f"fused codes {tag}")
        assert_bits_equal(ysh[:, lo:hi], so, f"fused scales {tag}")
        a_x = O.dequant_1x128(rxq[lo:hi], rxs[:, lo:hi])
        a_dy = O.dequant_1x128(rdq[lo:hi], rds[:, lo:hi])
        b_w = O.dequant_128x128(owq, ows)
        check_bf16_output(y16h[lo:hi], a_x @ b_w.T, oracle_absprod(a_x, b_w), f"fwd {tag}")
        check_bf16_output(dx16h[lo:hi], a_dy @ b_w, oracle_absprod(a_dy, b_w.T), f"dgrad {tag}")
        c0, c1 = int(col[e]), int(col[e + 1])
        a_dyT = O.dequant_128x1_T(rdqT[:, c0:c1], rdsT[c0 // 128:c1 // 128], hi - lo)
        a_xT = O.dequant_128x1_T(rxqT[:, c0:c1], rxsT[c0 // 128:c1 // 128], hi - lo)
        check_f32_output(dw32h[e], a_dyT @ a_xT.T, oracle_absprod(a_dyT, a_xT), f"wgrad {tag}")


def test_grouped_single_expert_equals_dense(gpu_lib):
    """E = 1: the grouped _pow2 GEMMs give the dense _pow2 results bit for
    bit (every output element's MFMA chain is the same in either kernel)."""
    J = gpu_lib
    M, N, K = 300, 256, 256
    x = inputs.activations_with_outliers(M, K, seed=3)
    w = inputs.normal_bf16((N, K), 0.02, seed=3, tensor_id=inputs.ID_W)
    dy = inputs.normal_bf16((M, N), 1e-3, seed=3, tensor_id=inputs.ID_DY)
    seg = torch.tensor([0, M], dtype=torch.int32, device="cuda")
    xq, xs = J.jet_quant_act_1x128_pow2(dev_bf16(x))
    dyq, dys = J.jet_quant_act_1x128_pow2(dev_bf16(dy))
    wq, ws, wqT = J.jet_quant_weight_128x128_pow2(dev_bf16(w))
    dyqT_g, dysT_g = J.jet_quant_act_128x1_T_grouped_pow2(dev_bf16(dy), seg)
    xqT_g, xsT_g = J.jet_quant_act_128x1_T_grouped_pow2(xq, seg, src_s=xs)
    y_g = J.jet_fp8_grouped_fwd_pow2(xq, xs, wq[None], ws[None], seg, out_dtype=torch.float32)
    y_d = J.jet_fp8_linear_fwd_pow2(xq, xs, wq, ws, out_dtype=torch.float32)
    dx_g = J.jet_fp8_grouped_dgrad_pow2(dyq, dys, wqT, ws[None], seg, out_dtype=torch.float32)
    dx_d = J.jet_fp8_linear_dgrad_pow2(dyq, dys, wqT, ws, out_dtype=torch.float32)
    dw_g = J.jet_fp8_grouped_wgrad_pow2(dyqT_g, dysT_g, xqT_g, xsT_g, seg, M)
    dyqT, dysT = J.jet_quant_act_128x1_T_pow2(dev_bf16(dy))
    xqT, xsT = J.jet_quant_act_128x1_T_pow2(xq, src_s=xs)
    dw_d = J.jet_fp8_linear_wgrad_pow2(dyqT, dysT, xqT, xsT, M)
    torch.cuda.synchronize()
    Mp = dyqT.shape[1]
    assert torch.equal(dyqT_g[:, :Mp], dyqT) and torch.equal(xsT_g[:Mp // 128], xsT)
    assert_bits_equal(host(y_g), host(y_d), "grouped vs dense fwd")
    assert_bits_equal(host(dx_g), host(dx_d), "grouped vs dense dgrad")
    assert_bits_equal(host(dw_g)[0], host(dw_d), "grouped vs dense wgrad")


DECODE = {"qkv": (6144, 4096), "o": (4096, 4096), "gate_up": (28672, 4096), "down": (4096, 14336)}


@pytest.mark.parametrize("name", list(DECODE))
def test_decode_rows_equal_training_rows(gpu_lib, name):
    """Rollout decode on the Llama-8B layers: rows computed at M = 1, 64 and
    100 (the weight-streaming kernel, one K range) equal the same rows of a
    2048-row batch (the tiled kernel) bit for bit, in BF16, in the fused codes
    and scales, and in FP32; the M = 64 rows meet the GEMM rule against the
    oracle on sampled columns."""
    J = gpu_lib
    N, K = DECODE[name]
    x = inputs.activations_with_outliers(2048, K, seed=5)
    w = inputs.normal_bf16((N, K), 0.02, seed=5, tensor_id=inputs.ID_W)
    xq, xs = J.jet_quant_act_1x128_pow2(dev_bf16(x))
    wq, ws, _ = J.jet_quant_weight_128x128_pow2(dev_bf16(w), transposed=False)
    y, yq, ys = J.jet_fp8_linear_fwd_pow2(xq, xs, wq, ws, fuse_quant=True)
    y32 = J.jet_fp8_linear_fwd_pow2(xq, xs, wq, ws, out_dtype=torch.float32)
    torch.cuda.synchronize()
    for lo, m in ((7, 1), (100, 64), (1000, 100)):
        sx, ss = xq[lo:lo + m].contiguous(), xs[:, lo:lo + m].contiguous()
        yd, yqd, ysd = J.jet_fp8_linear_fwd_pow2(sx, ss, wq, ws, fuse_quant=True)
        y32d = J.jet_fp8_linear_fwd_pow2(sx, ss, wq, ws, out_dtype=torch.float32)
        torch.cuda.synchronize()
        tag = f"{name} rows {lo}:{lo + m}"
        assert torch.equal(yd, y[lo:lo + m]), f"BF16 {tag}"
        assert torch.equal(yqd, yq[lo:lo + m]) and torch.equal(ysd, ys[:, lo:lo + m]), f"fused {tag}"
        assert_bits_equal(host(y32d), host(y32[lo:lo + m]), f"FP32 {tag}")
    rng = np.random.default_rng(N)
    cols = np.sort(rng.choice(N, 256, replace=False))
    q1, s1 = P.quant_1x128_pow2(x[100:164])
    assert_bits_equal(host(xq[100:164]), q1, "decode x codes")
    wq_h, ws_h = host(wq), host(ws)
    b = O.e4m3_decode(wq_h[cols]) * np.repeat(ws_h[cols // 128], 128, axis=1)
    a = O.dequant_1x128(q1, s1)
    check_f32_output(host(y32[100:164])[:, cols], a @ b.T, oracle_absprod(a, b), f"decode fwd {name}")


# --- fused producers of the 1x128 input ---------------------------------------

@pytest.mark.parametrize("M,H", [(1, 128), (37, 640), (100, 4096), (64, 8192)])
def test_rmsnorm_quant_pow2(gpu_lib, M, H):
    """The BF16 RMSNorm output is bit-identical to the FP32-scale producer's
    (only the scale rule differs) and its codes and scales are the oracle's
    power-of-two 1x128 quantization of it."""
    from oracle import fused_producers as F
    J = gpu_lib
    x = inputs.activations_with_outliers(M, H, seed=H)
    gam = O.bf16_rne(inputs.normal_bf16((H,), 0.1, seed=H, tensor_id=inputs.ID_W) + np.float32(1.0))
    xd, gd = dev_bf16(x), dev_bf16(gam)
    y2, q2, s2 = J.jet_rmsnorm_quant_1x128_pow2(xd, gd, 1e-5, return_y=True)
    y1, _, _ = J.jet_rmsnorm_quant_1x128(xd, gd, 1e-5, return_y=True)
    torch.cuda.synchronize()
    assert torch.equal(y2, y1), "BF16 output differs from the FP32-scale producer's"
    ref_y = F.rmsnorm_bf16(x, gam, 1e-5)
    assert np.all(np.abs(host(y2).astype(np.float64) - ref_y) <= np.maximum(F.bf16_ulp(ref_y), 2.0 ** -126))
    rq, rs = P.quant_1x128_pow2(host(y2))
    assert_bits_equal(host(q2), rq, f"rmsnorm pow2 codes M={M} H={H}")
    assert_bits_equal(host(s2), rs, f"rmsnorm pow2 scales M={M} H={H}")
    P.e8m0(host(s2))


@pytest.mark.parametrize("M,I", [(1, 128), (37, 384), (100, 14336)])
def test_swiglu_quant_pow2(gpu_lib, M, I):
    from oracle import fused_producers as F
    J = gpu_lib
    gu = inputs.normal_bf16((M, 2 * I), 2.0, seed=I, tensor_id=inputs.ID_X)
    gd = dev_bf16(gu)
    h2, q2, s2 = J.jet_swiglu_quant_1x128_pow2(gd, return_h=True)
    h1, _, _ = J.jet_swiglu_quant_1x128(gd, return_h=True)
    torch.cuda.synchronize()
    assert torch.equal(h2, h1), "BF16 output differs from the FP32-scale producer's"
    ref_h = F.swiglu_bf16(gu, I)
    assert np.all(np.abs(host(h2).astype(np.float64) - ref_h) <= np.maximum(F.bf16_ulp(ref_h), 2.0 ** -126))
    rq, rs = P.quant_1x128_pow2(host(h2))
    assert_bits_equal(host(q2), rq, f"swiglu pow2 codes M={M} I={I}")
    assert_bits_equal(host(s2), rs, f"swiglu pow2 scales M={M} I={I}")
