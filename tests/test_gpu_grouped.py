"""GPU parity of the grouped (mixture-of-experts) layer against the oracle.

Same rules as the dense tests (gpu_helpers): the grouped 128x1 quantizer is
bit-exact on the valid columns of the padded layout; the grouped GEMMs are
within the accumulation allowance and the relative Frobenius bounds; the
integer case is bit-exact; the fused 1x128 epilogue is bit-exact by
composition.  Segments cover the awkward cases: empty, single-row, ragged,
exactly 128 and just above 128 rows.
"""
import numpy as np
import pytest
import torch

from oracle import jet_oracle as O
from fp8_blockwise_quantized_amd import inputs
from tests.gpu_helpers import (assert_bits_equal, bf16_frobenius, check_bf16_output, check_f32_output,
                               dev_bf16, host, oracle_absprod)

pytestmark = pytest.mark.gpu

LENS = [5, 0, 200, 128, 1, 130, 0, 257]


def seg_from_lens(lens):
    off = np.zeros(len(lens) + 1, dtype=np.int32)
    off[1:] = np.cumsum(lens)
    return off


def dev_seg(seg):
    return torch.from_numpy(np.asarray(seg, np.int32)).cuda()


def quantize_grouped(J, x, w, dy, seg):
    """GPU quantization of a grouped layer (dense 1x128 and stacked 128x128,
    grouped 128x1), each output checked bit-exact against the oracle."""
    E, N, K = w.shape
    M = x.shape[0]
    segd = dev_seg(seg)
    xq, xs = J.jet_quant_act_1x128(dev_bf16(x))
    dyq, dys = J.jet_quant_act_1x128(dev_bf16(dy))
    wq2, ws2, wqT = J.jet_quant_weight_128x128(dev_bf16(w.reshape(E * N, K)))
    dyqT, dysT = J.jet_quant_act_128x1_T_grouped(dev_bf16(dy), segd)
    xqT, xsT = J.jet_quant_act_128x1_T_grouped(xq, segd, src_s=xs)
    torch.cuda.synchronize()
    ref = {}
    ref["xq"], ref["xs"] = O.quant_1x128(x)
    ref["dyq"], ref["dys"] = O.quant_1x128(dy)
    wq = np.empty((E, N, K), np.uint8)
    ws = np.empty((E, N // 128, K // 128), np.float32)
    for e in range(E):
        wq[e], ws[e] = O.quant_128x128(w[e])
    ref["dyqT"], ref["dysT"] = O.quant_128x1_T_grouped(dy, seg)
    ref["xqT"], ref["xsT"] = O.requant_128x1_T_grouped_from_1x128(ref["xq"], ref["xs"], seg)
    P = ref["dyqT"].shape[1]
    assert P <= J.grouped_columns(M, E)
    assert_bits_equal(host(xq), ref["xq"], "xq")
    assert_bits_equal(host(xs), ref["xs"], "xs")
    assert_bits_equal(host(dyq), ref["dyq"], "dyq")
    assert_bits_equal(host(dys), ref["dys"], "dys")
    assert_bits_equal(host(wq2).reshape(E, N, K), wq, "wq")
    assert_bits_equal(host(ws2).reshape(E, N // 128, K // 128), ws, "ws")
    assert_bits_equal(host(dyqT)[:, :P], ref["dyqT"], "dyqT grouped")
    assert_bits_equal(host(dysT)[:P // 128], ref["dysT"], "dysT grouped")
    assert_bits_equal(host(xqT)[:, :P], ref["xqT"], "xqT grouped")
    assert_bits_equal(host(xsT)[:P // 128], ref["xsT"], "xsT grouped")
    ref["wq"], ref["ws"] = wq, ws
    dev = dict(seg=segd, xq=xq, xs=xs, dyq=dyq, dys=dys, wq=wq2.view(E, N, K),
               ws=ws2.view(E, N // 128, K // 128), wqT=wqT, dyqT=dyqT, dysT=dysT, xqT=xqT, xsT=xsT)
    return dev, ref


def grouped_inputs(lens, N, K, seed):
    M = int(sum(lens))
    x = inputs.activations_with_outliers(M, K, seed=seed)
    w = inputs.normal_bf16((len(lens), N, K), 0.02, seed=seed, tensor_id=inputs.ID_W)
    dy = inputs.normal_bf16((M, N), 1e-3, seed=seed, tensor_id=inputs.ID_DY)
    return x, w, dy


def quantize_grouped_sampled(J, x, w, dy, seg, experts):
    """As quantize_grouped for large problems: the GPU quantizes everything;
    the oracle checks the rows, weights and padded columns of `experts`."""
    E, N, K = w.shape
    segd = dev_seg(seg)
    xq, xs = J.jet_quant_act_1x128(dev_bf16(x))
    dyq, dys = J.jet_quant_act_1x128(dev_bf16(dy))
    wq2, ws2, wqT = J.jet_quant_weight_128x128(dev_bf16(w.reshape(E * N, K)))
    dyqT, dysT = J.jet_quant_act_128x1_T_grouped(dev_bf16(dy), segd)
    xqT, xsT = J.jet_quant_act_128x1_T_grouped(xq, segd, src_s=xs)
    torch.cuda.synchronize()
    col = O.segment_columns(seg)
    r = {"xq": {}, "xs": {}, "dyq": {}, "dys": {}, "wq": {}, "ws": {}, "dyqT": {}, "dysT": {},
         "xqT": {}, "xsT": {}}
    hx, hxs, hdy, hdys = host(xq), host(xs), host(dyq), host(dys)
    hwq = host(wq2).reshape(E, N, K)
    hws = host(ws2).reshape(E, N // 128, K // 128)
    hdyqT, hdysT, hxqT, hxsT = host(dyqT), host(dysT), host(xqT), host(xsT)
    for e in experts:
        lo, hi = int(seg[e]), int(seg[e + 1])
        c0, c1 = int(col[e]), int(col[e + 1])
        tag = f"expert {e}"
        r["xq"][e], r["xs"][e] = O.quant_1x128(x[lo:hi])
        r["dyq"][e], r["dys"][e] = O.quant_1x128(dy[lo:hi])
        r["wq"][e], r["ws"][e] = O.quant_128x128(w[e])
        r["dyqT"][e], r["dysT"][e] = O.quant_128x1_T(dy[lo:hi])
        r["xqT"][e], r["xsT"][e] = O.requant_128x1_T_from_1x128(r["xq"][e], r["xs"][e])
        assert_bits_equal(hx[lo:hi], r["xq"][e], f"xq {tag}")
        assert_bits_equal(hxs[:, lo:hi], r["xs"][e], f"xs {tag}")
        assert_bits_equal(hdy[lo:hi], r["dyq"][e], f"dyq {tag}")
        assert_bits_equal(hdys[:, lo:hi], r["dys"][e], f"dys {tag}")
        assert_bits_equal(hwq[e], r["wq"][e], f"wq {tag}")
        assert_bits_equal(hws[e], r["ws"][e], f"ws {tag}")
        assert_bits_equal(hdyqT[:, c0:c1], r["dyqT"][e], f"dyqT {tag}")
        assert_bits_equal(hdysT[c0 // 128:c1 // 128], r["dysT"][e], f"dysT {tag}")
        assert_bits_equal(hxqT[:, c0:c1], r["xqT"][e], f"xqT {tag}")
        assert_bits_equal(hxsT[c0 // 128:c1 // 128], r["xsT"][e], f"xsT {tag}")
    dev = dict(seg=segd, xq=xq, xs=xs, dyq=dyq, dys=dys, wq=wq2.view(E, N, K),
               ws=ws2.view(E, N // 128, K // 128), wqT=wqT, dyqT=dyqT, dysT=dysT, xqT=xqT, xsT=xsT)
    return dev, r


def check_grouped(J, lens, N, K, seed, experts=None):
    """Full grouped layer on the GPU.  experts=None: every quantized tensor
    and every expert is checked; otherwise only the listed experts (large
    shapes), whose rows, weights and columns the oracle computes alone."""
    seg = seg_from_lens(lens)
    E = len(lens)
    x, w, dy = grouped_inputs(lens, N, K, seed)
    M = int(seg[-1])
    if experts is None:
        d, r = quantize_grouped(J, x, w, dy, seg)
        experts = range(E)
    else:
        d, r = quantize_grouped_sampled(J, x, w, dy, seg, experts)
    y16, yq, ys = J.jet_fp8_grouped_fwd(d["xq"], d["xs"], d["wq"], d["ws"], d["seg"], fuse_quant=True)
    dx16 = J.jet_fp8_grouped_dgrad(d["dyq"], d["dys"], d["wqT"], d["ws"], d["seg"])
    dw32 = J.jet_fp8_grouped_wgrad(d["dyqT"], d["dysT"], d["xqT"], d["xsT"], d["seg"], M)
    torch.cuda.synchronize()
    y16h, dx16h, dw32h = host(y16), host(dx16), host(dw32)
    yqh, ysh = host(yq), host(ys)
    col = O.segment_columns(seg)
    sampled = isinstance(r["wq"], dict)
    # BF16 outputs: the element rule per expert, the Frobenius bound over all
    # checked rows together (a one-row segment alone is 256 values, too few
    # for a norm of the rounding differences to mean anything)
    fy, ry, fdx, rdx = [], [], [], []
    for e in experts:
        lo, hi = int(seg[e]), int(seg[e + 1])
        tag = f"expert {e} rows {lo}:{hi}"
        if hi == lo:
            assert not dw32h[e].any(), f"empty {tag}: dW must be zero"
            continue
        # fused epilogue: bit-exact 1x128 quantization of the GPU's own BF16 Y rows
        qo, so = O.quant_1x128(y16h[lo:hi])
        assert_bits_equal(yqh[lo:hi], qo, f"grouped fused codes {tag}")
        assert_bits_equal(ysh[:, lo:hi], so, f"grouped fused scales {tag}")
        if sampled:
            a_x = O.dequant_1x128(r["xq"][e], r["xs"][e])
            a_dy = O.dequant_1x128(r["dyq"][e], r["dys"][e])
            b_w = O.dequant_128x128(r["wq"][e], r["ws"][e])
            dyqT_e, dysT_e, xqT_e, xsT_e = r["dyqT"][e], r["dysT"][e], r["xqT"][e], r["xsT"][e]
        else:
            a_x = O.dequant_1x128(r["xq"][lo:hi], r["xs"][:, lo:hi])
            a_dy = O.dequant_1x128(r["dyq"][lo:hi], r["dys"][:, lo:hi])
            b_w = O.dequant_128x128(r["wq"][e], r["ws"][e])
            c0, c1 = int(col[e]), int(col[e + 1])
            dyqT_e, dysT_e = r["dyqT"][:, c0:c1], r["dysT"][c0 // 128:c1 // 128]
            xqT_e, xsT_e = r["xqT"][:, c0:c1], r["xsT"][c0 // 128:c1 // 128]
        ref_y, ref_dx = a_x @ b_w.T, a_dy @ b_w
        check_bf16_output(y16h[lo:hi], ref_y, oracle_absprod(a_x, b_w), f"grouped fwd {tag}", fro=False)
        check_bf16_output(dx16h[lo:hi], ref_dx, oracle_absprod(a_dy, b_w.T), f"grouped dgrad {tag}", fro=False)
        fy.append(y16h[lo:hi]); ry.append(ref_y); fdx.append(dx16h[lo:hi]); rdx.append(ref_dx)
        a_dyT = O.dequant_128x1_T(dyqT_e, dysT_e, hi - lo)
        a_xT = O.dequant_128x1_T(xqT_e, xsT_e, hi - lo)
        check_f32_output(dw32h[e], a_dyT @ a_xT.T, oracle_absprod(a_dyT, a_xT), f"grouped wgrad {tag}")
    if fy:
        bf16_frobenius(fy, ry, "grouped fwd, all checked experts")
        bf16_frobenius(fdx, rdx, "grouped dgrad, all checked experts")


def test_grouped_small_all_steps(gpu_lib):
    check_grouped(gpu_lib, LENS, 256, 384, seed=21)


@pytest.mark.parametrize("E", [128, 200])
def test_grouped_many_experts_all_steps(gpu_lib, E):
    """128 experts (the wgrad takes them by decreasing contraction, found
    from the offsets in registers) and 200 (more than one register pass over
    the offsets: index order in wgrad, looped scans in the row-grouped
    GEMMs); the lengths repeat (equal contractions), include empty segments
    and cross 128- and 256-row boundaries.  Every expert checked."""
    rng = np.random.default_rng(E)
    lens = [int(v) for v in rng.choice([0, 1, 64, 127, 128, 129, 200, 255, 256, 257, 300], size=E)]
    check_grouped(gpu_lib, lens, 256, 256, seed=E)


def test_grouped_single_expert_equals_dense(gpu_lib):
    """E = 1: the grouped entry points reproduce the dense ones bit for bit."""
    J = gpu_lib
    M, N, K = 300, 256, 256
    x, w, dy = grouped_inputs([M], N, K, 3)
    seg = dev_seg([0, M])
    xq, xs = J.jet_quant_act_1x128(dev_bf16(x))
    dyq, dys = J.jet_quant_act_1x128(dev_bf16(dy))
    wq, ws, wqT = J.jet_quant_weight_128x128(dev_bf16(w[0]))
    y_g = J.jet_fp8_grouped_fwd(xq, xs, wq[None], ws[None], seg, out_dtype=torch.float32)
    y_d = J.jet_fp8_linear_fwd(xq, xs, wq, ws, out_dtype=torch.float32)
    dx_g = J.jet_fp8_grouped_dgrad(dyq, dys, wqT, ws[None], seg, out_dtype=torch.float32)
    dx_d = J.jet_fp8_linear_dgrad(dyq, dys, wqT, ws, out_dtype=torch.float32)
    dyqT_g, dysT_g = J.jet_quant_act_128x1_T_grouped(dev_bf16(dy), seg)
    xqT_g, xsT_g = J.jet_quant_act_128x1_T_grouped(xq, seg, src_s=xs)
    dyqT, dysT = J.jet_quant_act_128x1_T(dev_bf16(dy))
    xqT, xsT = J.jet_quant_act_128x1_T(xq, src_s=xs)
    dw_g = J.jet_fp8_grouped_wgrad(dyqT_g, dysT_g, xqT_g, xsT_g, seg, M)
    dw_d = J.jet_fp8_linear_wgrad(dyqT, dysT, xqT, xsT, M)
    torch.cuda.synchronize()
    Mp = dyqT.shape[1]
    assert torch.equal(dyqT_g[:, :Mp], dyqT) and torch.equal(xqT_g[:, :Mp], xqT)
    assert torch.equal(dysT_g[:Mp // 128], dysT) and torch.equal(xsT_g[:Mp // 128], xsT)
    # the grouped kernels take the 128x128 tile; the dense ones pick their own
    # tile, so compare to the oracle's tolerance rather than bitwise
    for g, dref, name in [(y_g, y_d, "fwd"), (dx_g, dx_d, "dgrad"), (dw_g[0], dw_d, "wgrad")]:
        rel = ((g - dref).norm() / dref.norm()).item()
        assert rel < 1e-5, f"{name}: grouped vs dense relative difference {rel}"


def anchored_segments(rng, lens, cols):
    """Integers in [-7, 7]; inside each 128-row group of a segment (nr rows),
    row r holds +-7 at the columns c with c % nr == r: every 1x128 and every
    128x1 group holds a +-7, so every scale is 7/448 = 2^-6 and every code
    product is a multiple of 4096."""
    out = []
    for n in lens:
        v = rng.integers(-7, 8, size=(n, cols)).astype(np.float32)
        for g0 in range(0, n, 128):
            nr = min(128, n - g0)
            anchor = np.arange(nr)[:, None] == (np.arange(cols)[None, :] % nr)
            blk = v[g0:g0 + nr]
            blk[anchor] = np.where(rng.integers(0, 2, size=int(anchor.sum())) == 1, 7.0, -7.0)
        out.append(v)
    return np.concatenate(out, axis=0)


def test_grouped_integer_case_bit_exact(gpu_lib):
    J = gpu_lib
    rng = np.random.default_rng(5)
    lens = LENS
    E, N, K = len(lens), 256, 384
    seg = seg_from_lens(lens)
    x = anchored_segments(rng, lens, K)
    dy = anchored_segments(rng, lens, N)
    w = rng.integers(-7, 8, size=(E, N, K)).astype(np.float32)
    diag = (np.arange(N)[:, None] % 128) == (np.arange(K)[None, :] % 128)
    for e in range(E):
        w[e][diag] = np.where(rng.integers(0, 2, size=int(diag.sum())) == 1, 7.0, -7.0)
    d, r = quantize_grouped(J, x, w, dy, seg)
    y = J.jet_fp8_grouped_fwd(d["xq"], d["xs"], d["wq"], d["ws"], d["seg"], out_dtype=torch.float32)
    dx = J.jet_fp8_grouped_dgrad(d["dyq"], d["dys"], d["wqT"], d["ws"], d["seg"], out_dtype=torch.float32)
    dw = J.jet_fp8_grouped_wgrad(d["dyqT"], d["dysT"], d["xqT"], d["xsT"], d["seg"], int(seg[-1]))
    torch.cuda.synchronize()
    xi, dyi, wi = x.astype(np.int64), dy.astype(np.int64), w.astype(np.int64)
    yh, dxh, dwh = host(y), host(dx), host(dw)
    for e in range(E):
        lo, hi = int(seg[e]), int(seg[e + 1])
        assert_bits_equal(yh[lo:hi], (xi[lo:hi] @ wi[e].T).astype(np.float32), f"fwd integer expert {e}")
        assert_bits_equal(dxh[lo:hi], (dyi[lo:hi] @ wi[e]).astype(np.float32), f"dgrad integer expert {e}")
        assert_bits_equal(dwh[e], (dyi[lo:hi].T @ xi[lo:hi]).astype(np.float32), f"wgrad integer expert {e}")


def test_grouped_wgrad_accumulate(gpu_lib):
    J = gpu_lib
    lens = [130, 0, 64]
    seg = seg_from_lens(lens)
    x, w, dy = grouped_inputs(lens, 256, 256, 8)
    d, r = quantize_grouped(J, x, w, dy, seg)
    c0 = torch.randn(len(lens), 256, 256, device="cuda")
    dw = c0.clone()
    J.jet_fp8_grouped_wgrad(d["dyqT"], d["dysT"], d["xqT"], d["xsT"], d["seg"], int(seg[-1]), dw=dw,
                            accumulate=True)
    torch.cuda.synchronize()
    ref = O.gemm_grouped_wgrad(r["dyqT"], r["dysT"], r["xqT"], r["xsT"], seg)
    col = O.segment_columns(seg)
    for e in range(len(lens)):
        if lens[e] == 0:
            assert torch.equal(dw[e], c0[e])
            continue
        c_0, c_1 = int(col[e]), int(col[e + 1])
        a_dyT = O.dequant_128x1_T(r["dyqT"][:, c_0:c_1], r["dysT"][c_0 // 128:c_1 // 128], lens[e])
        a_xT = O.dequant_128x1_T(r["xqT"][:, c_0:c_1], r["xsT"][c_0 // 128:c_1 // 128], lens[e])
        absprod = oracle_absprod(a_dyT, a_xT) + np.abs(host(c0[e]))
        check_f32_output(host(dw[e]), host(c0[e]).astype(np.float64) + ref[e], absprod,
                         f"grouped wgrad accumulate expert {e}")


def moe_routing(num_tokens=8192, experts=128, top_k=8, alpha=1.1, seed=0):
    ids = inputs.zipf_top8_routing(num_tokens, experts, top_k, alpha, seed)
    return inputs.segment_offsets(ids, experts)


@pytest.mark.parametrize("name,N,K", [("gate_up", 1536, 2048), ("down", 2048, 768)])
def test_moe_qwen3_30b_shapes_sampled(gpu_lib, name, N, K):
    """Qwen3-30B-A3B expert layers (128 experts, top-8 of 8192 tokens, Zipf(1.1)
    load): the whole grouped layer runs on the GPU; the oracle checks the
    smallest, the median and the largest expert in full."""
    seg = moe_routing()
    lens = np.diff(seg)
    order = np.argsort(lens, kind="stable")
    experts = [int(order[0]), int(order[len(order) // 2]), int(order[-1])]
    check_grouped(gpu_lib, list(lens), N, K, seed=0, experts=experts)
