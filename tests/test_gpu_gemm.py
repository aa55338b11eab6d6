"""GPU parity of the three block-scaled FP8 GEMMs (forward, dgrad, wgrad) and
the fused 1x128 epilogue against the oracle.

Rules (gpu_helpers): FP32 outputs within 2^-11 * sum|a*b| per element (the
measured sub-block precision of the FP8 MFMA, with margin) and 1e-4 relative
Frobenius of the float64 product of the dequantized operands; BF16 outputs
within one BF16 ulp plus that allowance and 1e-3 relative Frobenius of
bf16_rne(fl32(reference)); the integer special case and the fused
quantization are bit-exact.  Operands are always quantized on the GPU
and first checked bit-exact against the oracle's quantizers, so both sides
multiply the same codes and scales.
"""
import numpy as np
import pytest
import torch

from oracle import jet_oracle as O
from oracle import pow2_scales as P
from fp8_blockwise_quantized_amd import inputs
from tests.gpu_helpers import (assert_bits_equal, check_bf16_output, check_f32_output, dev_bf16,
                               host, oracle_absprod)

pytestmark = pytest.mark.gpu


def quantize_all(J, x, w, dy):
    """GPU quantization of one linear layer's tensors, checked against the oracle."""
    xd, wd, dyd = dev_bf16(x), dev_bf16(w), dev_bf16(dy)
    xq, xs = J.jet_quant_act_1x128(xd)
    wq, ws, wqT = J.jet_quant_weight_128x128(wd)
    dyq, dys = J.jet_quant_act_1x128(dyd)
    dyqT, dysT = J.jet_quant_act_128x1_T(dyd)
    xqT, xsT = J.jet_quant_act_128x1_T(xq, src_s=xs)
    torch.cuda.synchronize()
    ref = {}
    ref["xq"], ref["xs"] = O.quant_1x128(x)
    ref["wq"], ref["ws"] = O.quant_128x128(w)
    ref["dyq"], ref["dys"] = O.quant_1x128(dy)
    ref["dyqT"], ref["dysT"] = O.quant_128x1_T(dy)
    ref["xqT"], ref["xsT"] = O.requant_128x1_T_from_1x128(ref["xq"], ref["xs"])
    dev = dict(xq=xq, xs=xs, wq=wq, ws=ws, wqT=wqT, dyq=dyq, dys=dys, dyqT=dyqT, dysT=dysT,
               xqT=xqT, xsT=xsT)
    for k in ref:
        assert_bits_equal(host(dev[k]), ref[k], k)
    assert_bits_equal(host(wqT), ref["wq"].T, "wqT")
    return dev, ref


def layer_inputs(M, N, K, seed):
    x = inputs.activations_with_outliers(M, K, seed=seed)
    w = inputs.normal_bf16((N, K), 0.02, seed=seed, tensor_id=inputs.ID_W)
    dy = inputs.normal_bf16((M, N), 1e-3, seed=seed, tensor_id=inputs.ID_DY)
    return x, w, dy


def run_and_check(J, M, N, K, seed, out_f32=True):
    x, w, dy = layer_inputs(M, N, K, seed)
    d, r = quantize_all(J, x, w, dy)
    a_x = O.dequant_1x128(r["xq"], r["xs"])
    b_w = O.dequant_128x128(r["wq"], r["ws"])
    a_dy = O.dequant_1x128(r["dyq"], r["dys"])
    a_dyT = O.dequant_128x1_T(r["dyqT"], r["dysT"], M)
    a_xT = O.dequant_128x1_T(r["xqT"], r["xsT"], M)
    # forward
    y_ref = a_x @ b_w.T
    y_abs = oracle_absprod(a_x, b_w)
    y16, yq, ys = J.jet_fp8_linear_fwd(d["xq"], d["xs"], d["wq"], d["ws"], fuse_quant=True)
    dx16 = J.jet_fp8_linear_dgrad(d["dyq"], d["dys"], d["wqT"], d["ws"])
    dw32 = J.jet_fp8_linear_wgrad(d["dyqT"], d["dysT"], d["xqT"], d["xsT"], M)
    torch.cuda.synchronize()
    tag = f"M={M} N={N} K={K}"
    check_bf16_output(host(y16), y_ref, y_abs, f"fwd bf16 {tag}")
    # fused epilogue: bit-exact 1x128 quantization of the GPU's own BF16 Y
    qo, so = O.quant_1x128(host(y16))
    assert_bits_equal(host(yq), qo, f"fused codes {tag}")
    assert_bits_equal(host(ys), so, f"fused scales {tag}")
    dx_ref = a_dy @ b_w
    check_bf16_output(host(dx16), dx_ref, oracle_absprod(a_dy, b_w.T), f"dgrad bf16 {tag}")
    dw_ref = a_dyT @ a_xT.T
    check_f32_output(host(dw32), dw_ref, oracle_absprod(a_dyT, a_xT), f"wgrad f32 {tag}")
    if out_f32:
        y32 = J.jet_fp8_linear_fwd(d["xq"], d["xs"], d["wq"], d["ws"], out_dtype=torch.float32)
        dx32 = J.jet_fp8_linear_dgrad(d["dyq"], d["dys"], d["wqT"], d["ws"], out_dtype=torch.float32)
        dw16 = J.jet_fp8_linear_wgrad(d["dyqT"], d["dysT"], d["xqT"], d["xsT"], M,
                                      out_dtype=torch.bfloat16)
        torch.cuda.synchronize()
        check_f32_output(host(y32), y_ref, y_abs, f"fwd f32 {tag}")
        check_f32_output(host(dx32), dx_ref, oracle_absprod(a_dy, b_w.T), f"dgrad f32 {tag}")
        check_bf16_output(host(dw16), dw_ref, oracle_absprod(a_dyT, a_xT), f"wgrad bf16 {tag}")
    return d, r


def test_config_single_layer_256x512x512(gpu_lib):
    """The small parity configuration: M=256 tokens, K=512, N=512, seed 0."""
    M, N, K = 256, 512, 512
    x = inputs.normal_bf16((M, K), 1.0, seed=0, tensor_id=inputs.ID_X)
    w = inputs.normal_bf16((N, K), 0.02, seed=0, tensor_id=inputs.ID_W)
    dy = inputs.normal_bf16((M, N), 1e-3, seed=0, tensor_id=inputs.ID_DY)
    d, r = quantize_all(gpu_lib, x, w, dy)
    y = gpu_lib.jet_fp8_linear_fwd(d["xq"], d["xs"], d["wq"], d["ws"], out_dtype=torch.float32)
    dx = gpu_lib.jet_fp8_linear_dgrad(d["dyq"], d["dys"], d["wqT"], d["ws"], out_dtype=torch.float32)
    dw = gpu_lib.jet_fp8_linear_wgrad(d["dyqT"], d["dysT"], d["xqT"], d["xsT"], M)
    torch.cuda.synchronize()
    a_x, b_w = O.dequant_1x128(r["xq"], r["xs"]), O.dequant_128x128(r["wq"], r["ws"])
    check_f32_output(host(y), O.gemm_fwd(r["xq"], r["xs"], r["wq"], r["ws"]),
                     oracle_absprod(a_x, b_w), "fwd")
    a_dy = O.dequant_1x128(r["dyq"], r["dys"])
    check_f32_output(host(dx), O.gemm_dgrad(r["dyq"], r["dys"], r["wq"], r["ws"]),
                     oracle_absprod(a_dy, b_w.T), "dgrad")
    a_dyT = O.dequant_128x1_T(r["dyqT"], r["dysT"], M)
    a_xT = O.dequant_128x1_T(r["xqT"], r["xsT"], M)
    check_f32_output(host(dw), O.gemm_wgrad(r["dyqT"], r["dysT"], r["xqT"], r["xsT"], M),
                     oracle_absprod(a_dyT, a_xT), "wgrad")


@pytest.mark.parametrize("M,N,K", [(1, 128, 128), (63, 256, 384), (65, 384, 256), (200, 256, 512),
                                   (129, 128, 1024), (384, 640, 384)])
def test_ragged_shapes_all_gemms(gpu_lib, M, N, K):
    run_and_check(gpu_lib, M, N, K, seed=M + N + K)


def anchored_small_int(rng, rows, cols):
    """Integers in [-7, 7] with +-7 on the diagonal rows == cols (mod 128), so
    every 1x128, 128x1 and 128x128 group holds a +-7: every scale is exactly
    7/448 = 2^-6 and every code is exact (64*v)."""
    v = rng.integers(-7, 8, size=(rows, cols)).astype(np.float32)
    diag = (np.arange(rows)[:, None] % 128) == (np.arange(cols)[None, :] % 128)
    v[diag] = np.where(rng.integers(0, 2, size=int(diag.sum())) == 1, 7.0, -7.0)
    return v


def test_integer_case_bit_exact(gpu_lib):
    """Every product of codes is a multiple of 64*64 = 4096, far above the
    MFMA's internal sub-block resolution, every per-step partial and every
    FP32 partial sum is exactly representable, and the scales are powers of
    two: the FP32 results must equal the integer matrix products exactly.
    A single dropped, duplicated or misplaced product would show."""
    rng = np.random.default_rng(0)
    M, N, K = 256, 384, 1024
    x, w, dy = anchored_small_int(rng, M, K), anchored_small_int(rng, N, K), anchored_small_int(rng, M, N)
    d, r = quantize_all(gpu_lib, x, w, dy)
    for key in ("xs", "ws", "dys", "dysT", "xsT"):
        assert np.all(r[key] == np.float32(2.0 ** -6))
    y = gpu_lib.jet_fp8_linear_fwd(d["xq"], d["xs"], d["wq"], d["ws"], out_dtype=torch.float32)
    dx = gpu_lib.jet_fp8_linear_dgrad(d["dyq"], d["dys"], d["wqT"], d["ws"], out_dtype=torch.float32)
    dw = gpu_lib.jet_fp8_linear_wgrad(d["dyqT"], d["dysT"], d["xqT"], d["xsT"], M)
    torch.cuda.synchronize()
    xi, wi, dyi = x.astype(np.int64), w.astype(np.int64), dy.astype(np.int64)
    assert_bits_equal(host(y), (xi @ wi.T).astype(np.float32), "fwd integer")
    assert_bits_equal(host(dx), (dyi @ wi).astype(np.float32), "dgrad integer")
    assert_bits_equal(host(dw), (dyi.T @ xi).astype(np.float32), "wgrad integer")


# Shapes whose 256x256-tile grid fills (almost) whole waves of 256 CUs, so all
# three GEMMs take the large-tile kernel; the small-shape tests above take the
# 128x128 kernel.  3969 tokens leave a ragged last row tile and 128x1 group.
BIG_TILE_SHAPE = (3969, 3840, 3968)


def test_ragged_big_tile_all_gemms(gpu_lib):
    M, N, K = BIG_TILE_SHAPE
    run_and_check(gpu_lib, M, N, K, seed=11, out_f32=False)


def test_integer_case_bit_exact_big_tile(gpu_lib):
    """As test_integer_case_bit_exact, at a shape that takes the 256x256 tile
    in every GEMM (M a multiple of 128 so every 128x1 group holds a +-7).
    Integer products below 2^53 make the float64 matmul exact."""
    rng = np.random.default_rng(1)
    M, N, K = 3968, 3840, 3968
    x, w, dy = anchored_small_int(rng, M, K), anchored_small_int(rng, N, K), anchored_small_int(rng, M, N)
    d, r = quantize_all(gpu_lib, x, w, dy)
    for key in ("xs", "ws", "dys", "dysT", "xsT"):
        assert np.all(r[key] == np.float32(2.0 ** -6))
    y = gpu_lib.jet_fp8_linear_fwd(d["xq"], d["xs"], d["wq"], d["ws"], out_dtype=torch.float32)
    dx = gpu_lib.jet_fp8_linear_dgrad(d["dyq"], d["dys"], d["wqT"], d["ws"], out_dtype=torch.float32)
    dw = gpu_lib.jet_fp8_linear_wgrad(d["dyqT"], d["dysT"], d["xqT"], d["xsT"], M)
    torch.cuda.synchronize()
    xf, wf, dyf = x.astype(np.float64), w.astype(np.float64), dy.astype(np.float64)
    assert_bits_equal(host(y), (xf @ wf.T).astype(np.float32), "fwd integer")
    assert_bits_equal(host(dx), (dyf @ wf).astype(np.float32), "dgrad integer")
    assert_bits_equal(host(dw), (dyf.T @ xf).astype(np.float32), "wgrad integer")


def test_wgrad_accumulate_and_empty_tokens(gpu_lib):
    M, N, K = 200, 256, 384
    x, w, dy = layer_inputs(M, N, K, 9)
    d, r = quantize_all(gpu_lib, x, w, dy)
    c0 = torch.randn(N, K, device="cuda")
    dw = c0.clone()
    gpu_lib.jet_fp8_linear_wgrad(d["dyqT"], d["dysT"], d["xqT"], d["xsT"], M, dw=dw, accumulate=True)
    ref = O.gemm_wgrad(r["dyqT"], r["dysT"], r["xqT"], r["xsT"], M)
    # M = 0 tokens: the weight gradient is zero (or unchanged when accumulating)
    z = torch.full((N, K), 7.0, device="cuda")
    gpu_lib.jet_fp8_linear_wgrad(d["dyqT"][:, :0], d["dysT"][:0], d["xqT"][:, :0], d["xsT"][:0], 0, dw=z)
    torch.cuda.synchronize()
    a_dyT = O.dequant_128x1_T(r["dyqT"], r["dysT"], M)
    a_xT = O.dequant_128x1_T(r["xqT"], r["xsT"], M)
    absprod = oracle_absprod(a_dyT, a_xT) + np.abs(host(c0))
    check_f32_output(host(dw), host(c0).astype(np.float64) + ref, absprod, "wgrad accumulate")
    assert not host(z).any()


def test_gemms_deterministic(gpu_lib):
    M, N, K = 512, 512, 1024
    x, w, dy = layer_inputs(M, N, K, 4)
    d, _ = quantize_all(gpu_lib, x, w, dy)
    outs = []
    for _ in range(2):
        outs.append((gpu_lib.jet_fp8_linear_fwd(d["xq"], d["xs"], d["wq"], d["ws"]),
                     gpu_lib.jet_fp8_linear_dgrad(d["dyq"], d["dys"], d["wqT"], d["ws"]),
                     gpu_lib.jet_fp8_linear_wgrad(d["dyqT"], d["dysT"], d["xqT"], d["xsT"], M)))
    torch.cuda.synchronize()
    for a, b in zip(*outs):
        assert torch.equal(a, b)


# --- small M: the split-K forward (rollout decode) ---------------------------

@pytest.mark.parametrize("M", [1, 16, 64, 100, 128])
@pytest.mark.parametrize("K", [128, 1280])
def test_small_m_forward(gpu_lib, M, K):
    """M <= 128 takes the split-K forward (64-row and 128-row variants; one K
    step, and ten steps in up to ten ranges): BF16 with the fused 1x128 output
    and FP32 against the oracle, deterministic, and an explicit workspace of
    the reported size gives the same bits."""
    N = 384
    x = inputs.activations_with_outliers(M, K, seed=M + K)
    w = inputs.normal_bf16((N, K), 0.02, seed=M, tensor_id=inputs.ID_W)
    xq, xs = gpu_lib.jet_quant_act_1x128(dev_bf16(x))
    wq, ws, _ = gpu_lib.jet_quant_weight_128x128(dev_bf16(w), transposed=False)
    need = gpu_lib.jet_workspace_bytes(gpu_lib.JET_OP_FWD, M, N, K)
    assert (need > 0) == (K > 128)          # a single K step is never split
    y16, yq, ys = gpu_lib.jet_fp8_linear_fwd(xq, xs, wq, ws, fuse_quant=True)
    y32 = gpu_lib.jet_fp8_linear_fwd(xq, xs, wq, ws, out_dtype=torch.float32)
    wsp = torch.full((max(need, 16),), 0x7F, dtype=torch.uint8, device="cuda")
    y16b = gpu_lib.jet_fp8_linear_fwd(xq, xs, wq, ws, workspace=wsp)
    torch.cuda.synchronize()
    a = O.dequant_1x128(host(xq), host(xs))
    b = O.dequant_128x128(host(wq), host(ws))
    ref, absp = a @ b.T, oracle_absprod(a, b)
    tag = f"M={M} K={K}"
    check_bf16_output(host(y16), ref, absp, f"small-M fwd bf16 {tag}")
    check_f32_output(host(y32), ref, absp, f"small-M fwd f32 {tag}")
    qo, so = O.quant_1x128(host(y16))
    assert_bits_equal(host(yq), qo, f"small-M fused codes {tag}")
    assert_bits_equal(host(ys), so, f"small-M fused scales {tag}")
    assert torch.equal(y16, y16b), "explicit workspace changed the result"


def _small_m_problem(gpu_lib, M, N, K, seed):
    x = inputs.activations_with_outliers(M, K, seed=seed)
    w = inputs.normal_bf16((N, K), 0.02, seed=seed, tensor_id=inputs.ID_W)
    xq, xs = gpu_lib.jet_quant_act_1x128(dev_bf16(x))
    wq, ws, _ = gpu_lib.jet_quant_weight_128x128(dev_bf16(w), transposed=False)
    return xq, xs, wq, ws


def test_small_m_workspace_reuse_and_stale_contents(gpu_lib):
    """One workspace filled with random bytes, shared by shapes with 10, 8 and
    4 K ranges called in an interleaved order, gives every call the bits of a
    call on its own fresh workspace (no state is carried between calls)."""
    shapes = [(64, 384, 1280), (64, 2048, 2048), (32, 4096, 512)]
    needs = [gpu_lib.jet_workspace_bytes(gpu_lib.JET_OP_FWD, *sh) for sh in shapes]
    assert min(needs) > 0
    probs = [_small_m_problem(gpu_lib, *sh, seed=i) for i, sh in enumerate(shapes)]
    refs = []
    for (xq, xs, wq, ws) in probs:
        y, yq, ys = gpu_lib.jet_fp8_linear_fwd(xq, xs, wq, ws, fuse_quant=True)
        refs.append((y, yq, ys))
    g = torch.Generator(device="cuda")
    g.manual_seed(11)
    shared = torch.randint(0, 256, (max(needs),), dtype=torch.uint8, device="cuda", generator=g)
    for it, i in enumerate([0, 1, 2, 0, 2, 1, 1, 0]):
        xq, xs, wq, ws = probs[i]
        y, yq, ys = gpu_lib.jet_fp8_linear_fwd(xq, xs, wq, ws, fuse_quant=True, workspace=shared)
        torch.cuda.synchronize()
        for a, b, what in zip((y, yq, ys), refs[i], ("Y", "codes", "scales")):
            assert torch.equal(a, b), f"call {it} (shape {shapes[i]}): {what} differ on a shared workspace"


def test_small_m_graph_replay(gpu_lib):
    """A captured split-K forward (the split kernel and its finishing pass)
    replays correctly: eager work on the same workspace and a synchronization
    run between the replays; every replay equals the eager result."""
    M, N, K = 64, 4096, 4096
    xq, xs, wq, ws = _small_m_problem(gpu_lib, M, N, K, seed=3)
    need = gpu_lib.jet_workspace_bytes(gpu_lib.JET_OP_FWD, M, N, K)
    assert need > 0
    wsp = torch.empty(need, dtype=torch.uint8, device="cuda")
    y_eager, yq_eager, ys_eager = gpu_lib.jet_fp8_linear_fwd(xq, xs, wq, ws, fuse_quant=True, workspace=wsp)
    y = torch.empty(M, N, dtype=torch.bfloat16, device="cuda")
    yq = torch.empty(M, N, dtype=torch.uint8, device="cuda")
    ys = torch.empty(N // 128, M, dtype=torch.float32, device="cuda")
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):     # warm-up on the capture stream
        gpu_lib.jet_fp8_linear_fwd(xq, xs, wq, ws, y=y, fuse_quant=True, yq=yq, ys=ys, workspace=wsp)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        gpu_lib.jet_fp8_linear_fwd(xq, xs, wq, ws, y=y, fuse_quant=True, yq=yq, ys=ys, workspace=wsp)
    torch.cuda.synchronize()
    for r in range(4):
        y.zero_(); yq.zero_(); ys.zero_()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(y, y_eager) and torch.equal(yq, yq_eager) and torch.equal(ys, ys_eager), \
            f"graph replay {r} differs from the eager call"
        # eager work on the same workspace between replays (fresh tags)
        gpu_lib.jet_fp8_linear_fwd(xq, xs, wq, ws, fuse_quant=True, workspace=wsp)
        torch.cuda.synchronize()


def test_forward_on_a_side_stream_with_its_own_workspace(gpu_lib):
    """The binding allocates the split-K workspace itself when none is given;
    on a side stream the result equals the current-stream call bit for bit."""
    M, N, K = 64, 1024, 4096
    assert gpu_lib.jet_workspace_bytes(gpu_lib.JET_OP_FWD, M, N, K) > 0
    x, w, _ = layer_inputs(M, N, K, 12)
    xq, xs = gpu_lib.jet_quant_act_1x128(dev_bf16(x))
    wq, ws, _ = gpu_lib.jet_quant_weight_128x128(dev_bf16(w), transposed=False)
    ref, refq, refs = gpu_lib.jet_fp8_linear_fwd(xq, xs, wq, ws, fuse_quant=True)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    outs = []
    for _ in range(3):
        y = torch.empty_like(ref)
        yq = torch.empty_like(refq)
        ys = torch.empty_like(refs)
        with torch.cuda.stream(side):
            y.record_stream(side); yq.record_stream(side); ys.record_stream(side)
        gpu_lib.jet_fp8_linear_fwd(xq, xs, wq, ws, y=y, fuse_quant=True, yq=yq, ys=ys, stream=side)
        # work on the current stream that may reuse freed blocks meanwhile
        junk = torch.empty(M * N * 16, dtype=torch.uint8, device="cuda").fill_(0xA5)
        del junk
        outs.append((y, yq, ys))
    torch.cuda.synchronize()
    for y, yq, ys in outs:
        assert torch.equal(y, ref) and torch.equal(yq, refq) and torch.equal(ys, refs)


def test_small_m_matches_exact_integer_case(gpu_lib):
    """Integer operands with +-7 anchors (every scale 2^-6): the split-K sums
    are exact, so the small-M forward equals the int64 matmul bit for bit."""
    M, N, K = 48, 256, 2048
    rng = np.random.default_rng(5)
    def anchored(rows, cols):
        v = rng.integers(-7, 8, size=(rows, cols)).astype(np.float32)
        v[:, ::128] = 7.0
        return v
    x, w = anchored(M, K), anchored(N, K)
    w[np.arange(N)[:, None] % 128 == np.arange(K)[None, :] % 128] = -7.0
    xq, xs = gpu_lib.jet_quant_act_1x128(dev_bf16(x))
    wq, ws, _ = gpu_lib.jet_quant_weight_128x128(dev_bf16(w), transposed=False)
    y = gpu_lib.jet_fp8_linear_fwd(xq, xs, wq, ws, out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert np.all(host(xs) == np.float32(2.0 ** -6)) and np.all(host(ws) == np.float32(2.0 ** -6))
    assert_bits_equal(host(y), (x.astype(np.int64) @ w.astype(np.int64).T).astype(np.float32),
                      "small-M integer fwd")


# --- Llama-3.1-8B shapes ----------------------------------------------------

LLAMA = {"qkv": (6144, 4096), "o": (4096, 4096), "gate_up": (28672, 4096), "down": (4096, 14336)}


@pytest.mark.parametrize("name", list(LLAMA))
def test_decode_forward_llama_shapes(gpu_lib, name):
    """Rollout decode: M=64 tokens, forward only, full check."""
    N, K = LLAMA[name]
    M = 64
    x = inputs.activations_with_outliers(M, K, seed=0)
    w = inputs.normal_bf16((N, K), 0.02, seed=0, tensor_id=inputs.ID_W)
    xq, xs = gpu_lib.jet_quant_act_1x128(dev_bf16(x))
    wq, ws, _ = gpu_lib.jet_quant_weight_128x128(dev_bf16(w), transposed=False)
    y = gpu_lib.jet_fp8_linear_fwd(xq, xs, wq, ws)
    torch.cuda.synchronize()
    q1, s1 = O.quant_1x128(x)
    assert_bits_equal(host(xq), q1, "decode x codes")
    rng = np.random.default_rng(N)
    cols = np.sort(rng.choice(N, 512, replace=False))
    wsub = w[cols]
    # oracle on 512 sampled output columns: their weight rows re-quantized by block
    wq_h, ws_h = host(wq), host(ws)
    b = O.e4m3_decode(wq_h[cols]) * np.repeat(ws_h[cols // 128], 128, axis=1)
    a = O.dequant_1x128(q1, s1)
    check_bf16_output(host(y)[:, cols], a @ b.T, oracle_absprod(a, b), f"decode fwd {name}")
    del wsub


@pytest.mark.parametrize("name", list(LLAMA))
def test_training_shapes_sampled(gpu_lib, name):
    """Training M=8192, every Llama-3.1-8B linear: all three GEMMs at full
    size with FP32 scales, checked on sampled rows."""
    N, K = LLAMA[name]
    M = 8192
    x, w, dy = layer_inputs(M, N, K, 0)
    xd, wd, dyd = dev_bf16(x), dev_bf16(w), dev_bf16(dy)
    xq, xs = gpu_lib.jet_quant_act_1x128(xd)
    wq, ws, wqT = gpu_lib.jet_quant_weight_128x128(wd)
    dyq, dys = gpu_lib.jet_quant_act_1x128(dyd)
    dyqT, dysT = gpu_lib.jet_quant_act_128x1_T(dyd)
    xqT, xsT = gpu_lib.jet_quant_act_128x1_T(xq, src_s=xs)
    y, yq, ys = gpu_lib.jet_fp8_linear_fwd(xq, xs, wq, ws, fuse_quant=True)
    dx = gpu_lib.jet_fp8_linear_dgrad(dyq, dys, wqT, ws)
    dw = gpu_lib.jet_fp8_linear_wgrad(dyqT, dysT, xqT, xsT, M)
    torch.cuda.synchronize()
    rng = np.random.default_rng(5)
    rows = np.sort(rng.choice(M, 64, replace=False))
    ridx = torch.from_numpy(rows).cuda()
    # quantizer parity on the sampled rows, then GEMM rows from the GPU's codes
    qx, sx = O.quant_1x128(x[rows])
    assert_bits_equal(host(xq[ridx]), qx, "x codes")
    qd, sd = O.quant_1x128(dy[rows])
    assert_bits_equal(host(dyq[ridx]), qd, "dy codes")
    wq_h, ws_h = host(wq), host(ws)
    bw = O.dequant_128x128(wq_h, ws_h)
    ax = O.dequant_1x128(qx, sx)
    check_bf16_output(host(y[ridx]), ax @ bw.T, oracle_absprod(ax, bw), f"fwd {name}")
    qo, so = O.quant_1x128(host(y[ridx]))
    assert_bits_equal(host(yq[ridx]), qo, "fused codes")
    assert_bits_equal(host(ys[:, ridx]), so, "fused scales")
    ad = O.dequant_1x128(qd, sd)
    check_bf16_output(host(dx[ridx]), ad @ bw, oracle_absprod(ad, bw.T), f"dgrad {name}")
    del bw
    # wgrad: 64 sampled output rows n, all k, from the GPU's 128x1 codes
    nrows = np.sort(rng.choice(N, 64, replace=False))
    nidx = torch.from_numpy(nrows).cuda()
    a = O.dequant_128x1_T(host(dyqT[nidx]), host(dysT[:, nidx]), M)
    b = O.dequant_128x1_T(host(xqT), host(xsT), M)
    check_f32_output(host(dw[nidx]), a @ b.T, oracle_absprod(a, b), f"wgrad {name}")


# --- grids of big tiles that end in a partial wave ----------------------------

@pytest.mark.parametrize("pow2", [False, True])
@pytest.mark.parametrize("M,N", [(4096, 4352), (4352, 3968)])
def test_partial_wave_split_gemms(gpu_lib, pow2, M, N):
    """Layers whose grids of 256 x 256 tiles end in a partial wave on 256
    CUs.  4096 tokens, 4096 -> 4352: the forward's 16 x 17 grid runs as 16 x
    16 big tiles plus the last 256 output columns in 128 x 128 tiles, and
    wgrad's 17 x 16 grid as 16 x 16 big tiles plus the last 256 output rows
    in small ones.  4352 tokens, 4096 -> 3968 (N not a multiple of the
    256-column tile): the forward's 17 x 16 grid as 16 x 16 big tiles plus
    the last 256 token rows in small ones.  BF16 forward with its fused 1x128 output, FP32
    forward and FP32 wgrad (also accumulating) against the oracle on sampled
    rows, half of them in the last 256 rows of each output."""
    J = gpu_lib
    K = 4096
    x, w, dy = layer_inputs(M, N, K, 3)
    xd, wd, dyd = dev_bf16(x), dev_bf16(w), dev_bf16(dy)
    if pow2:
        xq, xs, xqT, xsT = J.jet_quant_act_1x128_128x1_T_pow2(xd, True)
        dyq, dys, dyqT, dysT = J.jet_quant_act_1x128_128x1_T_pow2(dyd, False)
        wq, ws, wqT = J.jet_quant_weight_128x128_pow2(wd)
        fwd, wgrad = J.jet_fp8_linear_fwd_pow2, J.jet_fp8_linear_wgrad_pow2
    else:
        xq, xs, xqT, xsT = J.jet_quant_act_1x128_128x1_T(xd, True)
        dyq, dys, dyqT, dysT = J.jet_quant_act_1x128_128x1_T(dyd, False)
        wq, ws, wqT = J.jet_quant_weight_128x128(wd)
        fwd, wgrad = J.jet_fp8_linear_fwd, J.jet_fp8_linear_wgrad
    y, yq, ys = fwd(xq, xs, wq, ws, fuse_quant=True)
    y32 = fwd(xq, xs, wq, ws, out_dtype=torch.float32)
    dw = wgrad(dyqT, dysT, xqT, xsT, M)
    dw2 = dw.clone()
    wgrad(dyqT, dysT, xqT, xsT, M, dw=dw2, accumulate=True)
    torch.cuda.synchronize()
    del xd, wd, dyd
    rng = np.random.default_rng(9)
    last256 = lambda n: np.sort(np.concatenate([rng.choice(n - 256, 16, replace=False),
                                                n - 256 + rng.choice(256, 16, replace=False)]))
    rows = last256(M)
    ridx = torch.from_numpy(rows).cuda()
    bw = O.dequant_128x128(host(wq), host(ws))
    ax = O.dequant_1x128(host(xq[ridx]), host(xs[:, ridx]))
    ref, absp = ax @ bw.T, oracle_absprod(ax, bw)
    tag = "pow2" if pow2 else "fp32 scales"
    check_bf16_output(host(y[ridx]), ref, absp, f"split fwd bf16 {tag}")
    check_f32_output(host(y32[ridx]), ref, absp, f"split fwd f32 {tag}")
    quant = P.quant_1x128_pow2 if pow2 else O.quant_1x128
    qo, so = quant(host(y[ridx]))
    assert_bits_equal(host(yq[ridx]), qo, f"split fused codes {tag}")
    assert_bits_equal(host(ys[:, ridx]), so, f"split fused scales {tag}")
    del bw
    nrows = last256(N)
    nidx = torch.from_numpy(nrows).cuda()
    a = O.dequant_128x1_T(host(dyqT[nidx]), host(dysT[:, nidx]), M)
    b = O.dequant_128x1_T(host(xqT), host(xsT), M)
    ref, absp = a @ b.T, oracle_absprod(a, b)
    check_f32_output(host(dw[nidx]), ref, absp, f"split wgrad {tag}")
    check_f32_output(host(dw2[nidx]), 2 * ref, 2 * absp, f"split wgrad accumulate {tag}")


# --- Qwen-14B/32B shapes at M=16384 (sampled) ---------------------------------

# (N, K): hidden 5120; QKV with 40 query and 8 key/value heads of 128; the
# fused gate+up projections of the 14B (intermediate 17408) and 32B (27648)
# models and their down projections.
QWEN = {"qkv": (7168, 5120), "o": (5120, 5120), "gate_up_14b": (34816, 5120),
        "gate_up_32b": (55296, 5120), "down_14b": (5120, 17408), "down_32b": (5120, 27648)}


@pytest.mark.parametrize("name", list(QWEN))
def test_qwen_shapes_sampled(gpu_lib, name):
    """Every Qwen-14B/32B-shaped linear at M=16384 training tokens: the step's
    quantizers (both activation groupings from one read) and all three GEMMs
    at full size, checked on sampled rows and columns against the oracle."""
    N, K = QWEN[name]
    M = 16384
    x, w, dy = layer_inputs(M, N, K, 3)
    xd, wd, dyd = dev_bf16(x), dev_bf16(w), dev_bf16(dy)
    xq, xs, xqT, xsT = gpu_lib.jet_quant_act_1x128_128x1_T(xd, True)
    dyq, dys, dyqT, dysT = gpu_lib.jet_quant_act_1x128_128x1_T(dyd, False)
    wq, ws, wqT = gpu_lib.jet_quant_weight_128x128(wd)
    y, yq, ys = gpu_lib.jet_fp8_linear_fwd(xq, xs, wq, ws, fuse_quant=True)
    dx = gpu_lib.jet_fp8_linear_dgrad(dyq, dys, wqT, ws)
    dw = gpu_lib.jet_fp8_linear_wgrad(dyqT, dysT, xqT, xsT, M)
    torch.cuda.synchronize()
    del xd, wd, dyd
    rng = np.random.default_rng(17)
    rows = np.sort(rng.choice(M, 32, replace=False))
    ncols = np.sort(rng.choice(N, 256, replace=False))
    kcols = np.sort(rng.choice(K, 256, replace=False))
    ridx, nidx, kidx = (torch.from_numpy(a).cuda() for a in (rows, ncols, kcols))
    # quantizers on the sampled rows (1x128) and one 128-row group (128x1)
    qx, sx = O.quant_1x128(x[rows])
    assert_bits_equal(host(xq[ridx]), qx, "x codes")
    assert_bits_equal(host(xs[:, ridx]), sx, "x scales")
    qd, sd = O.quant_1x128(dy[rows])
    assert_bits_equal(host(dyq[ridx]), qd, "dy codes")
    g = int(rng.integers(0, M // 128))
    gs = slice(g * 128, g * 128 + 128)
    cq, cs = O.quant_1x128(x[gs])
    rq, rs = O.requant_128x1_T_from_1x128(cq, cs)
    assert_bits_equal(host(xqT[:, gs]), rq, "x 128x1 codes")
    assert_bits_equal(host(xsT[g]), rs[0], "x 128x1 scales")
    tq, ts = O.quant_128x1_T(dy[gs])
    assert_bits_equal(host(dyqT[:, gs]), tq, "dy 128x1 codes")
    bi, bj = int(rng.integers(0, N // 128)), int(rng.integers(0, K // 128))
    wb = w[bi * 128:(bi + 1) * 128, bj * 128:(bj + 1) * 128]
    wqo, wso = O.quant_128x128(wb)
    assert_bits_equal(host(wq[bi * 128:(bi + 1) * 128, bj * 128:(bj + 1) * 128]), wqo, "w block codes")
    del x, w, dy
    # GEMMs from the GPU's own codes, on sampled rows x sampled columns
    wq_h, ws_h = host(wq), host(ws)
    bw_n = O.e4m3_decode(wq_h[ncols]) * np.repeat(ws_h[ncols // 128], 128, axis=1)          # [256, K]
    ax = O.dequant_1x128(qx, sx)
    check_bf16_output(host(y[ridx][:, nidx]), ax @ bw_n.T, oracle_absprod(ax, bw_n), f"fwd {name}")
    qo, so = O.quant_1x128(host(y[ridx]))
    assert_bits_equal(host(yq[ridx]), qo, "fused codes")
    bw_k = (O.e4m3_decode(wq_h[:, kcols]) * np.repeat(ws_h[:, kcols // 128], 128, axis=0)).T  # [256, N]
    ad = O.dequant_1x128(qd, sd)
    check_bf16_output(host(dx[ridx][:, kidx]), ad @ bw_k.T, oracle_absprod(ad, bw_k), f"dgrad {name}")
    del wq_h, bw_n, bw_k
    a = O.dequant_128x1_T(host(dyqT[nidx[:32]]), host(dysT[:, nidx[:32]]), M)
    b = O.dequant_128x1_T(host(xqT[kidx]), host(xsT[:, kidx]), M)
    check_f32_output(host(dw[nidx[:32]][:, kidx]), a @ b.T, oracle_absprod(a, b), f"wgrad {name}")


# --- batch invariance (rollout rows == training rows, bit for bit) ------------

@pytest.mark.parametrize("name", list(LLAMA))
def test_batch_invariant_forward_matches_training_batch(gpu_lib, name):
    """Rows computed by jet_fp8_linear_fwd_batch_invariant in a rollout-sized
    batch (M = 1, 37, 64, 128: the weight-streaming kernel) equal the same rows
    computed in a training-sized batch (M = 2048: the tiled kernel), bit for
    bit: BF16 Y, its fused 1x128 codes and scales, and FP32 Y.  The default
    split-K forward of the same rows stays within the GEMM tolerance but is not
    bit-identical; its mismatch is reported."""
    N, K = LLAMA[name]
    Mb = 2048
    x = inputs.activations_with_outliers(Mb, K, seed=11)
    w = inputs.normal_bf16((N, K), 0.02, seed=11, tensor_id=inputs.ID_W)
    xq, xs = gpu_lib.jet_quant_act_1x128(dev_bf16(x))
    wq, ws, _ = gpu_lib.jet_quant_weight_128x128(dev_bf16(w), transposed=False)
    yb, yqb, ysb = gpu_lib.jet_fp8_linear_fwd(xq, xs, wq, ws, fuse_quant=True)
    y32b = gpu_lib.jet_fp8_linear_fwd(xq, xs, wq, ws, out_dtype=torch.float32)
    report = []
    for M, r0 in ((1, 5), (37, 100), (64, 1000), (128, 1900)):
        rows = slice(r0, r0 + M)
        xq_s, xs_s = xq[rows].contiguous(), xs[:, rows].contiguous()
        y, yq, ys = gpu_lib.jet_fp8_linear_fwd_batch_invariant(xq_s, xs_s, wq, ws, fuse_quant=True)
        y32 = gpu_lib.jet_fp8_linear_fwd_batch_invariant(xq_s, xs_s, wq, ws, out_dtype=torch.float32)
        y_split = gpu_lib.jet_fp8_linear_fwd(xq_s, xs_s, wq, ws, out_dtype=torch.float32)
        torch.cuda.synchronize()
        assert torch.equal(y, yb[rows]), f"{name} M={M}: BF16 rows differ from the training batch"
        assert torch.equal(yq, yqb[rows]) and torch.equal(ys, ysb[:, rows]), f"{name} M={M}: fused codes differ"
        assert torch.equal(y32, y32b[rows]), f"{name} M={M}: FP32 rows differ from the training batch"
        diff = (y_split - y32b[rows]).abs()
        report.append(f"M={M}: split-K differs in {int((diff > 0).sum())}/{diff.numel()} elements, "
                      f"max {float(diff.max()):.2e}")
    print(f"{name}: " + "; ".join(report))


@pytest.mark.parametrize("K", [384, 1152, 8320])
def test_batch_invariant_forward_odd_k_steps(gpu_lib, K):
    """The 16-row weight-streaming groups load two K steps per ring stage; an
    odd number of K steps (3, 9, and 65 on the 64-column path for long
    contractions) leaves a last stage with one step.  Rows of the
    batch-invariant forward at M = 1, 16 and 37 still equal those of the
    training-sized batch bit for bit, and the result meets the GEMM
    tolerance against the oracle."""
    N, Mb = 256, 512
    x = inputs.activations_with_outliers(Mb, K, seed=K)
    w = inputs.normal_bf16((N, K), 0.02, seed=K, tensor_id=inputs.ID_W)
    xq, xs = gpu_lib.jet_quant_act_1x128(dev_bf16(x))
    wq, ws, _ = gpu_lib.jet_quant_weight_128x128(dev_bf16(w), transposed=False)
    yb, yqb, ysb = gpu_lib.jet_fp8_linear_fwd(xq, xs, wq, ws, fuse_quant=True)
    y32b = gpu_lib.jet_fp8_linear_fwd(xq, xs, wq, ws, out_dtype=torch.float32)
    for M, r0 in ((1, 3), (16, 40), (37, 300)):
        rows = slice(r0, r0 + M)
        xq_s, xs_s = xq[rows].contiguous(), xs[:, rows].contiguous()
        y, yq, ys = gpu_lib.jet_fp8_linear_fwd_batch_invariant(xq_s, xs_s, wq, ws, fuse_quant=True)
        y32 = gpu_lib.jet_fp8_linear_fwd_batch_invariant(xq_s, xs_s, wq, ws, out_dtype=torch.float32)
        torch.cuda.synchronize()
        tag = f"K={K} M={M}"
        assert torch.equal(y, yb[rows]), f"{tag}: BF16 rows differ from the training batch"
        assert torch.equal(yq, yqb[rows]) and torch.equal(ys, ysb[:, rows]), f"{tag}: fused codes differ"
        assert torch.equal(y32, y32b[rows]), f"{tag}: FP32 rows differ from the training batch"
        a = O.dequant_1x128(host(xq_s), host(xs_s))
        b = O.dequant_128x128(host(wq), host(ws))
        check_f32_output(host(y32), a @ b.T, oracle_absprod(a, b), f"invariant fwd f32 {tag}")


@pytest.mark.parametrize("pow2", [False, True])
def test_empty_batch_every_entry_point(gpu_lib, pow2):
    """M = 0 tokens (an empty rollout or micro-batch): every quantizer and GEMM
    entry point returns JET_OK with empty outputs and launches nothing; the
    library then still serves an ordinary call."""
    J, sfx = gpu_lib, ("_pow2" if pow2 else "")
    f = lambda name: getattr(J, name + sfx)
    N, K = 256, 384
    x, w, dy = layer_inputs(3, N, K, 21)
    wq, ws, wqT = f("jet_quant_weight_128x128")(dev_bf16(w))
    x0 = torch.empty((0, K), dtype=torch.bfloat16, device="cuda")
    dy0 = torch.empty((0, N), dtype=torch.bfloat16, device="cuda")
    xq, xs = f("jet_quant_act_1x128")(x0)
    assert xq.shape == (0, K) and xs.shape == (K // 128, 0)
    for requant in (False, True):
        q, s, qT, sT = f("jet_quant_act_1x128_128x1_T")(x0, requant)
        assert q.shape == (0, K) and qT.shape == (K, 0) and sT.shape == (0, K)
    qT, sT = f("jet_quant_act_128x1_T")(x0)
    assert qT.shape == (K, 0) and sT.shape == (0, K)
    qT, sT = f("jet_quant_act_128x1_T")(xq, src_s=xs)
    assert qT.shape == (K, 0)
    y, yq, ys = f("jet_fp8_linear_fwd")(xq, xs, wq, ws, fuse_quant=True)
    assert y.shape == (0, N) and yq.shape == (0, N) and ys.shape == (N // 128, 0)
    assert f("jet_fp8_linear_fwd")(xq, xs, wq, ws, out_dtype=torch.float32).shape == (0, N)
    if not pow2:
        assert J.jet_fp8_linear_fwd_batch_invariant(xq, xs, wq, ws).shape == (0, N)
    dyq, dys = f("jet_quant_act_1x128")(dy0)
    assert f("jet_fp8_linear_dgrad")(dyq, dys, wqT, ws).shape == (0, K)
    torch.cuda.synchronize()
    # ordinary calls afterwards: no error was left behind
    if pow2:
        xq3, xs3 = f("jet_quant_act_1x128")(dev_bf16(x))
        y3 = f("jet_fp8_linear_fwd")(xq3, xs3, wq, ws)
        torch.cuda.synchronize()
        assert y3.shape == (3, N) and torch.isfinite(y3.float()).all()
    else:
        quantize_all(J, x, w, dy)   # asserts bit-exact codes and scales
