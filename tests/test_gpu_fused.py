"""GPU parity of the fused producers of the 1x128 input (RMSNorm and SwiGLU
fused with the quantization) against the oracle (oracle/fused_producers.py).

The bar:
  * codes and scales: bit-exact against the oracle's 1x128 quantization of the
    GPU's own BF16 output (both sides take the rounding decisions on the same
    BF16 values);
  * the BF16 output: within one BF16 spacing of the oracle's float64 value
    rounded to BF16 (elementwise).  The kernels compute in FP32 (RMSNorm: IEEE
    divide and square root, a 64-term per-lane sum then a butterfly for the
    mean square; SwiGLU: the hardware exp2 of -|g|*log2(e) and the hardware
    reciprocal, each within about 1 ulp), which stays within a few 2^-24
    relative of the exact value for the values that occur (the exp2 argument's
    rounding adds |g|*2^-24); BF16 keeps 8 bits, so the two roundings can
    differ only where the exact value lies that close to a BF16 midpoint, and
    then by one step.  Results below the FP32 normal range are allowed an
    absolute 2^-126.
"""
import numpy as np
import pytest
import torch

from oracle import fused_producers as F
from oracle import jet_oracle as O
from fp8_blockwise_quantized_amd import inputs
from tests.gpu_helpers import assert_bits_equal, dev_bf16, host

pytestmark = pytest.mark.gpu


def check_bf16_within_one_step(got, ref, what):
    got64, ref64 = np.asarray(got, np.float64), np.asarray(ref, np.float64)
    bad = np.abs(got64 - ref64) > np.maximum(F.bf16_ulp(ref64), 2.0 ** -126)
    if bad.any():
        i = np.argwhere(bad)[0]
        raise AssertionError(f"{what}: {int(bad.sum())} elements off by more than one BF16 step, "
                             f"first at {tuple(i)}: gpu {got64[tuple(i)]!r} oracle {ref64[tuple(i)]!r}")
    return int((got64 != ref64).sum())


def gamma_for(H, seed):
    return inputs.normal_bf16((H,), 0.1, seed=seed, tensor_id=inputs.ID_W) + np.float32(1.0)


# --- RMSNorm ----------------------------------------------------------------

@pytest.mark.parametrize("M,H", [(1, 128), (7, 384), (100, 4096), (33, 5120), (16, 8192), (9, 640)])
def test_rmsnorm_quant_parity(gpu_lib, M, H):
    x = inputs.activations_with_outliers(M, H, seed=M + H)
    g = O.bf16_rne(gamma_for(H, M))
    eps = 1e-5
    y, q, s = gpu_lib.jet_rmsnorm_quant_1x128(dev_bf16(x), dev_bf16(g), eps, return_y=True)
    q2, s2 = gpu_lib.jet_rmsnorm_quant_1x128(dev_bf16(x), dev_bf16(g), eps)
    torch.cuda.synchronize()
    yh = host(y)
    tag = f"M={M} H={H}"
    check_bf16_within_one_step(yh, F.rmsnorm_bf16(x, g, eps), f"rmsnorm y {tag}")
    qo, so = O.quant_1x128(yh)
    assert_bits_equal(host(q), qo, f"rmsnorm codes {tag}")
    assert_bits_equal(host(s), so, f"rmsnorm scales {tag}")
    assert torch.equal(q, q2) and torch.equal(s, s2), "the optional BF16 output changed the codes"


def test_rmsnorm_quant_strides_eps_and_extremes(gpu_lib):
    """A row stride wider than H (a column slice of a wider tensor), several
    eps values, and rows that are constant, tiny, huge or all zero (inside
    the FP32 range of the mean square: |x| below about 1e19)."""
    M, H, W = 12, 256, 384
    x = inputs.activations_with_outliers(M, W, seed=3)
    x[0] = 2.0 ** -60                  # tiny constant row (x^2 an exact FP32 denormal)
    x[1] = -1.0e18                     # huge constant row (sum of x^2 still below FP32's max)
    x[2] = 0.0                         # zero row: eps alone
    x[3, :H] = np.where(np.arange(H) % 2 == 0, 1.0, -1.0)
    x = O.bf16_rne(x)
    g = O.bf16_rne(gamma_for(H, 3))
    xd = dev_bf16(x)
    for eps in (0.0, 1e-6, 1e-5, 1.0):
        if eps == 0.0:
            rows = slice(0, 2)         # eps 0 divides by the row's own mean square: skip the zero row
        else:
            rows = slice(0, M)
        xs = xd[rows, :H]
        y, q, s = gpu_lib.jet_rmsnorm_quant_1x128(xs, dev_bf16(g), eps, return_y=True)
        torch.cuda.synchronize()
        yh = host(y)
        check_bf16_within_one_step(yh, F.rmsnorm_bf16(x[rows, :H], g, eps), f"rmsnorm y eps={eps}")
        qo, so = O.quant_1x128(yh)
        assert_bits_equal(host(q), qo, f"rmsnorm codes eps={eps}")
        assert_bits_equal(host(s), so, f"rmsnorm scales eps={eps}")


def test_rmsnorm_quant_full_size_sampled(gpu_lib):
    """Llama-3.1-8B hidden size at the training batch (M=8192, H=4096): the
    whole tensor on the GPU, 64 rows checked against the oracle."""
    M, H = 8192, 4096
    x = inputs.activations_with_outliers(M, H, seed=0)
    g = O.bf16_rne(gamma_for(H, 0))
    y, q, s = gpu_lib.jet_rmsnorm_quant_1x128(dev_bf16(x), dev_bf16(g), 1e-5, return_y=True)
    torch.cuda.synchronize()
    rows = np.sort(np.random.default_rng(1).choice(M, 64, replace=False))
    yh = host(y)[rows]
    check_bf16_within_one_step(yh, F.rmsnorm_bf16(x[rows], g, 1e-5), "rmsnorm y full size")
    qo, so = O.quant_1x128(yh)
    assert_bits_equal(host(q)[rows], qo, "rmsnorm codes full size")
    assert_bits_equal(host(s)[:, rows], so, "rmsnorm scales full size")


# --- SwiGLU -----------------------------------------------------------------

@pytest.mark.parametrize("M,I", [(1, 128), (5, 256), (100, 1536), (64, 14336), (37, 384)])
def test_swiglu_quant_parity(gpu_lib, M, I):
    gu = inputs.normal_bf16((M, 2 * I), 1.3, seed=M + I, tensor_id=inputs.ID_X)
    h, q, s = gpu_lib.jet_swiglu_quant_1x128(dev_bf16(gu), return_h=True)
    q2, s2 = gpu_lib.jet_swiglu_quant_1x128(dev_bf16(gu))
    torch.cuda.synchronize()
    hh = host(h)
    tag = f"M={M} I={I}"
    check_bf16_within_one_step(hh, F.swiglu_bf16(gu, I), f"swiglu h {tag}")
    qo, so = O.quant_1x128(hh)
    assert_bits_equal(host(q), qo, f"swiglu codes {tag}")
    assert_bits_equal(host(s), so, f"swiglu scales {tag}")
    assert torch.equal(q, q2) and torch.equal(s, s2), "the optional BF16 output changed the codes"


def test_swiglu_quant_extremes_and_stride(gpu_lib):
    """Gate values at 0, -0, very small, and large of both signs (where
    exp(-g) would overflow), with a row stride wider than 2I."""
    M, I, W = 6, 256, 640
    gu = inputs.normal_bf16((M, W), 1.0, seed=9, tensor_id=inputs.ID_X)
    special = np.array([0.0, -0.0, 1e-30, -1e-30, 80.0, -80.0, 100.0, -100.0, 30.0, -30.0,
                        1e4, -1e4, 1e30, -1e30, 5.0, -5.0], np.float32)
    gu[:, :16] = special
    gu[:, I:I + 16] = np.float32(2.0)
    gu = O.bf16_rne(gu)
    d = dev_bf16(gu)
    h, q, s = gpu_lib.jet_swiglu_quant_1x128(d[:, :2 * I], inter=I, return_h=True)
    torch.cuda.synchronize()
    hh = host(h)
    check_bf16_within_one_step(hh, F.swiglu_bf16(gu[:, :2 * I], I), "swiglu h extremes")
    qo, so = O.quant_1x128(hh)
    assert_bits_equal(host(q), qo, "swiglu codes extremes")
    assert_bits_equal(host(s), so, "swiglu scales extremes")
    assert np.all(hh[:, 0] == 0.0) and np.all(hh[:, 1] == 0.0), "silu(+-0) * up must be zero"


def test_swiglu_quant_full_size_sampled(gpu_lib):
    """Llama-3.1-8B MLP (I=14336) at the training batch (M=8192): the whole
    tensor on the GPU, 32 rows checked against the oracle."""
    M, I = 8192, 14336
    gu = inputs.normal_bf16((M, 2 * I), 1.3, seed=0, tensor_id=inputs.ID_X)
    h, q, s = gpu_lib.jet_swiglu_quant_1x128(dev_bf16(gu), return_h=True)
    torch.cuda.synchronize()
    rows = np.sort(np.random.default_rng(2).choice(M, 32, replace=False))
    hh = host(h)[rows]
    check_bf16_within_one_step(hh, F.swiglu_bf16(gu[rows], I), "swiglu h full size")
    qo, so = O.quant_1x128(hh)
    assert_bits_equal(host(q)[rows], qo, "swiglu codes full size")
    assert_bits_equal(host(s)[:, rows], so, "swiglu scales full size")


def test_fused_producers_match_unfused_quantizer(gpu_lib):
    """The fused output equals jet_quant_act_1x128 applied to the fused
    kernel's own BF16 output, on the GPU (bit for bit)."""
    x = inputs.activations_with_outliers(64, 4096, seed=5)
    g = O.bf16_rne(gamma_for(4096, 5))
    y, q, s = gpu_lib.jet_rmsnorm_quant_1x128(dev_bf16(x), dev_bf16(g), 1e-5, return_y=True)
    qq, ss = gpu_lib.jet_quant_act_1x128(y)
    gu = inputs.normal_bf16((64, 2 * 1536), 1.3, seed=5, tensor_id=inputs.ID_X)
    h, q2, s2 = gpu_lib.jet_swiglu_quant_1x128(dev_bf16(gu), return_h=True)
    qq2, ss2 = gpu_lib.jet_quant_act_1x128(h)
    torch.cuda.synchronize()
    assert torch.equal(q, qq) and torch.equal(s, ss)
    assert torch.equal(q2, qq2) and torch.equal(s2, ss2)
