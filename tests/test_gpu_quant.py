"""GPU parity of the three quantizers against the oracle: codes and scales
must be bit-exact.  Shapes span several tiles and ragged tails; inputs include
the hard cases of gpu_helpers.edge_matrix and the full Llama-3.1-8B sizes
(checked on sampled groups)."""
import numpy as np
import pytest
import torch

from oracle import jet_oracle as O
from fp8_blockwise_quantized_amd import inputs
from tests.gpu_helpers import assert_bits_equal, dev_bf16, edge_matrix, host

pytestmark = pytest.mark.gpu

RAGGED_M = [1, 63, 64, 65, 127, 128, 129, 200, 256]


def test_e4m3_packing_order_and_ties(gpu_lib):
    # amax 448 -> r = 1: the codes are the plain encodings of the inputs
    x = np.zeros((2, 128), np.float32)
    x[0, :8] = [448.0, 1.0, 2.0, 3.0, -0.5, -0.0, 168.0, 2.0 ** -10]
    x[1, :4] = [-448.0, 1.5 * 2.0 ** -9, 464.0 / 2, 0.0]
    q, s = gpu_lib.jet_quant_act_1x128(dev_bf16(x))
    torch.cuda.synchronize()
    qo, so = O.quant_1x128(x)
    assert_bits_equal(host(q), qo, "codes")
    assert_bits_equal(host(s), so, "scales")


@pytest.mark.parametrize("M", RAGGED_M)
def test_quant_1x128_parity(gpu_lib, M):
    K = 512
    x = inputs.normal_bf16((M, K), 1.0, seed=M, tensor_id=inputs.ID_X)
    q, s = gpu_lib.jet_quant_act_1x128(dev_bf16(x))
    torch.cuda.synchronize()
    qo, so = O.quant_1x128(x)
    assert_bits_equal(host(q), qo, f"1x128 codes M={M}")
    assert_bits_equal(host(s), so, f"1x128 scales M={M}")


def test_quant_1x128_edge_values_and_strided_input(gpu_lib):
    x = edge_matrix(512)
    wide = np.zeros((x.shape[0], 768), np.float32)
    wide[:, 128:640] = x
    xd = dev_bf16(wide)[:, 128:640]                        # ldx = 768 > K
    qbuf = torch.zeros((x.shape[0], 528), dtype=torch.uint8, device="cuda")   # ldq = 528
    q, s = gpu_lib.jet_quant_act_1x128(xd, q=qbuf[:, :512])
    torch.cuda.synchronize()
    qo, so = O.quant_1x128(x)
    assert_bits_equal(host(q), qo, "edge codes")
    assert_bits_equal(host(s), so, "edge scales")
    assert not host(qbuf)[:, 512:].any(), "write outside the row"


def test_quant_1x128_outliers(gpu_lib):
    x = inputs.activations_with_outliers(300, 4096, seed=0)
    q, s = gpu_lib.jet_quant_act_1x128(dev_bf16(x))
    torch.cuda.synchronize()
    qo, so = O.quant_1x128(x)
    assert_bits_equal(host(q), qo, "outlier codes")
    assert_bits_equal(host(s), so, "outlier scales")


@pytest.mark.parametrize("N,K", [(128, 128), (256, 512), (384, 256)])
def test_quant_weight_parity(gpu_lib, N, K):
    w = inputs.normal_bf16((N, K), 0.02, seed=N + K, tensor_id=inputs.ID_W)
    if N == 256:
        e = edge_matrix(K)
        w[:e.shape[0]] = e                                # edge rows in the first block row
    q, s, qT = gpu_lib.jet_quant_weight_128x128(dev_bf16(w))
    torch.cuda.synchronize()
    qo, so = O.quant_128x128(w)
    assert_bits_equal(host(q), qo, "weight codes")
    assert_bits_equal(host(s), so, "weight scales")
    assert_bits_equal(host(qT), qo.T, "transposed weight codes")


@pytest.mark.parametrize("M", RAGGED_M)
def test_quant_128x1_T_bf16_parity(gpu_lib, M):
    K = 384
    x = inputs.normal_bf16((M, K), 1e-3, seed=M, tensor_id=inputs.ID_DY)
    if M >= 9:
        x[:9] = edge_matrix(K)[:, :K]
    Mp = -(-M // 128) * 128
    qbuf = torch.full((K, Mp + 16), 0xAB, dtype=torch.uint8, device="cuda")
    qT, sT = gpu_lib.jet_quant_act_128x1_T(dev_bf16(x), qT=qbuf[:, :Mp])
    torch.cuda.synchronize()
    qo, so = O.quant_128x1_T(x)
    assert_bits_equal(host(qT), qo, f"128x1 codes M={M}")
    assert_bits_equal(host(sT), so, f"128x1 scales M={M}")
    assert np.all(host(qbuf)[:, Mp:] == 0xAB), "write past the padded row"


@pytest.mark.parametrize("M", RAGGED_M)
@pytest.mark.parametrize("K", [384, 512])
def test_quant_128x1_T_requant_from_fp8_parity(gpu_lib, M, K):
    x = inputs.activations_with_outliers(M, K, seed=M + K)
    if M >= 9:
        x[:9] = edge_matrix(K)
    xq, xs = gpu_lib.jet_quant_act_1x128(dev_bf16(x))
    qT, sT = gpu_lib.jet_quant_act_128x1_T(xq, src_s=xs)
    torch.cuda.synchronize()
    q1, s1 = O.quant_1x128(x)
    assert_bits_equal(host(xq), q1, "1x128 codes")
    qo, so = O.requant_128x1_T_from_1x128(q1, s1)
    assert_bits_equal(host(qT), qo, f"requant codes M={M} K={K}")
    assert_bits_equal(host(sT), so, f"requant scales M={M} K={K}")


@pytest.mark.parametrize("M", RAGGED_M)
@pytest.mark.parametrize("requant", [False, True])
def test_quant_1x128_128x1_T_parity(gpu_lib, M, requant):
    """One read, both groupings: the 1x128 outputs equal quant_1x128 and the
    128x1 outputs quant_128x1_T of the BF16 values (output gradients) or of
    the dequantized 1x128 values (activations), bit for bit."""
    K = 512
    x = inputs.activations_with_outliers(M, K, seed=M + 7)
    if M >= 9:
        x[:9] = edge_matrix(K)
    Mp = -(-M // 128) * 128
    qbuf = torch.full((K, Mp + 16), 0xAB, dtype=torch.uint8, device="cuda")
    q, s, qT, sT = gpu_lib.jet_quant_act_1x128_128x1_T(dev_bf16(x), requant, qT=qbuf[:, :Mp])
    torch.cuda.synchronize()
    q1, s1 = O.quant_1x128(x)
    assert_bits_equal(host(q), q1, f"1x128 codes M={M}")
    assert_bits_equal(host(s), s1, f"1x128 scales M={M}")
    qo, so = O.requant_128x1_T_from_1x128(q1, s1) if requant else O.quant_128x1_T(x)
    assert_bits_equal(host(qT), qo, f"128x1 codes M={M} requant={requant}")
    assert_bits_equal(host(sT), so, f"128x1 scales M={M} requant={requant}")
    assert np.all(host(qbuf)[:, Mp:] == 0xAB), "write past the padded row"


def test_quantizers_deterministic(gpu_lib):
    x = dev_bf16(inputs.activations_with_outliers(1000, 1024, seed=3))
    a = [gpu_lib.jet_quant_act_1x128(x) for _ in range(2)]
    b = [gpu_lib.jet_quant_act_128x1_T(x) for _ in range(2)]
    torch.cuda.synchronize()
    assert torch.equal(a[0][0], a[1][0]) and torch.equal(a[0][1], a[1][1])
    assert torch.equal(b[0][0], b[1][0]) and torch.equal(b[0][1], b[1][1])


# --- full Llama-3.1-8B sizes, sampled groups --------------------------------

@pytest.mark.parametrize("M,K", [(8192, 4096), (8192, 14336)])
def test_full_size_activation_quantizers_sampled(gpu_lib, M, K):
    x = inputs.activations_with_outliers(M, K, seed=0)
    xd = dev_bf16(x)
    xq, xs = gpu_lib.jet_quant_act_1x128(xd)
    qT, sT = gpu_lib.jet_quant_act_128x1_T(xq, src_s=xs)
    torch.cuda.synchronize()
    rng = np.random.default_rng(M + K)
    rows = np.sort(rng.choice(M, 256, replace=False))
    qo, so = O.quant_1x128(x[rows])
    assert_bits_equal(host(xq[torch.from_numpy(rows).cuda()]), qo, "sampled 1x128 codes")
    assert_bits_equal(host(xs[:, torch.from_numpy(rows).cuda()]), so, "sampled 1x128 scales")
    # re-quantization: two 128-row groups, 512 columns, from the GPU's own 1x128 output
    xq_h, xs_h = host(xq), host(xs)
    for g in rng.choice(M // 128, 2, replace=False):
        c0 = int(rng.integers(0, K // 128 - 3)) * 128
        sl = slice(g * 128, g * 128 + 128)
        qo, so = O.requant_128x1_T_from_1x128(xq_h[sl, c0:c0 + 512], xs_h[c0 // 128:c0 // 128 + 4, sl])
        assert_bits_equal(host(qT[c0:c0 + 512, g * 128:(g + 1) * 128]), qo, "sampled requant codes")
        assert_bits_equal(host(sT[g, c0:c0 + 512]), so[0], "sampled requant scales")


@pytest.mark.parametrize("N,K", [(28672, 4096), (4096, 14336)])
def test_full_size_weight_quantizer_sampled(gpu_lib, N, K):
    w = inputs.normal_bf16((N, K), 0.02, seed=0, tensor_id=inputs.ID_W)
    q, s, qT = gpu_lib.jet_quant_weight_128x128(dev_bf16(w))
    torch.cuda.synchronize()
    rng = np.random.default_rng(N)
    for _ in range(4):
        bi, bj = int(rng.integers(0, N // 128)), int(rng.integers(0, K // 128))
        rs, cs = slice(bi * 128, bi * 128 + 128), slice(bj * 128, bj * 128 + 128)
        qo, so = O.quant_128x128(w[rs, cs])
        assert_bits_equal(host(q[rs, cs]), qo, "sampled weight codes")
        assert_bits_equal(host(s[bi:bi + 1, bj:bj + 1]), so, "sampled weight scale")
        assert_bits_equal(host(qT[cs, rs]), qo.T, "sampled transposed codes")


def test_full_size_dy_128x1_sampled(gpu_lib):
    M, N = 8192, 6144
    dy = inputs.normal_bf16((M, N), 1e-3, seed=0, tensor_id=inputs.ID_DY)
    qT, sT = gpu_lib.jet_quant_act_128x1_T(dev_bf16(dy))
    torch.cuda.synchronize()
    rng = np.random.default_rng(1)
    for g in rng.choice(M // 128, 3, replace=False):
        sl = slice(g * 128, g * 128 + 128)
        qo, so = O.quant_128x1_T(dy[sl])
        assert_bits_equal(host(qT[:, sl]), qo, "sampled dY 128x1 codes")
        assert_bits_equal(host(sT[g]), so[0], "sampled dY 128x1 scales")


@pytest.mark.parametrize("M,K,requant", [(8192, 4096, True), (8192, 14336, True), (8192, 6144, False)])
def test_full_size_both_groupings_match_separate_quantizers(gpu_lib, M, K, requant):
    """At full Llama sizes, the one-read quantizer equals the two separate
    quantizers on every byte (both are pinned to the oracle above), and a
    sampled 128-row group equals the oracle directly."""
    x = (inputs.activations_with_outliers(M, K, seed=1) if requant
         else inputs.normal_bf16((M, K), 1e-3, seed=1, tensor_id=inputs.ID_DY))
    xd = dev_bf16(x)
    q, s, qT, sT = gpu_lib.jet_quant_act_1x128_128x1_T(xd, requant)
    q1, s1 = gpu_lib.jet_quant_act_1x128(xd)
    qT1, sT1 = gpu_lib.jet_quant_act_128x1_T(q1, src_s=s1) if requant else gpu_lib.jet_quant_act_128x1_T(xd)
    torch.cuda.synchronize()
    assert torch.equal(q, q1) and torch.equal(s.view(torch.int32), s1.view(torch.int32))
    assert torch.equal(qT, qT1) and torch.equal(sT.view(torch.int32), sT1.view(torch.int32))
    g = int(np.random.default_rng(K).integers(0, M // 128))
    sl = slice(g * 128, g * 128 + 128)
    cq, cs = O.quant_1x128(x[sl])
    qo, so = O.requant_128x1_T_from_1x128(cq, cs) if requant else O.quant_128x1_T(x[sl])
    assert_bits_equal(host(qT[:, sl]), qo, "sampled group codes")
    assert_bits_equal(host(sT[g]), so[0], "sampled group scales")
