"""jet_fp8_linear_fwd_noalloc: the forward with its split-K partial sums in the
library's static device scratch gives the bits of jet_fp8_linear_fwd (which
takes a caller's workspace) on consecutive calls, each smaller than the one
before, so every call meets the scratch holding the previous call's partial
sums.  Outputs are preallocated: the calls allocate nothing."""
import numpy as np
import pytest
import torch

from fp8_blockwise_quantized_amd import inputs
from tests.gpu_helpers import dev_bf16

pytestmark = pytest.mark.gpu

# (M, N, K): the largest scratch need the forward has (32 column blocks, eight
# K ranges: 16,777,216 bytes, the whole array), 127 column blocks in two
# ranges, the decode QKV shape at M = 128 and M = 64, a 16-range split, a
# one-range M <= 128 shape (256 column blocks, no scratch) and a large M (the
# tiled kernel, no scratch).
SHAPES = [(128, 4096, 4096), (128, 16256, 512), (128, 6144, 4096), (64, 6144, 4096), (37, 1024, 2048),
          (16, 32768, 1024), (300, 512, 1024)]


def _operands(J, M, N, K, seed):
    x = inputs.activations_with_outliers(M, K, seed=seed)
    w = inputs.normal_bf16((N, K), 0.02, seed=seed, tensor_id=inputs.ID_W)
    xq, xs = J.jet_quant_act_1x128(dev_bf16(x))
    wq, ws, _ = J.jet_quant_weight_128x128(dev_bf16(w), transposed=False)
    return xq, xs, wq, ws


def test_noalloc_forward_matches_the_workspace_forward(gpu_lib):
    J = gpu_lib
    needs = [J.jet_workspace_bytes(J.JET_OP_FWD, *s) for s in SHAPES]
    assert needs[0] == 16 << 20 and needs == sorted(needs, reverse=True) and needs[-2] == 0
    for fused in (True, False):
        for i, (M, N, K) in enumerate(SHAPES):
            print(f"noalloc case M={M} N={N} K={K} fused={fused}", flush=True)
            xq, xs, wq, ws = _operands(J, M, N, K, 40 + i)
            dt = torch.bfloat16 if fused else torch.float32
            y = torch.empty(M, N, dtype=dt, device="cuda")
            yq = torch.empty(M, N, dtype=torch.uint8, device="cuda") if fused else None
            ys = torch.empty(N // 128, M, dtype=torch.float32, device="cuda") if fused else None
            torch.cuda.synchronize()
            J.jet_fp8_linear_fwd_noalloc(xq, xs, wq, ws, y=y, out_dtype=dt, fuse_quant=fused, yq=yq, ys=ys)
            ref = J.jet_fp8_linear_fwd(xq, xs, wq, ws, out_dtype=dt, fuse_quant=fused)
            torch.cuda.synchronize()
            if fused:
                assert torch.equal(y, ref[0]), (M, N, K, "y")
                assert torch.equal(yq, ref[1]), (M, N, K, "yq")
                assert torch.equal(ys, ref[2]), (M, N, K, "ys")
            else:
                assert torch.equal(y, ref), (M, N, K, "y")


def test_noalloc_two_calls_second_smaller(gpu_lib):
    """Back to back on one stream with no synchronization between them: the
    second, smaller call reads only partial sums it wrote itself."""
    J = gpu_lib
    big, small = (128, 6144, 4096), (64, 2048, 4096)
    ops = [_operands(J, *big, 7), _operands(J, *small, 8)]
    outs = [torch.empty(s[0], s[1], dtype=torch.bfloat16, device="cuda") for s in (big, small)]
    torch.cuda.synchronize()
    for (xq, xs, wq, ws), y in zip(ops, outs):
        J.jet_fp8_linear_fwd_noalloc(xq, xs, wq, ws, y=y)
    refs = [J.jet_fp8_linear_fwd(*o) for o in ops]
    torch.cuda.synchronize()
    for y, r in zip(outs, refs):
        assert torch.equal(y, r)
    assert np.isfinite(outs[1].float().cpu().numpy()).all()
