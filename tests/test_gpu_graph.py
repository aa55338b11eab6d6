"""HIP-graph capture of whole steps: the dense layer's training step (FP32 and
power-of-two scales) and the KV cache's recalibration and append, captured
once and replayed three times with eager work and synchronizations between
the replays; every replay's outputs must equal the eager step's bit for bit
(the library records no memset and allocates nothing, so a captured step is
the eager step)."""
import numpy as np
import pytest
import torch

from fp8_blockwise_quantized_amd import inputs
from tests.gpu_helpers import dev_bf16

pytestmark = pytest.mark.gpu


def step_fns(J, x, w, dy, M, pow2):
    sfx = "_pow2" if pow2 else ""
    f = lambda name: getattr(J, name + sfx)
    N, K = w.shape
    e = lambda shape, dt: torch.empty(shape, dtype=dt, device="cuda")
    Mp = -(-M // 128) * 128
    o = dict(wq=e((N, K), torch.uint8), ws=e((N // 128, K // 128), torch.float32), wqT=e((K, N), torch.uint8),
             xq=e((M, K), torch.uint8), xs=e((K // 128, M), torch.float32),
             xqT=e((K, Mp), torch.uint8), xsT=e((Mp // 128, K), torch.float32),
             y=e((M, N), torch.bfloat16), yq=e((M, N), torch.uint8), ys=e((N // 128, M), torch.float32),
             dyq=e((M, N), torch.uint8), dys=e((N // 128, M), torch.float32),
             dyqT=e((N, Mp), torch.uint8), dysT=e((Mp // 128, N), torch.float32),
             dx=e((M, K), torch.bfloat16), dw=e((N, K), torch.float32))

    def run():
        f("jet_quant_weight_128x128")(w, q=o["wq"], s=o["ws"], qT=o["wqT"])
        f("jet_quant_act_1x128_128x1_T")(x, True, q=o["xq"], s=o["xs"], qT=o["xqT"], sT=o["xsT"])
        f("jet_fp8_linear_fwd")(o["xq"], o["xs"], o["wq"], o["ws"], y=o["y"], fuse_quant=True, yq=o["yq"],
                                ys=o["ys"])
        f("jet_quant_act_1x128_128x1_T")(dy, False, q=o["dyq"], s=o["dys"], qT=o["dyqT"], sT=o["dysT"])
        if pow2:
            J.jet_fp8_linear_dgrad_pow2(o["dyq"], o["dys"], o["wqT"], o["ws"], dx=o["dx"])
            J.jet_fp8_linear_wgrad_pow2(o["dyqT"], o["dysT"], o["xqT"], o["xsT"], M, dw=o["dw"])
        else:
            J.jet_fp8_linear_dgrad(o["dyq"], o["dys"], o["wqT"], o["ws"], dx=o["dx"])
            J.jet_fp8_linear_wgrad(o["dyqT"], o["dysT"], o["xqT"], o["xsT"], M, dw=o["dw"])
    return run, o


@pytest.mark.parametrize("pow2", [False, True])
def test_training_step_graph_replay(gpu_lib, pow2):
    J = gpu_lib
    M, N, K = 384, 512, 640
    x = dev_bf16(inputs.activations_with_outliers(M, K, seed=2))
    w = dev_bf16(inputs.normal_bf16((N, K), 0.02, seed=2, tensor_id=inputs.ID_W))
    dy = dev_bf16(inputs.normal_bf16((M, N), 1e-3, seed=2, tensor_id=inputs.ID_DY))
    run, o = step_fns(J, x, w, dy, M, pow2)
    run()
    torch.cuda.synchronize()
    eager = {k: v.clone() for k, v in o.items()}
    for v in o.values():
        v.zero_()
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        run()                                   # warm-up on the capture stream
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    for v in o.values():
        v.zero_()
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        run()
    for rep in range(3):
        for v in o.values():
            v.fill_(0) if v.dtype != torch.float32 else v.fill_(float("nan"))
        junk = torch.randn(1 << 20, device="cuda") * 3         # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for k in o:
            a, b = o[k], eager[k]
            if a.dtype in (torch.float32, torch.bfloat16):
                a, b = a.view(torch.int32 if a.dtype == torch.float32 else torch.int16), \
                    b.view(torch.int32 if b.dtype == torch.float32 else torch.int16)
            assert torch.equal(a, b), f"replay {rep}: {k} differs from the eager step (pow2={pow2})"
        del junk


def test_kv_cache_graph_replay(gpu_lib):
    J = gpu_lib
    T, D, rows = 300, 1024, 512
    rng = np.random.default_rng(1)
    k = dev_bf16(inputs.normal_bf16((T, D), 2.0, seed=4, tensor_id=inputs.ID_X))
    v = dev_bf16(inputs.normal_bf16((T, D), 0.5, seed=4, tensor_id=inputs.ID_DY))
    slots = torch.from_numpy(rng.permutation(rows)[:T].astype(np.int64)).cuda()
    sc = torch.empty(6, dtype=torch.float32, device="cuda")
    kc = torch.zeros((rows, D), dtype=torch.uint8, device="cuda")
    vc = torch.zeros((rows, D), dtype=torch.uint8, device="cuda")

    def run():
        J.jet_kv_calibrate(k, v, kv_scales=sc)
        J.jet_kv_append(k, v, slots, sc, kc, vc)
    run()
    torch.cuda.synchronize()
    e_sc, e_kc, e_vc = sc[:4].clone(), kc.clone(), vc.clone()
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        run()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        run()
    for rep in range(3):
        sc.fill_(float("nan"))
        kc.zero_()
        vc.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(sc[:4].view(torch.int32), e_sc.view(torch.int32)), f"replay {rep}: scales"
        assert torch.equal(kc, e_kc) and torch.equal(vc, e_vc), f"replay {rep}: cache rows"
