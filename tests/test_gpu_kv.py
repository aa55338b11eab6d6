"""GPU parity of the FP8 KV cache (recalibrated per-tensor scales,
quantize-and-append to slot rows) against the oracle (oracle/kv_cache.py):
scales and every cache byte bit-exact, rows without a valid slot untouched."""
import numpy as np
import pytest
import torch

from oracle import kv_cache as KV
from oracle import jet_oracle as O
from fp8_blockwise_quantized_amd import inputs
from tests.gpu_helpers import assert_bits_equal, dev_bf16, host

pytestmark = pytest.mark.gpu


def qkv_output(T, seed, q_cols=4096, d=1024):
    """A QKV projection output [T, q_cols + 2d] (Llama-8B: 32 query heads and 8
    KV heads of 128); K and V are its column slices."""
    y = inputs.normal_bf16((T, q_cols + 2 * d), 1.3, seed=seed, tensor_id=inputs.ID_X)
    y[:, q_cols:q_cols + d] *= np.float32(3.0)          # K and V with different ranges
    return O.bf16_rne(y)


def scales_host(kv_scales):
    s = host(kv_scales)
    return (np.float32(s[0]), np.float32(s[1])), (np.float32(s[2]), np.float32(s[3]))


@pytest.mark.parametrize("T", [0, 1, 37, 300])
def test_kv_calibrate_parity(gpu_lib, T):
    q, d = 4096, 1024
    y = qkv_output(T, seed=T + 1)
    yd = dev_bf16(y) if T else torch.zeros((0, q + 2 * d), dtype=torch.bfloat16, device="cuda")
    k, v = yd[:, q:q + d], yd[:, q + d:]
    sc = gpu_lib.jet_kv_calibrate(k, v)
    torch.cuda.synchronize()
    (sk, rk), (sv, rv) = scales_host(sc)
    (ok, ork), (ov, orv) = KV.kv_calibrate(y[:, q:q + d], y[:, q + d:])
    assert (sk, rk, sv, rv) == (ok, ork, ov, orv), f"T={T}: scales differ"


def test_kv_append_parity_slots_padding_and_saturation(gpu_lib):
    q, d, rows = 4096, 1024, 700
    rng = np.random.default_rng(3)
    y = qkv_output(300, seed=3)
    yd = dev_bf16(y)
    k, v = yd[:, q:q + d], yd[:, q + d:]
    sc = gpu_lib.jet_kv_calibrate(k, v)
    kc0 = rng.integers(0, 256, size=(rows, d), dtype=np.uint8)
    vc0 = rng.integers(0, 256, size=(rows, d), dtype=np.uint8)
    kc, vc = torch.from_numpy(kc0).cuda(), torch.from_numpy(vc0).cuda()
    slots = rng.permutation(rows)[:300].astype(np.int64)
    slots[[0, 5, 299]] = -1                               # padding tokens
    slots[[7, 8]] = [rows, rows + 1000]                   # outside the cache: skipped
    gpu_lib.jet_kv_append(k, v, torch.from_numpy(slots).cuda(), sc, kc, vc)
    torch.cuda.synchronize()
    (sk, rk), (sv, rv) = KV.kv_calibrate(y[:, q:q + d], y[:, q + d:])
    ok = np.where(slots < rows, slots, -1)
    assert_bits_equal(host(kc), KV.kv_append(kc0, y[:, q:q + d], ok, rk), "K cache after prefill")
    assert_bits_equal(host(vc), KV.kv_append(vc0, y[:, q + d:], ok, rv), "V cache after prefill")
    # a decode step: new tokens with the same (static) scales, some far beyond
    # the calibration range (saturate at +-448), written to fresh slots
    y2 = qkv_output(64, seed=4)
    y2[:8, q:q + d] *= np.float32(50.0)
    y2 = O.bf16_rne(y2)
    y2d = dev_bf16(y2)
    free = np.setdiff1d(np.arange(rows), ok[ok >= 0])
    slots2 = rng.choice(free, 64, replace=False).astype(np.int64)
    kc_before, vc_before = host(kc), host(vc)
    gpu_lib.jet_kv_append(y2d[:, q:q + d], y2d[:, q + d:], torch.from_numpy(slots2).cuda(), sc, kc, vc)
    torch.cuda.synchronize()
    assert_bits_equal(host(kc), KV.kv_append(kc_before, y2[:, q:q + d], slots2, rk), "K cache after decode")
    assert_bits_equal(host(vc), KV.kv_append(vc_before, y2[:, q + d:], slots2, rv), "V cache after decode")
    sat = host(kc)[slots2[:8]] & 0x7F
    assert np.any(sat == 0x7E), "the scaled-up tokens must saturate"


def test_kv_full_prefill_llama8b(gpu_lib):
    """Llama-3.1-8B layer at a prefill of 8192 tokens (8 KV heads x 128):
    recalibration and append, the whole cache compared."""
    q, d, T = 4096, 1024, 8192
    y = qkv_output(T, seed=0)
    yd = dev_bf16(y)
    k, v = yd[:, q:q + d], yd[:, q + d:]
    sc = gpu_lib.jet_kv_calibrate(k, v)
    kc = torch.zeros((T, d), dtype=torch.uint8, device="cuda")
    vc = torch.zeros((T, d), dtype=torch.uint8, device="cuda")
    slots = torch.arange(T, dtype=torch.int64, device="cuda").flip(0)
    gpu_lib.jet_kv_append(k, v, slots, sc, kc, vc)
    torch.cuda.synchronize()
    (sk, rk), (sv, rv) = KV.kv_calibrate(y[:, q:q + d], y[:, q + d:])
    assert scales_host(sc) == ((sk, rk), (sv, rv))
    assert_bits_equal(host(kc)[::-1], KV.kv_codes(y[:, q:q + d], rk), "K cache full prefill")
    assert_bits_equal(host(vc)[::-1], KV.kv_codes(y[:, q + d:], rv), "V cache full prefill")


def test_kv_recalibration_reuses_the_scale_buffer(gpu_lib):
    """Repeated recalibrations into one kv_scales buffer (one after each
    weight update), 256 workgroups per tensor: each call's scales are the
    oracle's for its own batch, whichever workgroup holds the maximum and
    whatever the previous call left in the buffer."""
    q, d, T = 4096, 1024, 8192
    sc = torch.full((6,), 123.0, dtype=torch.float32, device="cuda")
    for it, (row, col, val) in enumerate([(8191, 5, 9.0), (0, 1000, 0.5), (4100, 512, -300.0)]):
        y = qkv_output(T, seed=20 + it)
        y[row, q + col] = np.float32(val)               # an outlier in K
        y[T - 1 - row, q + d + col] = np.float32(-val)  # and in V, in another workgroup's rows
        yd = dev_bf16(y)
        gpu_lib.jet_kv_calibrate(yd[:, q:q + d], yd[:, q + d:], kv_scales=sc)
        torch.cuda.synchronize()
        (sk, rk), (sv, rv) = KV.kv_calibrate(y[:, q:q + d], y[:, q + d:])
        assert scales_host(sc) == ((sk, rk), (sv, rv)), f"recalibration {it}: scales differ"
