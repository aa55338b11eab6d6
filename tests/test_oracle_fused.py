"""Pins of the fused-producer oracle (RMSNorm and SwiGLU, readings R12-R14 of
oracle/fused_producers.py) against things other than itself: hand-worked
values, closed forms and invariants, and torch's own rms_norm and silu in
float64.  CPU only.

Hand-worked values (BF16 keeps 8 significant bits: spacing 2^-8 in [0.5, 1),
2^-7 in [1, 2)):
  RMSNorm of [3, 4] (gamma 1, eps 0): mean square 12.5;
    3/sqrt(12.5) = 0.848528... -> 217/256 = 0.84765625;
    4/sqrt(12.5) = 1.131370... -> 145/128 = 1.1328125.
  SwiGLU gate 1, up 2: silu(1) = 1/(1 + e^-1) = 0.7310585786;
    times 2 = 1.4621171573 -> 187/128 = 1.4609375; gate 2, up 1:
    silu(2) = 1.7615941559 -> 225/128 = 1.7578125.
"""
import numpy as np
import pytest
import torch

from oracle import fused_producers as F
from oracle import jet_oracle as O
from fp8_blockwise_quantized_amd import inputs


def test_rmsnorm_hand_example():
    y = F.rmsnorm_bf16(np.array([[3.0, 4.0]], np.float32), np.ones(2, np.float32), 0.0)
    assert y.tolist() == [[0.84765625, 1.1328125]]


def test_swiglu_hand_example():
    gu = np.array([[1.0, 2.0]], np.float32)            # gate 1, up 2
    assert F.swiglu_bf16(gu, 1).tolist() == [[1.4609375]]
    swapped = np.array([[2.0, 1.0]], np.float32)       # gate 2, up 1: silu(2) = 1.7615941559
    assert F.swiglu_bf16(swapped, 1).tolist() == [[1.7578125]]  # 225.48 -> 225/128


def test_rmsnorm_matches_torch_rms_norm():
    x = inputs.activations_with_outliers(64, 512, seed=4)
    g = inputs.normal_bf16((512,), 0.5, seed=4, tensor_id=inputs.ID_W) + 1.0
    for eps in (1e-5, 1e-6, 0.25):
        ref = torch.nn.functional.rms_norm(torch.from_numpy(x.astype(np.float64)), (512,),
                                           weight=torch.from_numpy(g.astype(np.float64)), eps=eps)
        want = O.bf16_rne(O.fl32(ref.numpy()))
        assert np.array_equal(F.rmsnorm_bf16(x, g, eps), want), f"eps={eps}"


def test_rmsnorm_closed_forms():
    g = inputs.normal_bf16((256,), 1.0, seed=2, tensor_id=inputs.ID_W)
    # a constant row c (eps 0) normalizes to sign(c) * gamma exactly
    x = np.array([[2.5] * 256, [-0.375] * 256], np.float32)
    y = F.rmsnorm_bf16(x, g, 0.0)
    assert np.array_equal(y[0], g) and np.array_equal(y[1], -g)
    # scale invariance with eps 0 (powers of two keep every rounding)
    x = inputs.normal_bf16((8, 256), 1.0, seed=3, tensor_id=inputs.ID_X)
    y = F.rmsnorm_bf16(x, g, 0.0)
    for j in (-20, -3, 5, 30):
        assert np.array_equal(F.rmsnorm_bf16(x * np.float32(2.0 ** j), g, 0.0), y)
    # rows are independent; a joint permutation of columns and gamma permutes y
    perm = np.random.default_rng(0).permutation(256)
    assert np.array_equal(F.rmsnorm_bf16(x[:, perm], g[perm], 1e-5), F.rmsnorm_bf16(x, g, 1e-5)[:, perm])
    assert np.array_equal(F.rmsnorm_bf16(x[::-1], g, 1e-5), F.rmsnorm_bf16(x, g, 1e-5)[::-1])
    # eps equal to the mean square halves the square of the norm factor
    x = np.array([[1.0, -1.0, 1.0, -1.0]], np.float32)
    assert F.rmsnorm_bf16(x, np.ones(4, np.float32), 1.0).tolist() == [[0.70703125, -0.70703125] * 2]


def test_silu_identities_and_torch():
    g = np.concatenate([np.linspace(-30, 30, 2001), [0.0, -0.0, 1e-30, -1e-30, 700.0, -700.0, -800.0]])
    s = F.silu(g)
    assert np.all(s[g == 0] == 0.0)
    # silu(x) - silu(-x) = x
    assert np.allclose(s - F.silu(-g), g, rtol=1e-14, atol=1e-300)
    # large arguments: silu(x) -> x, silu(-x) -> -0
    assert F.silu(np.array([700.0]))[0] == 700.0 and F.silu(np.array([-800.0]))[0] == 0.0
    ref = torch.nn.functional.silu(torch.from_numpy(np.linspace(-30, 30, 2001))).numpy()
    assert np.allclose(F.silu(np.linspace(-30, 30, 2001)), ref, rtol=1e-15, atol=1e-300)


def test_swiglu_matches_torch():
    M, I = 32, 384
    gu = inputs.normal_bf16((M, 2 * I), 1.5, seed=7, tensor_id=inputs.ID_X)
    t = torch.from_numpy(gu.astype(np.float64))
    ref = (torch.nn.functional.silu(t[:, :I]) * t[:, I:]).numpy()
    assert np.array_equal(F.swiglu_bf16(gu, I), O.bf16_rne(O.fl32(ref)))
    # only the first 2*I columns are read (a wider row stride is allowed)
    wide = np.concatenate([gu, np.full((M, 128), np.nan, np.float32)], axis=1)
    assert np.array_equal(F.swiglu_bf16(wide, I), F.swiglu_bf16(gu, I))


def test_fused_outputs_are_the_1x128_quantization_of_the_bf16_tensor():
    x = inputs.activations_with_outliers(16, 384, seed=1)
    g = inputs.normal_bf16((384,), 0.5, seed=1, tensor_id=inputs.ID_W) + 1.0
    y, q, s = F.rmsnorm_quant_1x128(x, g, 1e-5)
    q2, s2 = O.quant_1x128(y)
    assert np.array_equal(q, q2) and np.array_equal(s, s2) and q.shape == (16, 384) and s.shape == (3, 16)
    gu = inputs.normal_bf16((16, 512), 1.0, seed=1, tensor_id=inputs.ID_X)
    h, q, s = F.swiglu_quant_1x128(gu, 256)
    q2, s2 = O.quant_1x128(h)
    assert np.array_equal(q, q2) and np.array_equal(s, s2) and q.shape == (16, 256) and s.shape == (2, 16)


def test_bf16_ulp():
    assert F.bf16_ulp(np.array([1.0, 1.9, 0.75, 2.0 ** -130, 0.0])).tolist() == \
        [2.0 ** -7, 2.0 ** -7, 2.0 ** -8, 2.0 ** -133, 2.0 ** -133]


# --- planted mistakes: plausible wrong versions must fail a pin above ---------

_RMSNORM = F.rmsnorm_bf16

def _rms_mean_abs(x, g, eps):
    x64 = np.asarray(x, np.float64)
    return O.bf16_rne(O.fl32(x64 / (np.mean(np.abs(x64), axis=1, keepdims=True) + eps) * g))


def _rms_no_eps(x, g, eps):
    return _RMSNORM(x, g, 0.0)


def _rms_eps_outside(x, g, eps):
    x64 = np.asarray(x, np.float64)
    return O.bf16_rne(O.fl32(x64 / (np.sqrt(np.mean(x64 * x64, axis=1, keepdims=True)) + eps) * g))


def _swiglu_sigmoid(gu, inter):
    gu = np.asarray(gu, np.float64)
    return O.bf16_rne(O.fl32(1.0 / (1.0 + np.exp(-gu[:, :inter])) * gu[:, inter:2 * inter]))


def _swiglu_swapped(gu, inter):
    gu = np.asarray(gu, np.float64)
    return O.bf16_rne(O.fl32(F.silu(gu[:, inter:2 * inter]) * gu[:, :inter]))


@pytest.mark.parametrize("bad", [_rms_mean_abs, _rms_no_eps, _rms_eps_outside])
def test_planted_rmsnorm_mistakes_are_caught(bad, monkeypatch):
    monkeypatch.setattr(F, "rmsnorm_bf16", bad)
    failed = 0
    for pin in (test_rmsnorm_hand_example, test_rmsnorm_matches_torch_rms_norm, test_rmsnorm_closed_forms):
        try:
            pin()
        except AssertionError:
            failed += 1
    assert failed >= 1, f"{bad.__name__} passed every pin"


@pytest.mark.parametrize("bad", [_swiglu_sigmoid, _swiglu_swapped])
def test_planted_swiglu_mistakes_are_caught(bad, monkeypatch):
    monkeypatch.setattr(F, "swiglu_bf16", bad)
    failed = 0
    for pin in (test_swiglu_hand_example, test_swiglu_matches_torch):
        try:
            pin()
        except AssertionError:
            failed += 1
    assert failed >= 1, f"{bad.__name__} passed every pin"
