"""Pins of oracle/mismatch.py (the multiplicative probability error of the
nmedialink NeMo-RL FP8 page, section "FP8面临的关键挑战：数值分歧").

Pins: hand-worked softmax values; probabilities summing to one and shift
invariance (closed forms of the softmax); a brute-force softmax in Python
floats on a tiny case; the metric's hand-worked values, its value 1 exactly
for identical log-probabilities, symmetry, its lower bound 1, and the closed
form exp(|d|) for a constant offset; planted mistakes (a sign instead of the
absolute value, the exponent of the mean instead of the mean of exponents,
the probability of the wrong token) each fail a pin."""
import math

import numpy as np
import pytest

from oracle import mismatch as MM


def test_hand_worked_logprobs():
    # logits [0, ln 3]: p = [1/4, 3/4]
    lp = MM.token_logprobs(np.array([[0.0, math.log(3.0)], [0.0, math.log(3.0)]]), [0, 1])
    assert lp[0] == pytest.approx(math.log(0.25), abs=1e-15)
    assert lp[1] == pytest.approx(math.log(0.75), abs=1e-15)
    # uniform logits over V entries: log(1/V)
    V = 7
    assert MM.token_logprobs(np.full((1, V), 3.5), [4])[0] == pytest.approx(-math.log(V), abs=1e-15)


def test_logprobs_closed_forms():
    rng = np.random.default_rng(1)
    z = rng.normal(0, 4, size=(5, 50))
    full = np.stack([MM.token_logprobs(z, np.full(5, v)) for v in range(50)], axis=1)
    assert np.allclose(np.exp(full).sum(axis=1), 1.0, atol=1e-13)             # a distribution
    ids = rng.integers(0, 50, size=5)
    assert np.allclose(MM.token_logprobs(z + 123.0, ids), MM.token_logprobs(z, ids), atol=1e-12)   # shift
    # large logits do not overflow
    big = MM.token_logprobs(np.array([[1000.0, 999.0]]), [1])[0]
    assert big == pytest.approx(-math.log1p(math.e), abs=1e-12)


def test_logprobs_brute_force():
    rng = np.random.default_rng(2)
    z = rng.normal(0, 2, size=(3, 6))
    ids = [5, 0, 2]
    for i, t in enumerate(ids):
        den = sum(math.exp(v) for v in z[i])
        assert MM.token_logprobs(z, ids)[i] == pytest.approx(math.log(math.exp(z[i, t]) / den), abs=1e-14)


def test_metric_hand_worked():
    # differences 0 and ln 2: (e^0 + e^ln2) / 2 = 1.5
    assert MM.token_mult_prob_error([0.0, -1.0], [0.0, -1.0 - math.log(2.0)]) == pytest.approx(1.5, abs=1e-15)
    # differences ln 1.5, -ln 1.5, 0 (absolute value): (1.5 + 1.5 + 1) / 3
    d = math.log(1.5)
    assert MM.token_mult_prob_error([d, 0.0, -2.0], [0.0, d, -2.0]) == pytest.approx(4.0 / 3.0, abs=1e-15)


def test_metric_identity_symmetry_bound():
    rng = np.random.default_rng(3)
    a = -rng.exponential(2.0, size=100)
    assert MM.token_mult_prob_error(a, a) == 1.0                     # identical log-probs: exactly 1
    b = a + rng.normal(0, 0.05, size=100)
    assert MM.token_mult_prob_error(a, b) == MM.token_mult_prob_error(b, a)
    assert MM.token_mult_prob_error(a, b) > 1.0
    for d in (1e-3, 0.03, 0.5):                                      # constant offset: exp(|d|)
        assert MM.token_mult_prob_error(a, a - d) == pytest.approx(math.exp(d), rel=1e-12)
    with pytest.raises(ValueError):
        MM.token_mult_prob_error([], [])


def _planted_signed(a, b):
    return float(np.mean(np.exp(np.asarray(a) - np.asarray(b))))


def _planted_exp_of_mean(a, b):
    return float(np.exp(np.mean(np.abs(np.asarray(a) - np.asarray(b)))))


def test_planted_mistakes_fail_a_pin():
    d = math.log(1.5)
    # signed difference: the hand-worked (1.5 + 1.5 + 1)/3 case gives (1.5 + 2/3 + 1)/3
    assert _planted_signed([d, 0.0, -2.0], [0.0, d, -2.0]) != pytest.approx(4.0 / 3.0, abs=1e-6)
    # exp of the mean: (0 + ln 2)/2 -> sqrt(2), not 1.5
    assert _planted_exp_of_mean([0.0, -1.0], [0.0, -1.0 - math.log(2.0)]) != pytest.approx(1.5, abs=1e-6)
    # the wrong token's probability: logits [0, ln 3] with id 0 must give ln(1/4), not ln(3/4)
    wrong = MM.token_logprobs(np.array([[math.log(3.0), 0.0]]), [0])[0]
    assert wrong != pytest.approx(math.log(0.25), abs=1e-6)
