"""Pins of the KV-cache oracle (readings R15-R17 of oracle/kv_cache.py) against
hand-worked codes, invariants and planted mistakes.  CPU only.

Hand-worked: a calibration batch whose largest magnitude is 448 gets s = r = 1,
so the codes are those of the values themselves (OCP E4M3: 448 = 0x7E,
1.0 = 0x38, 0.5 = 0x30, sign bit 0x80; -0.0 = 0x80).
"""
import numpy as np
import pytest

from oracle import jet_oracle as O
from oracle import kv_cache as KV
from fp8_blockwise_quantized_amd import inputs


def test_hand_example_and_saturation():
    k = np.array([[448.0, -1.0], [0.5, -0.0]], np.float32)
    v = np.array([[2.0, 1.0], [-4.0, 0.25]], np.float32)
    (sk, rk), (sv, rv) = KV.kv_calibrate(k, v)
    assert (sk, rk) == (1.0, 1.0)
    assert sv == np.float32(4.0 / 448.0) and rv == np.float32(448.0 / 4.0)
    cache = np.zeros((4, 2), np.uint8)
    out = KV.kv_append(cache, k, [2, 0], rk)
    assert out[2].tolist() == [0x7E, 0xB8] and out[0].tolist() == [0x30, 0x80]
    assert out[1].tolist() == [0, 0] and out[3].tolist() == [0, 0]
    # later tokens beyond the calibrated range saturate at +-448
    late = np.array([[1000.0, -1000.0], [449.0, -448.0]], np.float32)
    assert KV.kv_codes(late, rk).tolist() == [[0x7E, 0xFE], [0x7E, 0xFE]]


def test_calibration_is_per_tensor_and_scale_invariant():
    k = inputs.activations_with_outliers(40, 256, seed=2)
    v = inputs.normal_bf16((40, 256), 0.5, seed=2, tensor_id=inputs.ID_DY)
    (sk, rk), (sv, rv) = KV.kv_calibrate(k, v)
    # the tensor's largest element encodes to +-448 with its own calibration
    i = np.unravel_index(np.argmax(np.abs(k)), k.shape)
    assert KV.kv_codes(k, rk)[i] in (0x7E, 0xFE)
    j = np.unravel_index(np.argmax(np.abs(v)), v.shape)
    assert KV.kv_codes(v, rv)[j] in (0x7E, 0xFE)
    # one scale for the whole tensor: rows with a smaller maximum do not reach 448
    row_max_codes = np.max(KV.kv_codes(k, rk) & 0x7F, axis=1)
    assert np.sum(row_max_codes == 0x7E) < k.shape[0]
    # x * 2^j -> s * 2^j, r / 2^j, the same codes
    for e in (-12, 7):
        f = np.float32(2.0 ** e)
        (sk2, rk2), _ = KV.kv_calibrate(k * f, v)
        assert sk2 == sk * f and rk2 == rk / f
        assert np.array_equal(KV.kv_codes(k * f, rk2), KV.kv_codes(k, rk))


def test_append_scatter_and_padding_slots():
    rng = np.random.default_rng(0)
    x = inputs.normal_bf16((50, 128), 1.0, seed=5, tensor_id=inputs.ID_X)
    (_, r), _ = KV.kv_calibrate(x, x)
    slots = rng.permutation(200)[:50].astype(np.int64)
    slots[[3, 17, 49]] = -1                      # padding tokens
    cache = rng.integers(0, 256, size=(200, 128), dtype=np.uint8)
    out = KV.kv_append(cache, x, slots, r)
    codes = KV.kv_codes(x, r)
    written = set()
    for t, sl in enumerate(slots):
        if sl >= 0:
            assert np.array_equal(out[sl], codes[t])
            written.add(int(sl))
    untouched = [i for i in range(200) if i not in written]
    assert np.array_equal(out[untouched], cache[untouched]), "rows without a token must be left as they were"
    # dequantized cache rows are within half an E4M3 spacing (times s) of the inputs
    s = np.float32(1.0) / r
    deq = O.e4m3_decode(codes) * np.float64(s)
    assert np.all(np.abs(deq - x) <= np.abs(x) * 2.0 ** -4 + 2.0 ** -10 * float(s) + 1e-30)


def test_empty_calibration_batch_uses_the_floor():
    (sk, rk), (sv, rv) = KV.kv_calibrate(np.zeros((0, 128), np.float32), np.zeros((3, 128), np.float32))
    floor = np.float32(2.0 ** -96)
    assert sk == np.float32(floor / np.float32(448.0)) and sv == sk and rk == rv


# --- planted mistakes ----------------------------------------------------------

_APPEND = KV.kv_append
_CODES = KV.kv_codes
_CAL = KV.kv_calibrate


def _append_negative_index(cache, x, slots, r):
    out = np.array(cache, dtype=np.uint8, copy=True)
    codes = KV.kv_codes(x, r)
    for t, slot in enumerate(slots):
        out[slot] = codes[t]                     # writes row -1 for padding tokens
    return out


def _codes_no_saturation(x, r):
    prod = np.asarray(x, np.float32) * np.float32(r)
    return np.where(np.abs(prod) > 448, 0x7F | (np.signbit(prod) << 7), _CODES(np.clip(x, -448 / r, 448 / r), r)).astype(np.uint8)


def _calibrate_per_row_max_of_first_row(k, v):
    out = []
    for x in (k, v):
        amax = np.float32(np.max(np.abs(np.asarray(x)[:1]))) if np.size(x) else np.float32(0)
        s, r = O.scale_pair(np.array([amax], np.float32))
        out.append((np.float32(s[0]), np.float32(r[0])))
    return tuple(out)


def _calibrate_dequant_scale_as_multiplier(k, v):
    (sk, rk), (sv, rv) = _CAL(k, v)
    return (sk, sk), (sv, sv)


@pytest.mark.parametrize("name,bad", [("kv_append", _append_negative_index),
                                      ("kv_codes", _codes_no_saturation),
                                      ("kv_calibrate", _calibrate_per_row_max_of_first_row),
                                      ("kv_calibrate", _calibrate_dequant_scale_as_multiplier)])
def test_planted_mistakes_are_caught(name, bad, monkeypatch):
    monkeypatch.setattr(KV, name, bad)
    failed = 0
    for pin in (test_hand_example_and_saturation, test_calibration_is_per_tensor_and_scale_invariant,
                test_append_scatter_and_padding_slots):
        try:
            pin()
        except AssertionError:
            failed += 1
    assert failed >= 1, f"{bad.__name__} passed every pin"
