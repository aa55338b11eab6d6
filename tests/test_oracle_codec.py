"""Pins of the oracle's E4M3 codec to things other than itself.

* the OCP E4M3 definition (bias 7, subnormal spacing 2^-9, max 448, one NaN
  pattern per sign) at landmark codes;
* the library routine torch.float8_e4m3fn (round to nearest even, not
  saturating) on values clamped to +-448, over every fp32 value near each
  E4M3 value and rounding midpoint plus a large random sample;
* hand-worked examples;
* planted mistakes (ties away from zero, truncation, no saturation, a lost
  sign of zero) that the same checks must reject.
"""
import numpy as np
import pytest
import torch

from oracle import jet_oracle as O


def torch_encode(v):
    v = np.clip(np.asarray(v, np.float32), -448.0, 448.0)
    return torch.from_numpy(v).to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def torch_decode_all():
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    return codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()


def boundary_sample():
    """fp32 values within +-300 ulps of every E4M3 value and of every midpoint
    between neighbouring E4M3 values, both signs, plus random values."""
    pos = O.DECODE[:0x7F]
    mids = (pos[:-1] + pos[1:]) / 2
    top = np.array([448.0, 456.0, 464.0, 470.0])
    centres = np.concatenate([pos, mids, top]).astype(np.float32)
    off = np.arange(-300, 301, dtype=np.int64)
    bits = centres.view(np.uint32).astype(np.int64)[:, None] + off[None, :]
    bits = bits[(bits >= 0) & (bits < 0x7F800000)].astype(np.uint32)
    vals = bits.view(np.float32)
    rng = np.random.default_rng(1234)
    rnd_bits = rng.integers(0, 0x43F00000, size=1_000_000, dtype=np.uint32)  # |v| < 480
    rnd = rnd_bits.view(np.float32)
    uni = rng.uniform(0, 460, size=500_000).astype(np.float32)
    den = rng.integers(1, 0x00800000, size=20_000, dtype=np.uint32).view(np.float32)
    allv = np.concatenate([vals, rnd, uni, den, np.array([0.0], np.float32)])
    return np.concatenate([allv, -allv])


def check_codec(encode):
    """Raise AssertionError if `encode` disagrees with the pins."""
    v = boundary_sample()
    got = encode(v)
    ref = torch_encode(v)
    bad = np.nonzero(got != ref)[0]
    assert bad.size == 0, f"{bad.size} mismatches, first at v={v[bad[0]]!r}: {got[bad[0]]:#x} vs {ref[bad[0]]:#x}"
    # hand-worked examples
    assert encode(np.float32([-0.0]))[0] == 0x80
    assert encode(np.float32([2.0 ** -10]))[0] == 0x00      # tie between 0 and 2^-9 -> even (0)
    assert encode(np.float32([1.5 * 2.0 ** -9]))[0] == 0x02  # tie between 1 and 2 (x2^-9) -> even (2)
    assert encode(np.float32([168.0]))[0] == 0x72            # tie 160|176 -> 160 (mantissa 4, even)
    assert encode(np.float32([500.0]))[0] == 0x7E            # saturates to 448
    assert encode(np.float32([-1000.0]))[0] == 0xFE


def test_decode_landmarks():
    # OCP E4M3: bias 7, 3 mantissa bits, subnormal step 2^-9, max 448
    assert O.DECODE[0x00] == 0.0 and np.signbit(O.DECODE[0x80])
    assert O.DECODE[0x01] == 2.0 ** -9
    assert O.DECODE[0x07] == 7 * 2.0 ** -9
    assert O.DECODE[0x08] == 2.0 ** -6
    assert O.DECODE[0x38] == 1.0
    assert O.DECODE[0x7E] == 448.0 and O.DECODE[0xFE] == -448.0
    assert np.isnan(O.DECODE[0x7F]) and np.isnan(O.DECODE[0xFF])
    assert np.sum(np.isnan(O.DECODE)) == 2


def test_decode_table_matches_library():
    ref = torch_decode_all()
    ok = (O.DECODE == ref) | (np.isnan(O.DECODE) & np.isnan(ref))
    assert ok.all()
    fin = ~np.isnan(ref)
    assert np.array_equal(np.signbit(O.DECODE[fin]), np.signbit(ref[fin]))


def test_encoder_matches_library_and_examples():
    check_codec(O.e4m3_encode)


def test_every_code_round_trips():
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], np.uint8)
    vals = O.DECODE[codes].astype(np.float32)
    assert np.array_equal(O.e4m3_encode(vals), codes)


def test_encoder_rejects_nonfinite():
    with pytest.raises(ValueError):
        O.e4m3_encode(np.float32([np.nan]))


# --- planted mistakes: each must be caught by check_codec ------------------

def _mutant(rounder=np.rint, saturate=True, keep_neg_zero=True):
    def enc(v):
        v = np.asarray(v, np.float32)
        a = np.abs(v.astype(np.float64))
        if saturate:
            a = np.minimum(a, 448.0)
        _, e = np.frexp(a)
        sp = np.ldexp(1.0, np.where(a < 2.0 ** -6, -9, e - 4).astype(np.int32))
        val = np.minimum(rounder(a / sp) * sp, 480.0)
        idx = np.searchsorted(np.append(O.DECODE[:0x7F], 480.0), val).astype(np.uint8)
        neg = np.signbit(v) if keep_neg_zero else (v < 0)
        return (idx | (neg.astype(np.uint8) << 7)).astype(np.uint8)
    return enc


@pytest.mark.parametrize("mut", [
    dict(rounder=lambda q: np.floor(q + 0.5)),     # ties away from zero
    dict(rounder=np.floor),                        # truncation
    dict(saturate=False),                          # overflow past 448
    dict(keep_neg_zero=False),                     # -0.0 encoded as +0
])
def test_codec_pins_reject_planted_mistakes(mut):
    with pytest.raises(AssertionError):
        check_codec(_mutant(**mut))
