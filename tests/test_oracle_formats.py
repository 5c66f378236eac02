"""Pins for the oracle's FP8 / E8M0 codecs, independent of the oracle itself.

* Decode: all 256 codes of each format against torch's own float8 dtypes
  (a library decode), plus closed forms of the format limits.
* Encode: exhaustive brute-force argmin over the finite grid (ties to the
  even code) for every bf16 pattern times a range of powers of two; the
  library cast torch.clamp(...).to(float8) (torch's cast is RNE but not
  saturating, so the clamp supplies the saturation); monotonicity; and
  hand-worked values.
"""

import numpy as np
import pytest
import torch

from oracle.formats import E4M3, E5M2, bf16_to_float64, decode, e8m0_decode, encode

TORCH_DT = {"e4m3": torch.float8_e4m3fn, "e5m2": torch.float8_e5m2}


def torch_decode(codes, fmt):
    t = torch.tensor(np.asarray(codes, dtype=np.uint8)).view(TORCH_DT[fmt.name])
    return t.to(torch.float64).numpy()


@pytest.mark.parametrize("fmt", [E4M3, E5M2], ids=lambda f: f.name)
def test_decode_all_codes_match_torch(fmt):
    codes = np.arange(256)
    ours = decode(codes, fmt)
    ref = torch_decode(codes, fmt)
    assert np.array_equal(np.isnan(ours), np.isnan(ref))
    ok = ~np.isnan(ref)
    assert np.array_equal(ours[ok], ref[ok])
    # signed zero
    assert np.signbit(ours[0x80]) and not np.signbit(ours[0x00])


def test_decode_closed_forms():
    assert decode(0x7E, E4M3) == 448.0 and decode(0xFE, E4M3) == -448.0
    assert np.isnan(decode(0x7F, E4M3)) and np.isnan(decode(0xFF, E4M3))
    assert decode(0x01, E4M3) == 2.0 ** -9 and decode(0x08, E4M3) == 2.0 ** -6
    assert decode(0x38, E4M3) == 1.0
    assert decode(0x7B, E5M2) == 57344.0 and decode(0x01, E5M2) == 2.0 ** -16
    assert decode(0x04, E5M2) == 2.0 ** -14 and decode(0x3C, E5M2) == 1.0
    assert decode(0x7C, E5M2) == np.inf and decode(0xFC, E5M2) == -np.inf
    assert all(np.isnan(decode(c, E5M2)) for c in (0x7D, 0x7E, 0x7F))


def test_e8m0_matches_torch():
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.tensor(codes).view(torch.float8_e8m0fnu).to(torch.float64).numpy()
    ours = e8m0_decode(codes)
    assert np.array_equal(np.isnan(ours), np.isnan(ref))
    assert np.array_equal(ours[:255], ref[:255])
    assert ours[127] == 1.0 and ours[0] == 2.0 ** -127 and ours[254] == 2.0 ** 127


def _all_finite_bf16():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    v = bf16_to_float64(bits)
    return v[np.isfinite(v)]


def _brute_force_encode(v, fmt):
    """Argmin over the finite non-negative codes of |a - value(c)|, ties to
    the even code, sign kept.  The grid comes from torch's decode."""
    grid = torch_decode(np.arange(fmt.max_code + 1), fmt)
    a = np.abs(v)
    out = np.empty(v.shape, dtype=np.uint8)
    step = 8192
    for i in range(0, v.size, step):
        d = np.abs(a[i:i + step, None] - grid[None, :])
        dmin = d.min(axis=1, keepdims=True)
        cand = d == dmin
        # prefer the even code among equal-distance candidates
        even = cand & (np.arange(grid.size)[None, :] % 2 == 0)
        pick = np.where(even.any(axis=1), even.argmax(axis=1), cand.argmax(axis=1))
        out[i:i + step] = pick
    return out | np.where(np.signbit(v), 0x80, 0).astype(np.uint8)


@pytest.mark.parametrize("fmt", [E4M3, E5M2], ids=lambda f: f.name)
def test_encode_brute_force_exhaustive_bf16(fmt):
    base = _all_finite_bf16()
    base = base[np.abs(base) < 2.0 ** 100]
    for shift in (-40, -24, -16, -8, 0, 4, 8, 12, 16):
        v = np.ldexp(base, shift)
        # keep the range where something interesting happens (and some saturation)
        v = v[(np.abs(v) < 4 * fmt.max_value) & (np.abs(v) > 2.0 ** -30) | (v == 0)]
        assert np.array_equal(encode(v, fmt), _brute_force_encode(v, fmt)), shift


@pytest.mark.parametrize("fmt", [E4M3, E5M2], ids=lambda f: f.name)
def test_encode_matches_torch_cast_after_clamp(fmt):
    base = _all_finite_bf16()
    for shift in (-30, -12, -6, 0, 6, 12):
        v = np.ldexp(base, shift)
        with np.errstate(over="ignore"):
            f32 = v.astype(np.float32)
        ok = np.isfinite(f32) & (f32.astype(np.float64) == v)  # exactly representable in fp32
        v = v[ok]
        t = torch.from_numpy(v.astype(np.float32))
        ref = torch.clamp(t, -fmt.max_value, fmt.max_value).to(TORCH_DT[fmt.name]).view(torch.uint8).numpy()
        assert np.array_equal(encode(v, fmt), ref), shift


@pytest.mark.parametrize("fmt", [E4M3, E5M2], ids=lambda f: f.name)
def test_encode_monotone(fmt):
    v = np.sort(np.concatenate([np.linspace(-2 * fmt.max_value, 2 * fmt.max_value, 200001),
                                np.ldexp(np.linspace(-3, 3, 20001), -14)]))
    mags = decode(encode(v, fmt), fmt)
    assert np.all(np.diff(mags) >= 0)


def test_encode_hand_values_e4m3():
    cases = [
        (0.0, 0x00), (-0.0, 0x80), (1.0, 0x38), (-1.0, 0xB8),
        (1.0625, 0x38),   # tie 1.0 / 1.125 -> even mantissa 0
        (1.1875, 0x3A),   # tie 1.125 / 1.25 -> even mantissa 2
        (448.0, 0x7E), (460.0, 0x7E), (464.0, 0x7E), (480.0, 0x7E), (1e30, 0x7E), (-1e30, 0xFE),
        (2.0 ** -9, 0x01), (2.0 ** -10, 0x00),   # tie 0 / 2^-9 -> 0
        (3 * 2.0 ** -10, 0x02),                  # tie 2^-9 / 2^-8 -> code 2
        (-(2.0 ** -11), 0x80),                   # negative underflow keeps the sign
        (2.0 ** -6, 0x08), (0.875 * 2.0 ** -6, 0x07),
    ]
    for x, c in cases:
        assert int(encode(np.float64(x), E4M3)) == c, x


def test_encode_hand_values_e5m2():
    cases = [
        (1.0, 0x3C), (1.125, 0x3C),   # tie 1.0 / 1.25 -> even
        (1.375, 0x3E),                # tie 1.25 / 1.5 -> even mantissa 2
        (57344.0, 0x7B), (61440.0, 0x7B), (1e9, 0x7B), (-1e9, 0xFB),
        (2.0 ** -16, 0x01), (2.0 ** -17, 0x00), (3 * 2.0 ** -17, 0x02),
        (-0.0, 0x80), (-(2.0 ** -18), 0x80),
    ]
    for x, c in cases:
        assert int(encode(np.float64(x), E5M2)) == c, x


def test_bf16_to_float64_matches_torch():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ours = bf16_to_float64(bits)
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(np.isnan(ours), np.isnan(ref))
    ok = ~np.isnan(ref)
    assert np.array_equal(ours[ok], ref[ok])
