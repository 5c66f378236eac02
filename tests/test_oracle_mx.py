"""Pins for the oracle's MXFP8 block quantization.

* Hand-worked blocks in tests/golden/mx_blocks.txt (rowwise and columnwise).
* Block scale: exhaustive over every positive finite bf16 amax, against the
  integer form max(biased_exponent_field(amax) - emax, 0) read from the bits,
  plus the defining interval 2^(s+emax) <= amax < 2^(s+emax+1).
* Invariants: power-of-two blocks reproduce exactly, dequantized magnitudes
  stay below max * 2^s, rounding-error bounds, values already on the fp8
  grid round-trip, and colwise(X) == rowwise(X^T).
"""

import os

import numpy as np
import pytest

from oracle.formats import E4M3, E5M2, bf16_to_float64, decode, format_by_name
from oracle.mx import block_scale_code, dequantize, quantize_colwise, quantize_rowwise

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "mx_blocks.txt")


def load_golden():
    cases = []
    for line in open(GOLDEN):
        line = line.strip()
        if not line or line.startswith("#"):
            continue
        fmt, xs, code, qs = [f.strip() for f in line.split("|")]
        x = np.zeros(32, dtype=np.uint16)
        vals = [int(h, 16) for h in xs.split()]
        x[:len(vals)] = vals
        q = np.zeros(32, dtype=np.uint8)
        qv = [int(h, 16) for h in qs.split()]
        q[:len(qv)] = qv
        cases.append((format_by_name(fmt), x, int(code), q))
    return cases


def test_golden_blocks_rowwise_and_colwise():
    cases = load_golden()
    assert len(cases) == 8
    for fmt, x, code, q in cases:
        qr, sr = quantize_rowwise(x[None, :], fmt)
        assert sr[0, 0] == code
        assert np.array_equal(qr[0], q)
        qc, sc = quantize_colwise(x[:, None], fmt)
        assert sc[0, 0] == code
        assert np.array_equal(qc[0], q)


def bexp(bits):
    return (np.asarray(bits, dtype=np.int64) >> 7) & 0xFF


@pytest.mark.parametrize("fmt", [E4M3, E5M2], ids=lambda f: f.name)
def test_block_scale_exhaustive_against_exponent_bits(fmt):
    bits = np.arange(1, 0x7F80, dtype=np.int64)  # every positive finite bf16
    amax = bf16_to_float64(bits.astype(np.uint16))
    code = block_scale_code(amax, fmt).astype(np.int64)
    assert np.array_equal(code, np.maximum(bexp(bits) - fmt.emax, 0))
    s = code - 127
    big = bexp(bits) >= fmt.emax + 1  # scale not clamped at the bottom
    lo = np.ldexp(1.0, s[big] + fmt.emax)
    assert np.all(lo <= amax[big]) and np.all(amax[big] < 2 * lo)


def test_block_scale_special_values():
    assert block_scale_code(0.0, E4M3) == 0
    assert block_scale_code(np.inf, E4M3) == 255
    assert block_scale_code(np.nan, E5M2) == 255
    assert block_scale_code(1.0, E4M3) == 119 and block_scale_code(1.0, E5M2) == 112
    assert block_scale_code(448.0, E4M3) == 127   # 448 = 1.75 * 2^8
    assert block_scale_code(512.0, E4M3) == 128


def bf16_bits(v):
    """float64 values exactly representable in bf16 -> bit patterns."""
    f = np.asarray(v, dtype=np.float64).astype(np.float32)
    assert np.array_equal(f.astype(np.float64), v)
    b = f.view(np.uint32)
    assert np.all(b & 0xFFFF == 0)
    return (b >> 16).astype(np.uint16)


@pytest.mark.parametrize("fmt", [E4M3, E5M2], ids=lambda f: f.name)
def test_power_of_two_blocks_reproduce_exactly(fmt):
    rng = np.random.default_rng(7)
    depth = 17 if fmt is E4M3 else 31  # down to the smallest subnormal after scaling
    R = 256
    e_amax = rng.integers(-100, 100, size=R)
    j = e_amax[:, None] - rng.integers(0, depth + 1, size=(R, 32))
    j[:, 0] = e_amax
    sign = rng.choice([-1.0, 1.0], size=(R, 32))
    zero = rng.random((R, 32)) < 0.1
    zero[:, 0] = False
    v = np.where(zero, 0.0, sign * np.ldexp(1.0, j))
    q, s = quantize_rowwise(bf16_bits(v), fmt)
    assert np.array_equal(dequantize(q, s, fmt), v)


@pytest.mark.parametrize("fmt", [E4M3, E5M2], ids=lambda f: f.name)
def test_quantize_error_bounds(fmt):
    rng = np.random.default_rng(11)
    x = rng.standard_normal((512, 256)).astype(np.float32)
    x[:, rng.choice(256, 8, replace=False)] *= 20
    x *= np.ldexp(1.0, rng.integers(-30, 30, size=(512, 1))).astype(np.float32)
    bits = (x.view(np.uint32) >> 16).astype(np.uint16)  # truncation is fine for test data
    xv = bf16_to_float64(bits)
    q, s = quantize_rowwise(bits, fmt)
    xh = dequantize(q, s, fmt)
    sc = np.repeat(np.ldexp(1.0, s.astype(np.int64) - 127), 32, axis=1)
    # (b) magnitude bound
    assert np.all(np.abs(xh) <= fmt.max_value * sc)
    y = np.abs(xv) / sc
    m = fmt.man_bits
    min_normal = 2.0 ** (1 - fmt.bias)
    err = np.abs(xh - xv)
    normal = (y >= min_normal) & (y <= fmt.max_value)
    assert np.all(err[normal] <= 2.0 ** -(m + 1) * np.abs(xv[normal]))
    sub = y < min_normal
    assert np.all(err[sub] <= 2.0 ** (1 - fmt.bias - m - 1) * sc[sub])
    # (c) only magnitudes beyond the saturation threshold clamp (464 for E4M3, 61440 for E5M2)
    sat_threshold = fmt.max_value * (1 + 2.0 ** -(m + 1))
    clamped = y > fmt.max_value
    assert np.all(np.abs(xh[clamped]) == fmt.max_value * sc[clamped])
    assert np.all(y < 2.0 ** (fmt.emax + 1))
    rounds_within = clamped & (y < sat_threshold)
    assert np.all(err[rounds_within] <= 2.0 ** -(m + 1) * np.abs(xv[rounds_within]))


@pytest.mark.parametrize("fmt", [E4M3, E5M2], ids=lambda f: f.name)
def test_on_grid_blocks_round_trip(fmt):
    rng = np.random.default_rng(3)
    codes = rng.integers(0, 256, size=(64, 32)).astype(np.uint8)
    vals = decode(codes, fmt)
    codes = np.where(np.isfinite(vals), codes, 0x00).astype(np.uint8)
    codes[:, 0] = fmt.max_code  # largest finite magnitude sets the scale 2^0 ... times the block shift below
    shift = rng.integers(-60, 60, size=(64, 1))
    v = decode(codes, fmt) * np.ldexp(1.0, shift)
    q, s = quantize_rowwise(bf16_bits(v), fmt)
    assert np.array_equal(s[:, 0].astype(np.int64), (shift[:, 0] + 127))
    assert np.array_equal(dequantize(q, s, fmt), v)
    # codes themselves come back, except that -0 and +0 keep their sign
    assert np.array_equal(q, codes)


@pytest.mark.parametrize("fmt", [E4M3, E5M2], ids=lambda f: f.name)
def test_colwise_is_rowwise_of_transpose(fmt):
    rng = np.random.default_rng(5)
    x = (rng.standard_normal((96, 160)).astype(np.float32) * 3)
    bits = (x.view(np.uint32) >> 16).astype(np.uint16)
    qc, sc = quantize_colwise(bits, fmt)
    qr, sr = quantize_rowwise(np.ascontiguousarray(bits.T), fmt)
    assert qc.shape == (160, 96) and sc.shape == (160, 3)
    assert np.array_equal(qc, qr) and np.array_equal(sc, sr)


def test_shape_errors():
    with pytest.raises(ValueError):
        quantize_rowwise(np.zeros((4, 33), np.uint16), E4M3)
    with pytest.raises(ValueError):
        quantize_colwise(np.zeros((33, 4), np.uint16), E4M3)
