"""Pins for the oracle's blockwise FP8 (1x128 / 128x128 blocks) and its GEMM.

* pow2_at_least: powers of two map to themselves, others round up; zero -> 1.
* Quantizers: hand-worked blocks; no code exceeds the format maximum (the
  power-of-two scale is never below amax / fmt_max); power-of-two data
  round-trips exactly; the error is at most half a grid step; a 2-D block's
  scale is the one its largest 1-D amax gives; ragged last 2-D row block.
* GEMM: with power-of-two scales, equal to the MXFP8 GEMM whose E8M0 scales
  repeat each 128-block's scale over its four 32-blocks (and, for 2-D B,
  over the block's 128 rows); exact rational brute force with non-power-of-
  two FP32 scales; a transposition check (2-D scales follow n // 128).
"""

from fractions import Fraction

import numpy as np
import pytest

from oracle.blockwise import BLOCK, block_gemm, dequantize_1d, e8m0_of, pow2_at_least, quantize_1d, quantize_2d
from oracle.formats import E4M3, E5M2, decode
from oracle.gemm import mx_gemm


def bf16_bits(values) -> np.ndarray:
    f32 = np.asarray(values, dtype=np.float32)
    bits = f32.view(np.uint32)
    assert np.all(bits & 0xFFFF == 0)
    return (bits >> 16).astype(np.uint16)


def rand_bits(rng, shape, sigma=1.0):
    v = (rng.standard_normal(shape) * sigma).astype(np.float32)
    return (v.view(np.uint32) >> 16).astype(np.uint16)


def test_pow2_at_least():
    v = np.array([1.0, 0.5, 2.0 ** -130, 3.0, 0.3, 1.0000001, 0.0, 448.0, 100 / 448])
    want = np.array([1.0, 0.5, 2.0 ** -130, 4.0, 0.5, 2.0, 1.0, 512.0, 0.25])
    assert np.array_equal(pow2_at_least(v), want)
    assert np.array_equal(e8m0_of(np.array([1.0, 0.25, 3.0], np.float32)), np.array([127, 125, 129], np.uint8))
    # E8M0's range ends at 2^-127: smaller scales round up to it
    tiny = np.array([2.0 ** -127, 2.0 ** -130, 2.0 ** -126 * 0.75, 2.0 ** 127], np.float32)
    assert np.array_equal(e8m0_of(tiny), np.array([0, 0, 1, 254], np.uint8))
    # beyond 2^127 it saturates; zeros take the smallest value; NaN / negative have none
    special = np.array([np.finfo(np.float32).max, np.inf, 0.0, -0.0, np.nan, -1.0, -np.inf, 2.0 ** 126 * 1.5],
                       np.float32)
    assert np.array_equal(e8m0_of(special), np.array([254, 254, 0, 0, 255, 255, 255, 254], np.uint8))


def test_quantize_1d_hand_block_and_invariants():
    # one row, one block: amax 100 -> scale_inv = 2^ceil(log2(100/448)) = 0.25
    vals = np.zeros(BLOCK)
    vals[:4] = [100.0, -50.0, 1.0, 0.1015625]
    q, s = quantize_1d(bf16_bits(vals[None, :]), E4M3)
    assert s.shape == (1, 1) and s[0, 0] == np.float32(0.25)
    # 400 and -200 lie halfway between E4M3 neighbours (384 / 416, 192 / 208): ties go to the even mantissa
    assert np.array_equal(decode(q[0, :4], E4M3), np.array([384.0, -192.0, 4.0, 0.40625]))
    rng = np.random.default_rng(31)
    for fmt in (E4M3, E5M2):
        bits = rand_bits(rng, (8, 512), 3.0)
        q, s = quantize_1d(bits, fmt)
        vals = decode(q, fmt)
        assert np.all(np.abs(vals) <= fmt.max_value)
        x = np.asarray(bits, np.uint32).astype(np.uint32) << 16
        xf = x.view(np.float32).astype(np.float64)
        xh = dequantize_1d(q, s, fmt)
        step = 2.0 ** -3 if fmt is E4M3 else 2.0 ** -2
        sub = np.repeat(s.astype(np.float64), BLOCK, axis=1) * (2.0 ** -9 if fmt is E4M3 else 2.0 ** -16)
        assert np.all(np.abs(xh - xf) <= step / 2 * np.abs(xf) + sub / 2 + 1e-300)
    # power-of-two data round-trips
    p2 = np.where(rng.random((4, 256)) < 0.5, -1.0, 1.0) * 2.0 ** rng.integers(-6, 6, size=(4, 256))
    q, s = quantize_1d(bf16_bits(p2), E4M3)
    assert np.array_equal(dequantize_1d(q, s, E4M3), p2)


def test_quantize_2d_shares_and_ragged():
    rng = np.random.default_rng(32)
    bits = rand_bits(rng, (300, 256), 2.0)
    q2, s2 = quantize_2d(bits, E4M3)
    assert s2.shape == (3, 2)
    _, s1 = quantize_1d(bits, E4M3)
    for i in range(3):
        rows = slice(i * 128, min(300, (i + 1) * 128))
        assert np.array_equal(s2[i], s1[rows].max(axis=0))       # the largest 1-D scale of the block
    # each row block encodes with its shared scale
    x = (np.asarray(bits, np.uint32) << 16).view(np.float32).astype(np.float64)
    xh = decode(q2, E4M3) * np.repeat(np.repeat(s2.astype(np.float64), 128, axis=0)[:300], 128, axis=1)
    assert np.all(np.abs(xh - x) <= 2.0 ** -4 * np.abs(x) + 2.0 ** -10 * np.repeat(np.repeat(s2, 128, 0)[:300], 128, 1))
    assert np.all(np.abs(decode(q2, E4M3)) <= 448)


@pytest.mark.parametrize("b_2d", [False, True])
def test_block_gemm_equals_mx_gemm_with_expanded_scales(b_2d):
    rng = np.random.default_rng(33 + b_2d)
    M, N, K = 40, 300, 384
    qa, sa = quantize_1d(rand_bits(rng, (M, K)), E4M3)
    qb, sb = (quantize_2d if b_2d else quantize_1d)(rand_bits(rng, (N, K), 0.05), E4M3)
    d, _, s = block_gemm(qa, sa, E4M3, qb, sb, E4M3, b_2d)
    ea = np.repeat(e8m0_of(sa), 4, axis=1)
    sbe = np.repeat(sb, 128, axis=0)[:N] if b_2d else sb
    eb = np.repeat(e8m0_of(sbe), 4, axis=1)
    d_mx, _, s_mx = mx_gemm(qa, ea, E4M3, qb, eb, E4M3)
    assert np.array_equal(d, d_mx) and np.array_equal(s, s_mx)


def test_block_gemm_brute_force_fp32_scales_and_orientation():
    rng = np.random.default_rng(35)
    M, N, K = 2, 130, 256
    qa = rng.integers(0, 0x7F, size=(M, K)).astype(np.uint8)
    qb = rng.integers(0, 0x7F, size=(N, K)).astype(np.uint8)
    sa = np.array([[0.3, 1.7], [0.05, 2.5]], np.float32)
    sb = np.array([[0.7, 0.11], [3.0, 0.2]], np.float32)          # 2-D: rows 0..127 and 128..129
    d, _, _ = block_gemm(qa, sa, E4M3, qb, sb, E4M3, True)
    va, vb = decode(qa, E4M3), decode(qb, E4M3)
    for m in range(M):
        for n in (0, 127, 128, 129):
            exact = sum(Fraction(float(sa[m, kb])) * Fraction(float(sb[n // 128, kb])) *
                        sum(Fraction(float(va[m, k])) * Fraction(float(vb[n, k])) for k in range(kb * 128, (kb + 1) * 128))
                        for kb in range(2))
            assert abs(Fraction(float(d[m, n])) - exact) <= abs(exact) * Fraction(1, 2 ** 48)


def test_block_gemm_accumulate_beta_hand_case():
    # one-hot operands pick single products: Y = [[0, 1, 0], [0, 0, 2]]; D = beta C + Y, worked by hand
    qa = np.zeros((2, 128), np.uint8); qa[0, 3] = 0x38; qa[1, 70] = 0x40   # 1.0, 2.0 (E4M3)
    qb = np.zeros((3, 128), np.uint8); qb[1, 3] = 0x38; qb[2, 70] = 0x38
    sa, sb = np.ones((2, 1), np.float32), np.ones((3, 1), np.float32)
    c = np.array([[0, 1, 2], [3, 4, 5]], np.float32)
    d, _, _ = block_gemm(qa, sa, E4M3, qb, sb, E4M3, False, epi="accumulate", c_in=c, beta=-0.5)
    assert np.array_equal(d, [[0.0, 0.5, -1.0], [-1.5, -2.0, -0.5]])
    d, _, _ = block_gemm(qa, sa, E4M3, qb, sb, E4M3, False, epi="accumulate", c_in=c, beta=0.0)
    assert np.array_equal(d, [[0.0, 1.0, 0.0], [0.0, 0.0, 2.0]])
    d, _, _ = block_gemm(qa, sa, E4M3, qb, sb, E4M3, False, epi="accumulate", c_in=c)   # beta defaults to 1
    assert np.array_equal(d, [[0.0, 2.0, 2.0], [3.0, 4.0, 7.0]])
