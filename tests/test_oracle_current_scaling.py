"""Pins for the oracle's amax / current-scaling cast.

* amax: brute-force Python max over |x| on small tensors, signed zeros,
  planted maxima.
* scale / scale_inv: correct fp32 rounding of the exact rational quotient,
  computed here with fractions (round-half-even on the fp32 grid).
* cast: every element whose magnitude equals amax encodes to +-max; each
  fp32 product equals the correctly rounded exact rational product.
"""

from fractions import Fraction

import numpy as np

from oracle.current_scaling import amax, cast_current_scaling, current_scale
from oracle.formats import E4M3, E5M2, bf16_to_float64, encode


def fp32_round(q: Fraction) -> float:
    """Round a positive rational to the nearest float32 (ties to even); normal range."""
    assert q > 0
    e = q.numerator.bit_length() - q.denominator.bit_length()
    while Fraction(2) ** e > q:
        e -= 1
    while Fraction(2) ** (e + 1) <= q:
        e += 1
    quantum = Fraction(2) ** (e - 23)
    n = q / quantum
    fl = n.numerator // n.denominator
    rem = n - fl
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and fl % 2 == 1):
        fl += 1
    return float(fl * quantum)


def rand_bf16(rng, shape, scale=1.0):
    x = (rng.standard_normal(shape) * scale).astype(np.float32)
    return (x.view(np.uint32) >> 16).astype(np.uint16)


def test_amax_brute_force():
    rng = np.random.default_rng(1)
    for _ in range(20):
        bits = rand_bf16(rng, (17, 33), 10 ** rng.uniform(-5, 5))
        vals = [abs(float(v)) for v in bf16_to_float64(bits).ravel()]
        assert float(amax(bits)) == max(vals)


def test_amax_signed_zero_and_planted():
    z = np.array([0x8000, 0x0000, 0x8000], dtype=np.uint16)
    a = amax(z)
    assert a == 0 and not np.signbit(a)
    bits = np.full(1000, 0x3F80, dtype=np.uint16)  # 1.0
    bits[437] = 0xC2C8  # -100.0
    assert amax(bits) == np.float32(100.0)
    assert amax(np.zeros(0, np.uint16)) == 0


def test_scale_is_correctly_rounded_quotient():
    rng = np.random.default_rng(2)
    bits = rand_bf16(rng, 400, 1.0)
    bits = bits[(bits & 0x7FFF) != 0]
    for fmt in (E4M3, E5M2):
        for b in bits:
            a = np.float32(abs(bf16_to_float64(b)))
            s, s_inv = current_scale(a, fmt)
            want = fp32_round(Fraction(int(fmt.max_value)) / Fraction(float(a)))
            assert float(s) == want
            assert float(s_inv) == fp32_round(1 / Fraction(float(s)))


def test_scale_special_cases():
    s, si = current_scale(np.float32(0.0), E4M3)
    assert s == 1 and si == 1
    s, si = current_scale(np.float32(4.0), E4M3)
    assert s == 112.0 and si == np.float32(1 / 112)
    s, _ = current_scale(np.float32(2.0 ** -133), E4M3)  # quotient overflows fp32
    assert s == np.finfo(np.float32).max


def test_cast_amax_elements_hit_max_and_products_are_fp32():
    rng = np.random.default_rng(4)
    for fmt in (E4M3, E5M2):
        bits = rand_bf16(rng, (64, 96), 0.37)
        q, a, s, si = cast_current_scaling(bits, fmt)
        x = bf16_to_float64(bits)
        at_max = np.abs(x) == float(a)
        assert at_max.any()
        assert np.all((q[at_max] & 0x7F) == fmt.max_code)
        # y_i = fl32(x_i * scale) via exact rationals, then encode
        flat = x.ravel()
        idx = rng.choice(flat.size, 300, replace=False)
        for i in idx:
            v = flat[i]
            if v == 0:
                assert (q.ravel()[i] & 0x7F) == 0
                continue
            prod = Fraction(abs(v)) * Fraction(float(s))
            y = fp32_round(prod) * (1 if v > 0 else -1)
            assert q.ravel()[i] == encode(np.float64(y), fmt)


def test_cast_zero_tensor():
    bits = np.zeros((4, 32), np.uint16)
    bits[0, 0] = 0x8000
    q, a, s, si = cast_current_scaling(bits, E4M3)
    assert a == 0 and s == 1 and si == 1
    assert q[0, 0] == 0x80 and np.all(q.ravel()[1:] == 0)
