"""Pins for the oracle's delayed scaling and per-tensor FP8 GEMM.

* A hand-worked 5-step sequence (amaxes are powers of two, so every scale is
  exact): the history shifts newest-first, "max" keeps an old large amax,
  the cast of a step uses the previous step's scale (a growing amax
  saturates), and q_scale_inv is the inverse of the scale used.
* "most_recent", margins, zero and non-finite amaxes keep the scale, and a
  quotient beyond float32 becomes the largest finite float.
* With the scale the current-scaling rule gives, the cast equals the pinned
  current-scaling cast code for code.
* Per-tensor GEMM: equal to the MXFP8 GEMM with every block scale 2^0, times
  alpha (exact for power-of-two alphas); exact rational brute force.
"""

from fractions import Fraction

import numpy as np
import pytest

from oracle.current_scaling import cast_current_scaling
from oracle.delayed_scaling import delayed_scaling_step, fp8_gemm_per_tensor, next_scale
from oracle.formats import E4M3, E5M2, decode, encode
from oracle.gemm import mx_gemm


def bf16_bits(values) -> np.ndarray:
    f32 = np.asarray(values, dtype=np.float32)
    bits = f32.view(np.uint32)
    assert np.all(bits & 0xFFFF == 0)
    return (bits >> 16).astype(np.uint16)


def test_hand_worked_sequence_max():
    h = np.zeros(3, np.float32)
    s = np.float32(1.0)
    steps = [  # (tensor values, expected amax, expected history after, expected next scale)
        ([1.0, -2.0, 0.5], 2.0, [2.0, 0.0, 0.0], 224.0),
        ([8.0, 3.0, -1.0], 8.0, [8.0, 2.0, 0.0], 56.0),
        ([0.5, -0.25, 0.0], 0.5, [0.5, 8.0, 2.0], 56.0),      # the old amax 8 still rules
        ([1.0, -1.0, 0.125], 1.0, [1.0, 0.5, 8.0], 56.0),
        ([-1.0, 0.5, 0.5], 1.0, [1.0, 1.0, 0.5], 448.0),      # 8 has left the window
    ]
    used = []
    for vals, a_exp, h_exp, s_exp in steps:
        bits = bf16_bits(vals)
        q, q_inv, a, h, s_next = delayed_scaling_step(bits, E4M3, h, s)
        assert a == np.float32(a_exp)
        assert np.array_equal(h, np.array(h_exp, np.float32))
        assert s_next == np.float32(s_exp)
        assert q_inv == np.float32(1.0) / s
        assert np.array_equal(q, encode(np.asarray(vals, np.float64) * float(s), E4M3))
        used.append(float(s))
        s = s_next
    assert used == [1.0, 224.0, 56.0, 56.0, 56.0]
    # step 2 cast [8, 3, -1] with the delayed scale 224: 1792 and 672 saturate to 448
    q2, _, _, _, _ = delayed_scaling_step(bf16_bits([8.0, 3.0, -1.0]), E4M3, [2.0, 0, 0], np.float32(224.0))
    assert np.array_equal(decode(q2, E4M3), np.array([448.0, 448.0, -224.0]))


def test_most_recent_margin_and_kept_scales():
    h = np.array([1.0, 16.0, 4.0], np.float32)
    assert next_scale(h, 3.0, E4M3, "max") == np.float32(28.0)           # 448 / 16
    assert next_scale(h, 3.0, E4M3, "most_recent") == np.float32(448.0)  # 448 / 1
    assert next_scale(h, 3.0, E4M3, "max", margin=2) == np.float32(7.0)  # 448 / 16 / 4
    assert next_scale(h, 3.0, E5M2, "max") == np.float32(3584.0)         # 57344 / 16
    assert next_scale(np.zeros(4), 3.0, E4M3) == np.float32(3.0)         # no amax yet: keep
    assert next_scale([np.inf, 1.0], 3.0, E4M3) == np.float32(3.0)       # non-finite: keep
    assert next_scale([np.nan, 1.0], 3.0, E4M3, "most_recent") == np.float32(3.0)
    # quotient beyond float32 -> largest finite float32
    assert next_scale([np.float32(2.0 ** -133)], 1.0, E4M3) == np.float32(np.finfo(np.float32).max)
    # 448 / 3 is not exact: the correctly rounded float32 quotient
    assert next_scale([3.0], 1.0, E4M3) == np.float32(np.float32(448.0) / np.float32(3.0))
    with pytest.raises(ValueError):
        next_scale(h, 1.0, E4M3, "mean")


def test_cast_matches_current_scaling_with_the_same_scale():
    rng = np.random.default_rng(21)
    vals = (rng.standard_normal(4096) * 3).astype(np.float32)
    bits = (vals.view(np.uint32) >> 16).astype(np.uint16)
    q_cur, a, s_cur, s_inv_cur = cast_current_scaling(bits, E4M3)
    q, q_inv, a2, _, _ = delayed_scaling_step(bits, E4M3, np.zeros(16, np.float32), s_cur)
    assert a2 == a and q_inv == s_inv_cur
    assert np.array_equal(q, q_cur)


def test_per_tensor_gemm_equals_unit_block_scales_times_alpha():
    rng = np.random.default_rng(22)
    qa = rng.integers(0, 0x7F, size=(24, 256)).astype(np.uint8) | (rng.integers(0, 2, (24, 256)) * 0x80).astype(np.uint8)
    qb = rng.integers(0, 0x7F, size=(40, 256)).astype(np.uint8)
    ones_a = np.full((24, 8), 127, np.uint8)
    ones_b = np.full((40, 8), 127, np.uint8)
    y, _, s = mx_gemm(qa, ones_a, E4M3, qb, ones_b, E4M3)
    d, aux, s_pt = fp8_gemm_per_tensor(qa, 2.0 ** -3, E4M3, qb, 2.0 ** -5, E4M3)
    assert aux is None and np.array_equal(d, y * 2.0 ** -8) and np.array_equal(s_pt, s * 2.0 ** -8)
    bias = bf16_bits(np.arange(-20, 20) / 16.0)
    d, aux, _ = fp8_gemm_per_tensor(qa, 0.5, E4M3, qb, 0.25, E4M3, bias, "bias_gelu_aux")
    d_ref, aux_ref, _ = mx_gemm(qa, ones_a - 3, E4M3, qb, ones_b, E4M3, bias, "bias_gelu_aux")  # 2^-3 via A's scales
    assert np.array_equal(aux, aux_ref) and np.array_equal(d, d_ref)


def test_per_tensor_gemm_brute_force_exact():
    rng = np.random.default_rng(23)
    qa = rng.integers(0, 0x7F, size=(3, 128)).astype(np.uint8)
    qb = (rng.integers(0, 0x7B, size=(2, 128)).astype(np.uint8)) | 0x80
    sa, sb = 0.375, 1.25
    d, _, _ = fp8_gemm_per_tensor(qa, sa, E4M3, qb, sb, E5M2)
    va, vb = decode(qa, E4M3), decode(qb, E5M2)
    for i in range(3):
        for j in range(2):
            exact = Fraction(sa) * Fraction(sb) * sum(Fraction(float(va[i, k])) * Fraction(float(vb[j, k]))
                                                     for k in range(128))
            assert abs(Fraction(float(d[i, j])) - exact) <= abs(exact) * Fraction(1, 2 ** 50)
