"""Pins for the oracle's MXFP8 GEMM, epilogues, grouped GEMM and tolerance.

* GEMM: a pure-Python triple loop over exact rationals (brute force) on
  tiny non-square operands with distinct per-block scales, so that a
  transposed operand, a wrong scale index or a dropped block fails; hand
  cases (all-ones K=128 gives 128, one-hot rows, scale +1 on both sides
  multiplies by 4).
* GELU(tanh): torch.nn.functional.gelu(approximate="tanh") in float64,
  gelu(0) = 0, gelu(x) - gelu(-x) = x, gelu(x)/x -> 1.
* Epilogues: D - Y equals the bias exactly; aux equals the pre-activation.
* Grouped: one dense GEMM of all rows against all experts, from which each
  expert's row/column block is taken (a different computation from the
  per-expert loop), including empty experts.
* Tolerance: planted values just inside / outside the bound.
"""

from fractions import Fraction

import math

import numpy as np
import pytest
import torch

from oracle.formats import E4M3, E5M2, bf16_to_float64, decode
from oracle.gemm import dgelu_tanh, epilogue, gelu_tanh, grouped_mx_gemm, mx_gemm, tolerance_bound, within_tolerance


def rand_codes(rng, shape, fmt):
    c = rng.integers(0, 256, size=shape).astype(np.uint8)
    v = decode(c, fmt)
    return np.where(np.isfinite(v), c, 0x38 if fmt is E4M3 else 0x3C).astype(np.uint8)


def brute_gemm(qa, sa, fa, qb, sb, fb):
    M, K = qa.shape
    N = qb.shape[0]
    out = [[Fraction(0)] * N for _ in range(M)]
    for m in range(M):
        for n in range(N):
            acc = Fraction(0)
            for k in range(K):
                av = Fraction(float(decode(qa[m, k], fa))) * Fraction(2) ** (int(sa[m, k // 32]) - 127)
                bv = Fraction(float(decode(qb[n, k], fb))) * Fraction(2) ** (int(sb[n, k // 32]) - 127)
                acc += av * bv
            out[m][n] = acc
    return out


@pytest.mark.parametrize("fa,fb", [(E4M3, E4M3), (E5M2, E4M3), (E4M3, E5M2)], ids=["e4m3xe4m3", "e5m2xe4m3", "e4m3xe5m2"])
def test_gemm_brute_force_exact(fa, fb):
    rng = np.random.default_rng(9)
    M, N, K = 3, 5, 128
    qa, qb = rand_codes(rng, (M, K), fa), rand_codes(rng, (N, K), fb)
    sa = rng.integers(120, 135, size=(M, K // 32)).astype(np.uint8)
    sb = rng.integers(120, 135, size=(N, K // 32)).astype(np.uint8)
    d, aux, s = mx_gemm(qa, sa, fa, qb, sb, fb)
    ref = brute_gemm(qa, sa, fa, qb, sb, fb)
    assert aux is None
    for m in range(M):
        for n in range(N):
            # fp64 matmul of exactly representable operands: error far below 1e-12 * S
            assert abs(Fraction(d[m, n]) - ref[m][n]) <= Fraction(1e-12) * Fraction(s[m, n])


def test_gemm_hand_cases():
    K = 128
    ones = np.full((1, K), 0x38, np.uint8)
    s127 = np.full((1, K // 32), 127, np.uint8)
    d, _, s = mx_gemm(ones, s127, E4M3, ones, s127, E4M3)
    assert d[0, 0] == 128 and s[0, 0] == 128
    d, _, _ = mx_gemm(ones, s127 + 1, E4M3, ones, s127 + 1, E4M3)
    assert d[0, 0] == 512
    # one-hot row of A picks column k of each B row times the scales of block k // 32
    rng = np.random.default_rng(0)
    qb = rand_codes(rng, (4, K), E4M3)
    sb = rng.integers(125, 130, size=(4, K // 32)).astype(np.uint8)
    for k in (0, 31, 32, 77, 127):
        qa = np.zeros((1, K), np.uint8)
        qa[0, k] = 0x40  # 2.0
        sa = np.full((1, K // 32), 126, np.uint8)  # 0.5
        d, _, _ = mx_gemm(qa, sa, E4M3, qb, sb, E4M3)
        want = decode(qb[:, k], E4M3) * np.ldexp(1.0, sb[:, k // 32].astype(np.int64) - 127)
        assert np.array_equal(d[0], want)


def test_gemm_is_not_transposed():
    # A [2, 64] with distinct rows, B [3, 64]: D[m, n] = <A_m, B_n>, shape [2, 3]
    qa = np.zeros((2, 64), np.uint8)
    qb = np.zeros((3, 64), np.uint8)
    qa[0, 0] = 0x38; qa[1, 1] = 0x40          # A0 = e0, A1 = 2 e1
    qb[0, 0] = 0x48; qb[1, 1] = 0x38; qb[2, 0] = 0x38; qb[2, 1] = 0x38  # B0 = 4 e0, B1 = e1, B2 = e0 + e1
    s = np.full((2, 2), 127, np.uint8)
    d, _, _ = mx_gemm(qa, s, E4M3, qb, np.full((3, 2), 127, np.uint8), E4M3)
    assert np.array_equal(d, np.array([[4.0, 0.0, 1.0], [0.0, 2.0, 2.0]]))


def test_gelu_tanh_against_torch_and_identities():
    x = np.concatenate([np.linspace(-12, 12, 20001), np.ldexp(1.0, np.arange(-40, 10))])
    ref = torch.nn.functional.gelu(torch.from_numpy(x), approximate="tanh").numpy()
    # torch evaluates 1 + tanh(u) directly, which cancels for u << 0: compare
    # to it within a few ulps of |x|, and pin the far tail to its asymptote.
    assert np.all(np.abs(gelu_tanh(x) - ref) <= 4e-16 * np.maximum(np.abs(x), 1e-300) + 1e-300)
    mid = np.abs(ref) > 1e-2  # away from the cancelling tail torch's form is accurate
    assert np.allclose(gelu_tanh(x[mid]), ref[mid], rtol=1e-13, atol=0)
    tail = np.linspace(-19, -8, 101)  # e^{2u} < 1e-21 and results stay normal doubles
    u = math.sqrt(2 / math.pi) * (tail + 0.044715 * tail ** 3)
    # 0.5 x (1 + tanh u) = x e^{2u} / (1 + e^{2u}) = x e^{2u} (1 - e^{2u} + ...)
    assert np.allclose(gelu_tanh(tail), tail * np.exp(2 * u), rtol=1e-12, atol=0)
    assert gelu_tanh(0.0) == 0.0
    assert np.allclose(gelu_tanh(x) - gelu_tanh(-x), x, rtol=1e-12, atol=1e-15)
    assert np.all(gelu_tanh(x[x > 0]) > 0) and np.all(gelu_tanh(x[x < 0]) < 0)
    big = np.array([20.0, 50.0, 100.0])
    assert np.all(np.abs(gelu_tanh(big) / big - 1) < 1e-15)
    # the tanh-form constant: at x = 1, 0.5 (1 + tanh(sqrt(2/pi) * 1.044715))
    assert math.isclose(float(gelu_tanh(1.0)), 0.5 * (1 + math.tanh(math.sqrt(2 / math.pi) * 1.044715)), rel_tol=1e-15)


def test_dgelu_tanh_against_differences_autograd_and_limits():
    x = np.linspace(-8, 8, 4001)
    # central differences of the (separately pinned) gelu_tanh: error O(h^2)
    h = 1e-5
    fd = (gelu_tanh(x + h) - gelu_tanh(x - h)) / (2 * h)
    assert np.allclose(dgelu_tanh(x), fd, rtol=0, atol=1e-8)
    # torch autograd of its own tanh GELU, in float64
    t = torch.from_numpy(x.copy()).requires_grad_(True)
    torch.nn.functional.gelu(t, approximate="tanh").sum().backward()
    assert np.allclose(dgelu_tanh(x), t.grad.numpy(), rtol=1e-12, atol=1e-14)
    assert dgelu_tanh(0.0) == 0.5
    assert abs(float(dgelu_tanh(12.0)) - 1.0) < 1e-15 and abs(float(dgelu_tanh(-12.0))) < 1e-15
    # its maximum, ~1.1289 near x = 1.4 (also what bounds error propagation through GELU)
    assert 1.128 < np.max(dgelu_tanh(x)) < 1.13


def test_backward_epilogues():
    rng = np.random.default_rng(13)
    y = rng.standard_normal((3, 5))   # non-square: an elementwise mix-up of axes would fail
    pre = (rng.standard_normal((3, 5)).astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    d, aux = epilogue(y, None, "dgelu", aux_in=pre)
    assert aux is None and np.array_equal(d, y * dgelu_tanh(bf16_to_float64(pre)))
    zeros = np.zeros((3, 5), np.uint16)
    d, _ = epilogue(y, None, "dgelu", aux_in=zeros)
    assert np.array_equal(d, 0.5 * y)   # gelu'(0) = 1/2
    c = rng.standard_normal((3, 5)).astype(np.float32)
    d, aux = epilogue(y, None, "accumulate", c_in=c)
    assert aux is None and np.array_equal(d, c.astype(np.float64) + y)
    # through mx_gemm: one-hot operands pick single products
    qa = np.zeros((2, 128), np.uint8); qa[0, 3] = 0x38; qa[1, 70] = 0x40   # 1.0, 2.0 (E4M3)
    qb = np.zeros((3, 128), np.uint8); qb[1, 3] = 0x38; qb[2, 70] = 0x38
    sa = np.full((2, 4), 127, np.uint8); sb = np.full((3, 4), 127, np.uint8)
    cc = np.arange(6, dtype=np.float32).reshape(2, 3)
    d, _, _ = mx_gemm(qa, sa, E4M3, qb, sb, E4M3, epi="accumulate", c_in=cc)
    assert np.array_equal(d, cc + np.array([[0, 1.0, 0], [0, 0, 2.0]]))


def test_epilogue_bias_and_aux():
    rng = np.random.default_rng(12)
    y = rng.standard_normal((4, 16))
    bias = (rng.standard_normal(16).astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    b = bf16_to_float64(bias)
    d, aux = epilogue(y, None, "none")
    assert d is y and aux is None
    d, aux = epilogue(y, bias, "bias")
    assert aux is None and np.array_equal(d, y + b[None, :])
    d, aux = epilogue(y, bias, "bias_gelu_aux")
    assert np.array_equal(aux, y + b[None, :])
    assert np.array_equal(d, gelu_tanh(y + b[None, :]))
    with pytest.raises(ValueError):
        epilogue(y, bias, "gelu")


def test_grouped_against_dense_blocks():
    rng = np.random.default_rng(21)
    G, N, K = 4, 32, 128
    splits = [5, 0, 17, 3]
    T = sum(splits)
    qa = rand_codes(rng, (T, K), E4M3)
    sa = rng.integers(124, 131, size=(T, K // 32)).astype(np.uint8)
    qb = rand_codes(rng, (G * N, K), E4M3)
    sb = rng.integers(124, 131, size=(G * N, K // 32)).astype(np.uint8)
    bias = (rng.standard_normal((G, N)).astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    d, aux, s = grouped_mx_gemm(splits, qa, sa, E4M3, qb, sb, E4M3, N, bias, "bias_gelu_aux")
    full, _, full_s = mx_gemm(qa, sa, E4M3, qb, sb, E4M3)  # [T, G*N]
    off = 0
    for e, me in enumerate(splits):
        blk = full[off:off + me, e * N:(e + 1) * N] + bf16_to_float64(bias[e])[None, :]
        assert np.allclose(aux[off:off + me], blk, rtol=1e-15, atol=0)
        assert np.allclose(d[off:off + me], gelu_tanh(blk), rtol=1e-14, atol=0)
        assert np.array_equal(s[off:off + me], full_s[off:off + me, e * N:(e + 1) * N])
        off += me
    with pytest.raises(ValueError):
        grouped_mx_gemm([5, 0, 17, 2], qa, sa, E4M3, qb, sb, E4M3, N)


def test_tolerance_bound():
    y_ref = np.array([[1.0, -2.0, 0.0]])
    s = np.array([[10.0, 100.0, 1000.0]])
    bound = tolerance_bound(y_ref, s)
    assert np.allclose(bound, [[2 ** -8 + 1e-4, 2 ** -7 + 1e-3, 1e-2]])
    assert within_tolerance(y_ref + 0.99 * bound, y_ref, s).all()
    assert not within_tolerance(y_ref + 1.01 * bound, y_ref, s).any()
    bias = np.array([0x4000, 0x4000, 0x4000], np.uint16)  # 2.0
    assert np.allclose(tolerance_bound(y_ref, s, bias) - bound, 2e-5)
