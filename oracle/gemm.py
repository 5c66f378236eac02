"""MXFP8 GEMM with bias / GELU(tanh) / GELU-aux epilogues, dense and grouped.

Test infrastructure (see the package docstring).

What the pages fix:
* "HipKittens MXFP8 GEMM Support" (PR #566), description: an MXFP8 GEMM
  with BIAS and GELU AUX epilogues; review threads: the GEMM is wanted in
  "TN" layout, K must be a multiple of 128 and M, N multiples of 16.
* "Getting Started" (TE JAX quickstart), baseline MLP: the activation is
  GELU with the tanh approximation.
* "Transformer Engine On ROCm and AMDGPU", sections "Single-Launch Grouped
  GEMM" / "Grouped GEMM using CK_Tile": one grouped GEMM over all experts.

Definitions used (the GEMM has a plain definition, so the oracle is that
definition written out, in float64):
* Operands are MXFP8 tensors in "TN" layout: A is [M, K] and B is [N, K],
  both with 32-element blocks along K.  Each is dequantized exactly
  (code value times 2^(scale - 127)) and Y = A_hat @ B_hat^T in float64.
  The hardware accumulates in fp32; that difference is covered by the
  acceptance tolerance below, not modelled.
* Epilogues: none -> D = Y; bias -> D = Y + bias[n]; bias_gelu_aux ->
  pre = Y + bias[n], aux = pre, D = gelu_tanh(pre).
* Backward epilogues (readings; the pages name the bias_gelu_aux forward
  and the FP8 backward GEMMs, not these details):
  - dgelu: the GEMM that produces the gradient of GELU's output multiplies
    it by GELU's derivative at the saved pre-activation aux (bf16 [M, N]):
    D = Y * gelu_tanh'(aux).  That is the gradient of the pre-activation.
  - accumulate: the weight-gradient GEMM adds into an existing fp32 main
    gradient C [M, N]: D = beta C + Y, beta = 1 unless given ("Transformer
    Engine On ROCm and AMDGPU", "Blockwise FP8 GEMM support on ROCm (gfx942
    and gfx950)", lists beta among the blockwise GEMM's epilogues).
* gelu_tanh(x) = 0.5 x (1 + tanh(sqrt(2/pi) (x + 0.044715 x^3))) (the
  tanh approximation of Hendrycks and Gimpel, "Gaussian Error Linear
  Units", 2016; the pages only name the tanh approximation).
* Acceptance (reading): an output y matches its reference y_ref when
  |y - y_ref| <= 2^-8 |y_ref| + 1e-5 (S + |bias[n]|), where
  S[m, n] = sum_k |A_hat[m, k]| |B_hat[n, k]|.  The |bias| term covers
  epilogue outputs; it is zero without bias.
* Grouped: expert e owns rows [off_e, off_e + M_e) of A and D, where off_e
  is the sum of the earlier M_e; D_e = epilogue(A_e @ B_e^T, bias_e).
"""

from __future__ import annotations

import math

import numpy as np

from .formats import FP8Format, bf16_to_float64
from .mx import dequantize

EPILOGUES = ("none", "bias", "bias_gelu_aux", "dgelu", "accumulate")


def gelu_tanh(x) -> np.ndarray:
    """0.5 x (1 + tanh(u)), u = sqrt(2/pi) (x + 0.044715 x^3).

    1 + tanh(u) is evaluated as the identical quantity 2 / (1 + exp(-2u)),
    which does not cancel when tanh(u) is close to -1 (x well below zero).
    """
    x = np.asarray(x, dtype=np.float64)
    c = math.sqrt(2.0 / math.pi)
    u = c * (x + 0.044715 * x * x * x)
    with np.errstate(over="ignore"):
        one_plus_tanh = 2.0 / (1.0 + np.exp(-2.0 * u))
    return 0.5 * x * one_plus_tanh


def dgelu_tanh(x) -> np.ndarray:
    """d/dx gelu_tanh(x), from the product and chain rules.

    With s = (1 + tanh(u)) / 2 = 1 / (1 + exp(-2u)) and u' = sqrt(2/pi) (1 + 3 * 0.044715 x^2):
    gelu_tanh(x) = x s, and ds/dx = 2 s (1 - s) u', so the derivative is s + 2 x s (1 - s) u'.
    """
    x = np.asarray(x, dtype=np.float64)
    c = math.sqrt(2.0 / math.pi)
    u = c * (x + 0.044715 * x * x * x)
    du = c * (1.0 + 3.0 * 0.044715 * x * x)
    with np.errstate(over="ignore"):
        s = 1.0 / (1.0 + np.exp(-2.0 * u))
    return s + 2.0 * x * s * (1.0 - s) * du


def epilogue(y, bias_bf16, epi: str, aux_in=None, c_in=None, beta: float = 1.0):
    """Apply an epilogue to float64 GEMM results y [M, N].

    aux_in: bf16 bit patterns [M, N] of the saved pre-activation (dgelu only);
    c_in: the fp32 values [M, N] accumulated into, times beta (accumulate only).
    Returns (D, aux) as float64; aux is None unless epi == "bias_gelu_aux".
    """
    if epi not in EPILOGUES:
        raise ValueError(f"unknown epilogue {epi!r}")
    if epi == "none":
        return y, None
    if epi == "dgelu":
        return y * dgelu_tanh(bf16_to_float64(np.asarray(aux_in))), None
    if epi == "accumulate":
        return float(beta) * np.asarray(c_in, dtype=np.float64) + y, None
    b = bf16_to_float64(np.asarray(bias_bf16))
    pre = y + b[None, :]
    if epi == "bias":
        return pre, None
    return gelu_tanh(pre), pre


def mx_gemm(qa, sa, fmt_a: FP8Format, qb, sb, fmt_b: FP8Format, bias_bf16=None, epi: str = "none",
            aux_in=None, c_in=None):
    """D = epilogue(dequant(A) @ dequant(B)^T).

    qa [M, K] / sa [M, K/32] and qb [N, K] / sb [N, K/32] are MXFP8 codes and
    E8M0 scales.  Returns (D, aux, S): float64 reference outputs and the
    tolerance weight S = |A_hat| @ |B_hat|^T.
    """
    a = dequantize(qa, sa, fmt_a)
    b = dequantize(qb, sb, fmt_b)
    y = np.matmul(a, b.T)
    s = np.matmul(np.abs(a), np.abs(b).T)
    d, aux = epilogue(y, bias_bf16, epi, aux_in, c_in)
    return d, aux, s


def grouped_mx_gemm(m_splits, qa, sa, fmt_a: FP8Format, qb, sb, fmt_b: FP8Format, n: int,
                    bias_bf16=None, epi: str = "none"):
    """Grouped GEMM over experts; B is [G*N, K] stacked, bias [G, N].

    Returns (D, aux, S) over all total_m rows (aux None without GELU-aux).
    """
    splits = [int(m) for m in m_splits]
    total_m = qa.shape[0]
    if sum(splits) != total_m or any(m < 0 for m in splits):
        raise ValueError("m_splits must be non-negative and sum to the rows of A")
    d = np.zeros((total_m, n))
    s = np.zeros((total_m, n))
    aux = np.zeros((total_m, n)) if epi == "bias_gelu_aux" else None
    off = 0
    for e, me in enumerate(splits):
        rows = slice(off, off + me)
        cols = slice(e * n, (e + 1) * n)
        be = None if bias_bf16 is None else np.asarray(bias_bf16)[e]
        de, auxe, se = mx_gemm(qa[rows], sa[rows], fmt_a, qb[cols], sb[cols], fmt_b, be, epi)
        d[rows] = de
        s[rows] = se
        if aux is not None:
            aux[rows] = auxe
        off += me
    return d, aux, s


def tolerance_bound(y_ref, s, bias_bf16=None) -> np.ndarray:
    """Per-element acceptance bound 2^-8 |y_ref| + 1e-5 (S + |bias[n]|)."""
    y_ref = np.asarray(y_ref, dtype=np.float64)
    b = 0.0 if bias_bf16 is None else np.abs(bf16_to_float64(np.asarray(bias_bf16)))[None, :]
    return 2.0 ** -8 * np.abs(y_ref) + 1e-5 * (np.asarray(s) + b)


def within_tolerance(y, y_ref, s, bias_bf16=None) -> np.ndarray:
    """Boolean mask: which outputs y (any float dtype) meet the bound."""
    y = np.asarray(y, dtype=np.float64)
    return np.abs(y - np.asarray(y_ref, dtype=np.float64)) <= tolerance_bound(y_ref, s, bias_bf16)
