"""Blockwise FP8 (1-D 1x128 and 2-D 128x128 blocks) and the blockwise FP8 GEMM.

Test infrastructure (see the package docstring).

What the pages fix ("Transformer Engine On ROCm and AMDGPU", section
"Blockwise FP8 GEMM support on ROCm (gfx942 and gfx950)"):
* the GEMM takes 1Dx2D or 1Dx1D block scaling, E4M3 / E5M2 inputs in any
  pair except E5M2 x E5M2, and bias / DGELU epilogues;
* on gfx950 the default kernel casts the incoming FP32 scales to E8M0 (a
  power of two) and computes with those, and the same setting makes the
  blockwise recipe produce power-of-two scales; a second kernel uses the
  FP32 scales directly.

Readings where the pages are silent:
* A 1-D block is 128 consecutive elements of a row along K (the GEMM's
  contraction axis); a 2-D block is 128 rows x 128 K-elements.  Scales are
  stored as their inverses (the factor that dequantizes): scale_inv[r, kb]
  for 1-D, scale_inv[r // 128, kb] for 2-D.
* The recipe's power-of-two scale_inv for a block with amax a > 0 is the
  smallest power of two >= a / fmt_max, so every |x| / scale_inv <= fmt_max
  (no block saturates); a zero block gets scale_inv = 1.  Codes are the
  saturating round-to-nearest-even encodes of x / scale_inv (exact division).
* The E8M0 cast of an FP32 scale_inv s > 0 is the smallest power of two >= s
  (exact for the recipe's own power-of-two scales), kept within E8M0's range
  2^-127 .. 2^127; NaN and negative s have no E8M0 value and map to its NaN
  code.
* GEMM: D = epilogue(sum_kb sa[m, kb] * sb[n, kb] * sum_{k in kb} A_q[m, k] B_q[n, k]),
  with sb[n, kb] read at n // 128 for 2-D B.
"""

from __future__ import annotations

import numpy as np

from .formats import FP8Format, bf16_to_float64, decode, encode
from .gemm import epilogue

BLOCK = 128


def pow2_at_least(v) -> np.ndarray:
    """Elementwise smallest power of two >= v for v > 0 (float64); 1 for v == 0."""
    v = np.asarray(v, dtype=np.float64)
    out = np.ones_like(v)
    pos = v > 0
    m, e = np.frexp(v[pos])          # v = m 2^e with 0.5 <= m < 1
    out[pos] = np.ldexp(1.0, np.where(m == 0.5, e - 1, e))
    return out


def _block_scale_inv(amax, fmt: FP8Format) -> np.ndarray:
    return pow2_at_least(np.asarray(amax, dtype=np.float64) / fmt.max_value)


def quantize_1d(x_bf16, fmt: FP8Format):
    """[R, C] bf16 bits, C % 128 == 0 -> (codes [R, C], scale_inv float32 [R, C/128])."""
    x = bf16_to_float64(np.asarray(x_bf16))
    r, c = x.shape
    if c % BLOCK:
        raise ValueError("1-D blocks need cols % 128 == 0")
    xb = x.reshape(r, c // BLOCK, BLOCK)
    s = _block_scale_inv(np.abs(xb).max(axis=2), fmt)
    q = encode(xb / s[:, :, None], fmt).reshape(r, c)
    return q, s.astype(np.float32)


def quantize_2d(x_bf16, fmt: FP8Format):
    """[R, C] bf16 bits, C % 128 == 0 (R ragged) -> (codes [R, C], scale_inv float32 [ceil(R/128), C/128])."""
    x = bf16_to_float64(np.asarray(x_bf16))
    r, c = x.shape
    if c % BLOCK:
        raise ValueError("2-D blocks need cols % 128 == 0")
    rb = -(-r // BLOCK)
    s = np.ones((rb, c // BLOCK))
    q = np.zeros((r, c), np.uint8)
    for i in range(rb):
        rows = slice(i * BLOCK, min(r, (i + 1) * BLOCK))
        for j in range(c // BLOCK):
            cols = slice(j * BLOCK, (j + 1) * BLOCK)
            blk = x[rows, cols]
            s[i, j] = _block_scale_inv(np.abs(blk).max(), fmt)
            q[rows, cols] = encode(blk / s[i, j], fmt)
    return q, s.astype(np.float32)


def block_gemm(qa, sa_inv, fmt_a: FP8Format, qb, sb_inv, fmt_b: FP8Format, b_2d: bool,
               bias_bf16=None, epi: str = "none", aux_in=None, c_in=None, beta: float = 1.0):
    """D = epilogue(sum_kb sa[m, kb] sb[n(, /128), kb] A_q[m, kb] . B_q[n, kb]); with the accumulate
    epilogue D = beta C + that sum.

    Returns (D, aux, S) with S = sum_k |sa A_q| |sb B_q| (the tolerance weight).
    """
    a = decode(qa, fmt_a)
    b = decode(qb, fmt_b)
    m, k = a.shape
    n = b.shape[0]
    sa = np.asarray(sa_inv, dtype=np.float64)
    sb = np.asarray(sb_inv, dtype=np.float64)
    if b_2d:
        sb = np.repeat(sb, BLOCK, axis=0)[:n]
    a_hat = a * np.repeat(sa, BLOCK, axis=1)
    b_hat = b * np.repeat(sb, BLOCK, axis=1)
    y = np.matmul(a_hat, b_hat.T)
    s = np.matmul(np.abs(a_hat), np.abs(b_hat).T)
    d, aux = epilogue(y, bias_bf16, epi, aux_in, c_in, beta)
    return d, aux, s


def e8m0_of(scale_inv) -> np.ndarray:
    """The E8M0 codes (biased exponents) of the E8M0 cast of FP32 scale inverses: the smallest
    E8M0 value (2^-127 .. 2^127) >= s, or 2^127 above that range (+inf included); s = +-0 gives
    2^-127; NaN and negative s give the E8M0 NaN code 255 (there is no negative scale)."""
    v = np.asarray(scale_inv, dtype=np.float64)
    bad = np.isnan(v) | (v < 0)
    w = np.clip(np.where(bad, 1.0, v), 2.0 ** -127, 2.0 ** 127)
    code = np.log2(pow2_at_least(w)).round().astype(np.int64) + 127
    return np.where(bad, 255, code).astype(np.uint8)


def dequantize_1d(q, scale_inv, fmt: FP8Format) -> np.ndarray:
    return decode(q, fmt) * np.repeat(np.asarray(scale_inv, np.float64), BLOCK, axis=1)

