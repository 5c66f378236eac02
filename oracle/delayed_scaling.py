"""Delayed scaling (FP8 cast with a scale from an amax history) and the
per-tensor FP8 GEMM it feeds.

Test infrastructure (see the package docstring).

What the pages fix:
* "Getting Started" (TE JAX quickstart), the README example and "Enabling
  Quantization": the DelayedScaling recipe with margin 0, interval 1, the
  HYBRID format, an amax history of length 16 and the "max" algorithm.
* "Workflow: NVIDIA TransformerEngine FP8 Training Quickstart", Step 4:
  delayed scaling keeps a history window of amax values for a stable scale
  (current scaling instead takes the scale from the current tensor).

Readings where the pages are silent:
* A tensor's state is its scale s (initially 1) and its amax history
  h[0..L-1], newest first (initially zeros).  One step on a tensor x:
  1. x is cast with the scale the history has given so far:
     q = enc_sat_rne(fl32(x * s)), carried with q_scale_inv = fl32(1 / s);
  2. a = amax(x) enters the history: h <- [a, h[0], ..., h[L-2]];
  3. r = max(h) ("max") or h[0] ("most_recent"); when r is positive and
     finite the next scale is fl32(fl32(fmt_max / r) / 2^margin) (a quotient
     beyond float32 becomes the largest finite float32), otherwise s is kept.
  The scale is therefore "delayed": it reflects the amaxes of earlier steps.
  `interval` (how often the scale is updated) is left to the caller, which
  runs an update every interval steps.
* Per-tensor FP8 GEMM: D = epilogue(a_scale_inv * b_scale_inv * A_q . B_q^T)
  with A_q, B_q the decoded codes and the epilogues of the MXFP8 GEMM;
  a_scale_inv * b_scale_inv is the GEMM's alpha.
"""

from __future__ import annotations

import numpy as np

from .current_scaling import FLT_MAX, amax
from .formats import FP8Format, bf16_to_float64, decode, encode
from .gemm import epilogue

ALGOS = ("max", "most_recent")


def next_scale(history, scale, fmt: FP8Format, algo: str = "max", margin: int = 0) -> np.float32:
    """The scale for the next step from an amax history (newest first)."""
    if algo not in ALGOS:
        raise ValueError(f"unknown amax algorithm {algo!r}")
    h = np.asarray(history, dtype=np.float32)
    r = np.float32(h.max() if algo == "max" else h[0])
    if not (r > 0 and np.isfinite(r)):
        return np.float32(scale)
    with np.errstate(over="ignore"):
        s = np.float32(fmt.max_value) / r  # IEEE float32 division
    if not np.isfinite(s):
        s = FLT_MAX
    return np.float32(s / np.float32(2.0 ** margin))


def delayed_scaling_step(x_bf16, fmt: FP8Format, history, scale, algo: str = "max", margin: int = 0):
    """One step: -> (q, q_scale_inv, amax, new_history, new_scale)."""
    x = np.asarray(x_bf16)
    s = np.float32(scale)
    xf32 = bf16_to_float64(x).astype(np.float32)
    with np.errstate(over="ignore"):
        y = xf32 * s  # float32 multiply, round to nearest even
    q = encode(y.astype(np.float64), fmt).reshape(x.shape)
    q_scale_inv = np.float32(1.0) / s
    a = amax(x)
    h = np.asarray(history, dtype=np.float32)
    new_h = np.concatenate([[a], h[:-1]]).astype(np.float32)
    return q, q_scale_inv, a, new_h, next_scale(new_h, s, fmt, algo, margin)


def fp8_gemm_per_tensor(qa, a_scale_inv, fmt_a: FP8Format, qb, b_scale_inv, fmt_b: FP8Format,
                        bias_bf16=None, epi: str = "none"):
    """D = epilogue(a_scale_inv * b_scale_inv * decode(A) @ decode(B)^T).

    Returns (D, aux, S) with S = |alpha| |A_q| @ |B_q|^T, the tolerance weight.
    """
    alpha = float(np.float64(a_scale_inv) * np.float64(b_scale_inv))
    a = decode(qa, fmt_a)
    b = decode(qb, fmt_b)
    y = alpha * np.matmul(a, b.T)
    s = abs(alpha) * np.matmul(np.abs(a), np.abs(b).T)
    d, aux = epilogue(y, bias_bf16, epi)
    return d, aux, s
