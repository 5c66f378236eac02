"""Per-tensor current scaling: amax -> scale -> FP8 cast.

Test infrastructure (see the package docstring).

What the pages fix:
* "Transformer Engine On ROCm and AMDGPU", section "Two-stage amax
  Kernel": the amax of a tensor is computed as per-block maxima followed
  by a small reduction over them (no atomics).  The maximum of magnitudes
  does not depend on the reduction order, so the result is the plain
  maximum.
* "Workflow: NVIDIA TransformerEngine FP8 Training Quickstart", Step 4:
  Float8CurrentScaling derives the scale from the current tensor on each
  pass (as opposed to an amax history).
* "Getting Started" (TE JAX quickstart), "Enabling Quantization" and the
  README example: recipes use margin 0.

Readings where the pages are silent:
* scale = fl32(fmt_max / amax), fmt_max = 448 (E4M3) or 57344 (E5M2), as
  a correctly rounded float32 division.  amax == 0 gives scale = 1.  A
  quotient that overflows float32 is clamped to the largest finite
  float32.
* scale_inv = fl32(1 / scale), also a correctly rounded float32 division.
* Each element: y = fl32(x * scale) (float32 multiply, round to nearest
  even), then the saturating round-to-nearest-even FP8 encode of y.
"""

from __future__ import annotations

import numpy as np

from .formats import FP8Format, bf16_to_float64, encode

FLT_MAX = np.float32(np.finfo(np.float32).max)


def amax(x_bf16) -> np.float32:
    """max |x_i| over the whole tensor (exact; bf16 values are exact in float32)."""
    xf = bf16_to_float64(np.asarray(x_bf16).ravel())
    if xf.size == 0:
        return np.float32(0.0)
    return np.float32(np.max(np.abs(xf)))


def current_scale(amax_value, fmt: FP8Format):
    """(scale, scale_inv) as float32 from a float32 amax."""
    a = np.float32(amax_value)
    if a == 0:
        scale = np.float32(1.0)
    else:
        with np.errstate(over="ignore", divide="ignore"):
            scale = np.float32(fmt.max_value) / a  # IEEE float32 division
        if not np.isfinite(scale):
            scale = FLT_MAX
    scale_inv = np.float32(1.0) / scale
    return np.float32(scale), np.float32(scale_inv)


def cast_current_scaling(x_bf16, fmt: FP8Format):
    """bf16 tensor -> (codes uint8, amax, scale, scale_inv)."""
    x = np.asarray(x_bf16)
    a = amax(x)
    scale, scale_inv = current_scale(a, fmt)
    xf32 = bf16_to_float64(x).astype(np.float32)
    with np.errstate(over="ignore"):
        y = xf32 * scale  # float32 multiply, round to nearest even
    q = encode(y.astype(np.float64), fmt)
    return q.reshape(x.shape), a, scale, scale_inv
