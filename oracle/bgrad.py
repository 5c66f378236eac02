"""Bias gradient: the column sums of an output gradient.

Test infrastructure (see the package docstring).

What the pages fix: "Transformer Engine On ROCm and AMDGPU", section
"Experimental Triton Kernels on ROCm", names cast_transpose and
cast_transpose_bgrad as the kernels FP8 training leans on: the gradient of a
Linear's output is cast (both layouts, since the backward GEMMs want it
along either axis) and, in the same pass, reduced into the gradient of the
layer's bias.

Readings where the pages are silent:
* For an output gradient dY [tokens, features] and a Linear y = x W^T + b,
  the bias gradient is db[f] = sum over tokens t of dY[t, f]: the sum over
  the first axis, one value per column.
* dY is bf16 (the inputs of the quantize path are bf16).  Here the exactly
  decoded values are summed in float64, whose rounding error (at most about
  R * 2^-53 * sum |x|) is far below that of the GPU's fp32 accumulation; the
  two agree within the fp32 summation bound that the tests state.
"""

from __future__ import annotations

import numpy as np

from .formats import bf16_to_float64


def column_sums(x_bf16) -> np.ndarray:
    """db[c] = sum_r x[r, c] for a bf16 matrix given as uint16 bit patterns
    [R, C]; float64 [C].  R = 0 gives zeros."""
    x = bf16_to_float64(np.asarray(x_bf16, dtype=np.uint16))
    if x.ndim != 2:
        raise ValueError("column_sums takes a 2-D [rows, cols] array")
    out = np.zeros(x.shape[1], dtype=np.float64)
    for r in range(x.shape[0]):  # row by row: the definition, in row order
        out += x[r]
    return out


def column_abs_sums(x_bf16) -> np.ndarray:
    """sum_r |x[r, c]| per column: the scale of the fp32 summation error bound."""
    x = bf16_to_float64(np.asarray(x_bf16, dtype=np.uint16))
    return np.abs(x).sum(axis=0) if x.shape[0] else np.zeros(x.shape[1], dtype=np.float64)
