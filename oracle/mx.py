"""MXFP8 1-D block quantization (rowwise and columnwise) and dequantization.

Test infrastructure (see the package docstring).

What the pages fix:
* "Transformer Engine On ROCm and AMDGPU", section "MXFP8 support on ROCm
  (gfx95x only)": MXFP8 is a recipe on gfx95x; "HipKittens MXFP8 GEMM
  Support" (PR #566), review threads: the tensors carry the 1-D MXFP8
  scaling mode, and the GEMM needs K to be a multiple of 128.
* "Transformer Engine On ROCm and AMDGPU", section "Blockwise FP8 GEMM
  support": the block scale is E8M0, a power of two.
* "Workflow: NVIDIA TransformerEngine FP8 Training Quickstart", Step 4:
  E4M3 for forward tensors, E5M2 for gradients (HYBRID).

Readings where the pages are silent (OCP Microscaling convention):
* A block is 32 consecutive elements along the quantization axis (the K
  axis of the GEMM operand that will consume it).
* Block scale exponent: floor(log2(amax)) - emax_elem, where amax is the
  largest magnitude in the block and emax_elem is the exponent of the
  element format's largest finite value (8 for E4M3, 15 for E5M2),
  clamped to [-127, 127] and stored biased by 127 as E8M0.  A block whose
  amax is zero gets code 0 (log2(0) = -inf clamps to -127).  A block
  holding Inf or NaN gets code 255 (outside the tested domain).
* Element codes: saturating round-to-nearest-even of x / 2^(code - 127).
  With the floor rule, magnitudes in [464, 512) * 2^s saturate to 448 * 2^s.
* Rowwise: blocks along the last (contiguous) axis; data [R, C], scales
  [R, C/32].  Columnwise: blocks along the first axis, stored transposed;
  data [C, R], scales [C, R/32] (the transposed copy a "TN" GEMM needs for
  the backward pass, cf. the cast-transpose kernels named in "Experimental
  Triton Kernels on ROCm").
"""

from __future__ import annotations

import numpy as np

from .formats import FP8Format, bf16_to_float64, decode, encode, e8m0_decode

BLOCK = 32


def block_scale_code(amax, fmt: FP8Format) -> np.ndarray:
    """E8M0 code of a block scale from the block's (non-negative) amax."""
    a = np.asarray(amax, dtype=np.float64)
    finite = np.isfinite(a)
    pos = finite & (a > 0)
    # frexp gives a = f * 2^e with f in [0.5, 1): floor(log2(a)) = e - 1 exactly.
    _, e = np.frexp(np.where(pos, a, 1.0))
    unbiased = np.clip(e.astype(np.int64) - 1 - fmt.emax, -127, 127)
    code = np.where(pos, unbiased + 127, 0)
    code = np.where(finite, code, 255)
    return code.astype(np.uint8)


def _quantize_blocks(xb: np.ndarray, fmt: FP8Format, axis: int):
    """Quantize float64 values whose 32-element blocks lie along ``axis``."""
    amax = np.max(np.abs(xb), axis=axis)
    code = block_scale_code(amax, fmt)
    shift = np.expand_dims(code.astype(np.int64) - 127, axis)
    scaled = np.ldexp(xb, -shift)  # exact: multiplication by a power of two
    q = encode(scaled, fmt)
    return q, code


def quantize_rowwise(x_bf16, fmt: FP8Format):
    """bf16 [R, C] (uint16 bit patterns) -> (codes uint8 [R, C], scales uint8 [R, C/32])."""
    x = np.asarray(x_bf16)
    R, C = x.shape
    if C % BLOCK:
        raise ValueError("rowwise quantization needs cols % 32 == 0")
    xf = bf16_to_float64(x).reshape(R, C // BLOCK, BLOCK)
    q, code = _quantize_blocks(xf, fmt, axis=2)
    return q.reshape(R, C), code.reshape(R, C // BLOCK)


def quantize_colwise(x_bf16, fmt: FP8Format):
    """bf16 [R, C] -> blocks of 32 down each column, stored transposed:
    (codes uint8 [C, R], scales uint8 [C, R/32])."""
    x = np.asarray(x_bf16)
    R, C = x.shape
    if R % BLOCK:
        raise ValueError("columnwise quantization needs rows % 32 == 0")
    xf = bf16_to_float64(x).reshape(R // BLOCK, BLOCK, C)
    q, code = _quantize_blocks(xf, fmt, axis=1)
    # q: [R/32, 32, C] -> [R, C] -> transposed [C, R]; code: [R/32, C] -> [C, R/32]
    return np.ascontiguousarray(q.reshape(R, C).T), np.ascontiguousarray(code.T)


def dequantize(codes, scales, fmt: FP8Format) -> np.ndarray:
    """Exact float64 values of an MXFP8 tensor with blocks along the last axis."""
    q = np.asarray(codes)
    s = np.asarray(scales)
    R, C = q.shape
    if s.shape != (R, C // BLOCK):
        raise ValueError("scale shape must be [rows, cols/32]")
    vals = decode(q, fmt).reshape(R, C // BLOCK, BLOCK)
    return (vals * e8m0_decode(s)[:, :, None]).reshape(R, C)
