"""CPU oracle for the MXFP8 Linear hot path (test infrastructure only).

This package is a plain, slow, obviously-correct numpy implementation of
what the GPU path computes, written in float64 / exact integer arithmetic
from the definitions the pages give.  It is test infrastructure: only the
test-suite, the smoke check in ``__graft_entry__`` and the ``cpu_baseline``
leg of ``bench.py`` may import it.  The product package never does, and the
oracle imports nothing from the product package (they share no code).

Sources (web pages, cited by title and section):

* "Transformer Engine On ROCm and AMDGPU" (ROCm/TransformerEngine README):
  sections "MXFP8 support on ROCm (gfx95x only)", "Blockwise FP8 GEMM
  support on ROCm" (scales cast to E8M0, power of two), "Two-stage amax
  Kernel", "Experimental Triton Kernels on ROCm" (cast_transpose and
  cast_transpose_bgrad).
* "Getting Started" (Transformer Engine JAX quickstart): the baseline MLP
  (GELU with the tanh approximation) and "Enabling Quantization" (HYBRID
  format, DelayedScaling with margin 0).
* "Workflow: NVIDIA TransformerEngine FP8 Training Quickstart", Step 4:
  E4M3 for forward tensors and E5M2 for gradients in HYBRID mode;
  Float8CurrentScaling computes the scale from the current tensor.
* "HipKittens MXFP8 GEMM Support" (ROCm/TransformerEngine PR #566):
  description (BIAS and GELU AUX epilogues) and review threads (MXFP8 1D
  scaling mode, K multiple of 128, M and N multiples of 16).

The pages do not define the MX encoding itself.  The readings taken where
they are silent are the OCP 8-bit floating point and OCP Microscaling (MX)
conventions: 32-element blocks, scale exponent floor(log2(block amax))
minus the element format's largest exponent, saturating round to nearest
even.  Each module states the readings it relies on.

Parity status: every function here is pinned by the CPU tests in
``tests/test_oracle_*.py`` (exhaustive code enumeration, brute-force
argmin encoding, library casts, invariants, exact-integer GEMMs and
hand-worked golden blocks).  No function is parity-unpinned.
"""

from .formats import E4M3, E5M2, FP8Format, decode, encode, e8m0_decode, format_by_name
from .mx import block_scale_code, quantize_rowwise, quantize_colwise, dequantize
from .current_scaling import amax, current_scale, cast_current_scaling
from .bgrad import column_sums, column_abs_sums
from .delayed_scaling import delayed_scaling_step, next_scale, fp8_gemm_per_tensor
from .blockwise import quantize_1d, quantize_2d, block_gemm, pow2_at_least, e8m0_of
from .gemm import mx_gemm, gelu_tanh, dgelu_tanh, epilogue, grouped_mx_gemm, within_tolerance, tolerance_bound

__all__ = [
    "E4M3", "E5M2", "FP8Format", "decode", "encode", "e8m0_decode", "format_by_name",
    "block_scale_code", "quantize_rowwise", "quantize_colwise", "dequantize",
    "amax", "current_scale", "cast_current_scaling",
    "mx_gemm", "gelu_tanh", "epilogue", "grouped_mx_gemm", "within_tolerance", "tolerance_bound",
]
