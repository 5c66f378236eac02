"""FP8 element formats (E4M3, E5M2) and the E8M0 block-scale format.

Test infrastructure (see the package docstring): imported only by tests,
the smoke check and the CPU baseline.

What the pages fix:
* "Workflow: NVIDIA TransformerEngine FP8 Training Quickstart", Step 4:
  HYBRID mode uses E4M3 for forward tensors and E5M2 for gradients.
* "Transformer Engine On ROCm and AMDGPU", section "Blockwise FP8 GEMM
  support on ROCm (gfx942 and gfx950)": block scales are cast to E8M0, a
  power of two.

What the pages leave open, and the reading taken (OCP 8-bit floating point
specification, the "FN" E4M3 variant that gfx950 implements):
* E4M3: 1 sign, 4 exponent (bias 7), 3 mantissa bits.  Exponent field 0 is
  subnormal (value m * 2^-9).  Only S.1111.111 is NaN, so the largest
  finite magnitude is 1.75 * 2^8 = 448.  No infinities.
* E5M2: 1 sign, 5 exponent (bias 15), 2 mantissa bits, IEEE-like:
  subnormal m * 2^-16, exponent field 31 is Inf (m = 0) or NaN; largest
  finite magnitude 1.75 * 2^15 = 57344.
* E8M0: an unsigned 8-bit biased exponent, value 2^(c - 127) for c in
  [0, 254]; 255 is NaN.
* Encoding is round-to-nearest with ties to the even code, saturating:
  any magnitude at or above the largest finite value encodes to it.  The
  sign is always kept (negative values that round to zero give 0x80).
"""

from __future__ import annotations

from dataclasses import dataclass

import numpy as np


@dataclass(frozen=True)
class FP8Format:
    name: str
    exp_bits: int
    man_bits: int
    bias: int
    max_code: int      # largest finite positive code
    emax: int          # exponent of the largest finite value (floor(log2(max)))
    max_value: float   # largest finite magnitude

    @property
    def exp_field_max(self) -> int:
        return (1 << self.exp_bits) - 1


E4M3 = FP8Format("e4m3", exp_bits=4, man_bits=3, bias=7, max_code=0x7E, emax=8, max_value=448.0)
E5M2 = FP8Format("e5m2", exp_bits=5, man_bits=2, bias=15, max_code=0x7B, emax=15, max_value=57344.0)


def format_by_name(name: str) -> FP8Format:
    return {"e4m3": E4M3, "e5m2": E5M2}[name.lower()]


def decode(codes, fmt: FP8Format) -> np.ndarray:
    """Value of each 8-bit code as float64, from the bit fields."""
    c = np.asarray(codes, dtype=np.int64) & 0xFF
    sign = np.where((c >> 7) & 1, -1.0, 1.0)
    e = (c >> fmt.man_bits) & fmt.exp_field_max
    m = (c & ((1 << fmt.man_bits) - 1)).astype(np.float64)
    scale_m = float(1 << fmt.man_bits)
    normal = (1.0 + m / scale_m) * np.ldexp(1.0, (e - fmt.bias).astype(np.int64))
    subnormal = (m / scale_m) * np.ldexp(1.0, 1 - fmt.bias)
    mag = np.where(e == 0, subnormal, normal)
    if fmt.name == "e4m3":
        nan = (e == fmt.exp_field_max) & ((c & 0x7) == 0x7)
        mag = np.where(nan, np.nan, mag)
    else:
        special = e == fmt.exp_field_max
        mag = np.where(special & (m == 0), np.inf, mag)
        mag = np.where(special & (m != 0), np.nan, mag)
    return sign * mag


def _finite_grid(fmt: FP8Format) -> np.ndarray:
    """Non-negative finite values of the format, indexed by code 0..max_code.

    Codes 0..max_code are ordered by magnitude, so the grid is sorted and
    the code of a grid point equals its index.
    """
    grid = decode(np.arange(fmt.max_code + 1), fmt)
    assert np.all(np.diff(grid) > 0)
    return grid


def encode(v, fmt: FP8Format) -> np.ndarray:
    """Saturating round-to-nearest-even encode of exact real values.

    ``v`` is float64 (every value the hot path produces before rounding, a
    bf16 times a power of two or an fp32 product, is exact in float64).
    The result is the code of the finite grid point nearest to |v|; when
    |v| lies exactly half-way between two grid points, the one with the
    even code (even mantissa LSB) is taken.  Magnitudes at or beyond the
    largest finite value give the largest finite code.  NaN gives 0x7F
    (with the input's sign bit), which is NaN in both formats.
    """
    v = np.asarray(v, dtype=np.float64)
    grid = _finite_grid(fmt)
    a = np.abs(v)
    neg = np.signbit(v)
    nan = np.isnan(v)
    a_ok = np.where(nan, 0.0, a)
    # grid[hi - 1] < a <= grid[hi]
    hi = np.searchsorted(grid, a_ok, side="left")
    hi = np.clip(hi, 0, fmt.max_code)
    lo = np.clip(hi - 1, 0, fmt.max_code)
    d_lo = np.abs(a_ok - grid[lo])
    d_hi = np.abs(grid[hi] - a_ok)
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (hi % 2 == 0))
    code = np.where(pick_hi, hi, lo)
    code = np.where(a_ok >= fmt.max_value, fmt.max_code, code)
    code = np.where(nan, 0x7F, code)
    code = code | np.where(neg, 0x80, 0)
    return code.astype(np.uint8)


def e8m0_decode(codes) -> np.ndarray:
    """Value 2^(c - 127) of E8M0 scale codes; 255 is NaN."""
    c = np.asarray(codes, dtype=np.int64)
    out = np.ldexp(1.0, c - 127)
    return np.where(c == 255, np.nan, out)


def bf16_to_float64(bits) -> np.ndarray:
    """Exact value of bf16 bit patterns (uint16) as float64."""
    a = np.asarray(bits, dtype=np.uint16)
    b = np.ascontiguousarray(a.astype(np.uint32) << 16)
    with np.errstate(invalid="ignore"):  # NaN patterns stay NaN
        return b.view(np.float32).astype(np.float64).reshape(a.shape)
