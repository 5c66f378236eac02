// Blockwise FP8 scales (one FP32 scale inverse per 1 x 128 or 128 x 128
// block) cast to E8M0 and laid out as MXFP8 scales.
//
// "Transformer Engine On ROCm and AMDGPU", section "Blockwise FP8 GEMM
// support on ROCm (gfx942 and gfx950)": on gfx950 the default blockwise GEMM
// casts the incoming FP32 scales to E8M0 and computes with those.  A 128-wide
// block along K spans four 32-wide MX blocks, which all take its scale, so
// after this cast the MXFP8 GEMM runs unchanged on the blockwise operands.
//
// The cast of s is the smallest E8M0 value >= s (exact for the recipe's own
// power-of-two scales), saturating at 2^127 (+inf included); s = +-0 and
// positive values up to 2^-127 give 2^-127, the smallest E8M0 value.  NaN
// and negative s give the E8M0 NaN code 255.

#include "temx_internal.h"

namespace temx {
namespace {

__device__ __forceinline__ uint32_t e8m0_at_least(float s) {
  const uint32_t u = __float_as_uint(s);
  const uint32_t mag = u & 0x7FFFFFFFu;
  if (mag > 0x7F800000u || (u != mag && mag != 0)) return 255u;  // NaN, or negative non-zero
  const uint32_t e = mag >> 23, m = mag & 0x7FFFFFu;
  if (e == 0) return m > 0x400000u ? 1u : 0u;  // zero and subnormals: 2^-127 (= m 0x400000) or 2^-126
  if (e == 0xFFu) return 254u;                 // +inf
  const uint32_t c = e + (m != 0 ? 1u : 0u);
  return c > 254u ? 254u : c;
}

// Up to two tensors in one launch.  Tensor t has rows[t] rows and kb 128-blocks
// per row; its scale inverse for (row r, block j) is at
// src[t][(r >> shift[t]) * kb + j] (shift 0: 1-D blocks, 7: 128 x 128 blocks).
// Output: uint8 [rows, 4 kb], written as one uint32 (four equal codes) per
// 128-block, so dst[t] is read as uint32 [rows, kb].
struct ExpandParams {
  const float* src[2];
  uint32_t* dst[2];
  int64_t count[2];  // rows * kb
  int64_t kb;
  int shift[2];
};

__global__ __launch_bounds__(256) void block_scale_expand_kernel(ExpandParams p) {
  int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  int t = 0;
  if (i >= p.count[0]) {
    i -= p.count[0];
    t = 1;
    if (i >= p.count[1]) return;
  }
  const float* src = t ? p.src[1] : p.src[0];
  uint32_t* dst = t ? p.dst[1] : p.dst[0];
  const int shift = t ? p.shift[1] : p.shift[0];
  const int64_t r = i / p.kb, j = i - r * p.kb;
  const float s = src[(r >> shift) * p.kb + j];
  dst[i] = e8m0_at_least(s) * 0x01010101u;
}

}  // namespace

te_status launch_block_scale_expand(const float* sa, int64_t rows_a, int a_2d, uint8_t* out_a, const float* sb,
                                    int64_t rows_b, int b_2d, uint8_t* out_b, int64_t k_blocks,
                                    hipStream_t stream) {
  ExpandParams p{};
  p.src[0] = sa;
  p.src[1] = sb;
  p.dst[0] = reinterpret_cast<uint32_t*>(out_a);
  p.dst[1] = reinterpret_cast<uint32_t*>(out_b);
  p.count[0] = rows_a * k_blocks;
  p.count[1] = rows_b * k_blocks;
  p.kb = k_blocks;
  p.shift[0] = a_2d ? 7 : 0;
  p.shift[1] = b_2d ? 7 : 0;
  const int64_t total = p.count[0] + p.count[1];
  if (total == 0) return TE_OK;
  hipLaunchKernelGGL(block_scale_expand_kernel, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, stream, p);
  return launch_status();
}

}  // namespace temx

using namespace temx;

extern "C" te_status te_fp8_block_scales_to_mx(const float* scale_inv, int64_t rows, int64_t cols, int block_2d,
                                               uint8_t* mx_scale, hipStream_t stream) {
  TE_REQUIRE(rows >= 0 && cols >= 0 && cols % 128 == 0, TE_ERR_SHAPE);
  TE_REQUIRE(block_2d == 0 || block_2d == 1, TE_ERR_VALUE);
  const int64_t kb = cols / 128;
  TE_REQUIRE(rows <= ((int64_t)1 << 40) && kb <= ((int64_t)1 << 20) && (rows * kb + 255) / 256 < ((int64_t)1 << 31),
             TE_ERR_SHAPE);
  if (rows == 0 || kb == 0) return TE_OK;
  TE_REQUIRE(scale_inv != nullptr && mx_scale != nullptr, TE_ERR_NULL);
  TE_REQUIRE(((uintptr_t)scale_inv & 3u) == 0 && ((uintptr_t)mx_scale & 3u) == 0, TE_ERR_ALIGN);
  return launch_block_scale_expand(scale_inv, rows, block_2d, mx_scale, nullptr, 0, 0, nullptr, kb, stream);
}
