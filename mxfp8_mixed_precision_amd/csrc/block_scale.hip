// Blockwise FP8 scales (one FP32 scale inverse per 1 x 128 or 128 x 128
// block) cast to E8M0 and laid out as MXFP8 scales.
//
// "Transformer Engine On ROCm and AMDGPU", section "Blockwise FP8 GEMM
// support on ROCm (gfx942 and gfx950)": on gfx950 the default blockwise GEMM
// casts the incoming FP32 scales to E8M0 and computes with those.  A 128-wide
// block along K spans four 32-wide MX blocks, which all take its scale, so
// with the cast scales a blockwise operand is an MXFP8 operand that every
// MXFP8 kernel accepts.  (The blockwise GEMM makes the same cast inside its
// own kernel, as the scales arrive in LDS.)
//
// The cast of s is the smallest E8M0 value >= s (exact for the recipe's own
// power-of-two scales), saturating at 2^127 (+inf included); s = +-0 and
// positive values up to 2^-127 give 2^-127, the smallest E8M0 value.  NaN
// and negative s give the E8M0 NaN code 255.

#include "temx_device.h"

namespace temx {
namespace {

// One thread per 128-block: rows rows of kb 128-blocks; the scale inverse of
// (row r, block j) is src[(r >> shift) * kb + j] (shift 0: 1-D blocks, 7:
// 128 x 128 blocks).  The output uint8 [rows, 4 kb] is written as one uint32
// (four equal codes) per 128-block, i.e. dst is uint32 [rows, kb].
__global__ __launch_bounds__(256) void block_scale_expand_kernel(const float* __restrict__ src,
                                                                 uint32_t* __restrict__ dst, int64_t count,
                                                                 int64_t kb, int shift) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= count) return;
  const int64_t r = i / kb, j = i - r * kb;
  dst[i] = e8m0_at_least(src[(r >> shift) * kb + j]) * 0x01010101u;
}

}  // namespace
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
  TE_REQUIRE(device_is_gfx950(), TE_ERR_ARCH);
  const int64_t count = rows * kb;
  hipLaunchKernelGGL(block_scale_expand_kernel, dim3((unsigned)((count + 255) / 256)), dim3(256), 0, stream,
                     scale_inv, reinterpret_cast<uint32_t*>(mx_scale), count, kb, block_2d ? 7 : 0);
  return launch_status();
}
