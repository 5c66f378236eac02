// Blockwise FP8 GEMM: operands quantized in 1 x 128 blocks (A, and B in the
// 1-D x 1-D form) or 128 x 128 blocks (B in the 1-D x 2-D form), each block
// carried with an FP32 scale inverse.
//
// "Transformer Engine On ROCm and AMDGPU", section "Blockwise FP8 GEMM
// support on ROCm (gfx942 and gfx950)": 1-D x 2-D and 1-D x 1-D block
// scaling, E4M3 / E5M2 inputs (not E5M2 x E5M2), bias and DGELU epilogues;
// on gfx950 the default kernel computes with the scales cast to E8M0, and a
// second kernel uses the FP32 scales themselves.  Both are scale modes of
// the GEMM kernel of gemm_core.h, instantiated in block_gemm_e8m0.hip and
// block_gemm_fp32.hip; this file holds the entry point.  The FP32 scale rows
// ride the stage copies into LDS like E8M0 scale bytes, and each 128-deep
// MFMA covers one K block.
// * TE_BLOCK_SCALES_E8M0 (modes SM_BE1 / SM_BE2): each lane casts its row's
//   FP32 scale to E8M0 as it reads it and hands the code to the MFMA, which
//   applies it to all four 32-blocks of the 128-block: the MXFP8 arithmetic
//   on the cast scales.
// * TE_BLOCK_SCALES_FP32 (SM_FS1 / SM_FS2): each block's product is computed
//   with unit scales and added to the accumulators times sa * sb.
// No workspace either way.  The same section lists fp16 output and a beta
// epilogue among the blockwise GEMM's options: D may be fp16, and the
// accumulate epilogue scales the fp32 D it adds to by beta.
#include "gemm_core.h"

using namespace temx;

extern "C" size_t te_fp8_block_gemm_workspace_size(int64_t, int64_t, int64_t, te_block_scaling) { return 0; }

extern "C" te_status te_fp8_block_gemm(const uint8_t* a, const float* a_scale_inv, te_dtype a_fmt,
                                       const uint8_t* b, const float* b_scale_inv, te_dtype b_fmt, int b_block_2d,
                                       int64_t M, int64_t N, int64_t K, void* d, te_dtype d_dtype,
                                       te_epilogue epi, const uint16_t* bias, uint16_t* aux,
                                       te_block_scaling mode, float beta, void* workspace, size_t workspace_bytes,
                                       hipStream_t stream) {
  TE_REQUIRE(mode == TE_BLOCK_SCALES_E8M0 || mode == TE_BLOCK_SCALES_FP32, TE_ERR_VALUE);
  TE_REQUIRE(b_block_2d == 0 || b_block_2d == 1, TE_ERR_VALUE);
  TE_REQUIRE(M >= 0 && N >= 0 && K >= 0, TE_ERR_SHAPE);
  TE_REQUIRE(K % 128 == 0 && M % 16 == 0 && N % 16 == 0, TE_ERR_SHAPE);
  TE_REQUIRE(dense_shape_ok(M, N, K), TE_ERR_SHAPE);
  (void)workspace;
  (void)workspace_bytes;
  const uint8_t* sa = reinterpret_cast<const uint8_t*>(a_scale_inv);
  const uint8_t* sb = reinterpret_cast<const uint8_t*>(b_scale_inv);
  // the scale arrays stand in for the E8M0 ones in the common checks (non-NULL, 4-byte aligned when read)
  te_status st =
      check_common(a, sa, a_fmt, b, sb, b_fmt, d, d_dtype, epi, bias, aux, M > 0 && N > 0, K > 0, /*allow_fp16=*/true);
  if (st != TE_OK) return st;
  if (M == 0 || N == 0) return TE_OK;
  TE_REQUIRE(device_is_gfx950(), TE_ERR_ARCH);
  auto launch = mode == TE_BLOCK_SCALES_E8M0 ? launch_block_gemm_e8m0 : launch_block_gemm_fp32;
  return launch(a, a_scale_inv, b, b_scale_inv, b_block_2d, M, N, K, d, d_dtype, epi, bias, aux, beta, a_fmt, b_fmt,
                stream);
}
