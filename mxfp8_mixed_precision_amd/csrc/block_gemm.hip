// Blockwise FP8 GEMM: operands quantized in 1 x 128 blocks (A, and B in the
// 1-D x 1-D form) or 128 x 128 blocks (B in the 1-D x 2-D form), each block
// carried with an FP32 scale inverse.
//
// "Transformer Engine On ROCm and AMDGPU", section "Blockwise FP8 GEMM
// support on ROCm (gfx942 and gfx950)": 1-D x 2-D and 1-D x 1-D block
// scaling, E4M3 / E5M2 inputs (not E5M2 x E5M2), bias and DGELU epilogues;
// on gfx950 the default kernel computes with the scales cast to E8M0, and a
// second kernel uses the FP32 scales themselves.  Both are here:
// Both run the GEMM kernel of gemm_core.h; the FP32 scale rows ride the
// stage copies into LDS like E8M0 scale bytes, and each 128-deep MFMA covers
// one K block.
// * TE_BLOCK_SCALES_E8M0 (modes SM_BE1 / SM_BE2): each lane casts its row's
//   FP32 scale to E8M0 as it reads it and hands the code to the MFMA, which
//   applies it to all four 32-blocks of the 128-block: the MXFP8 arithmetic
//   on the cast scales.
// * TE_BLOCK_SCALES_FP32 (SM_FS1 / SM_FS2): each block's product is computed
//   with unit scales and added to the accumulators times sa * sb.
// No workspace either way.
#include "gemm_core.h"

namespace temx {
namespace {

template <class C, int FA, int FB, int EPI, int OUT, int SM>
te_status launch_fs5(const GemmParams& p, dim3 grid, hipStream_t stream) {
  hipLaunchKernelGGL((mx_gemm_kernel<C, FA, FB, EPI, OUT, SM>), grid, dim3(C::kThreads), 0, stream, p);
  return launch_status();
}

template <class C, int FA, int FB, int EPI, int SM>
te_status launch_fs4(const GemmParams& p, te_dtype out, dim3 grid, hipStream_t stream) {
  return out == TE_BF16 ? launch_fs5<C, FA, FB, EPI, TE_BF16, SM>(p, grid, stream)
                        : launch_fs5<C, FA, FB, EPI, TE_FP32, SM>(p, grid, stream);
}

template <class C, int FA, int FB, int SM>
te_status launch_fs3(const GemmParams& p, te_epilogue epi, te_dtype out, dim3 grid, hipStream_t stream) {
  switch (epi) {
    case TE_EPI_NONE: return launch_fs4<C, FA, FB, TE_EPI_NONE, SM>(p, out, grid, stream);
    case TE_EPI_BIAS: return launch_fs4<C, FA, FB, TE_EPI_BIAS, SM>(p, out, grid, stream);
    case TE_EPI_BIAS_GELU_AUX: return launch_fs4<C, FA, FB, TE_EPI_BIAS_GELU_AUX, SM>(p, out, grid, stream);
    case TE_EPI_DGELU: return launch_fs4<C, FA, FB, TE_EPI_DGELU, SM>(p, out, grid, stream);
    default: return launch_fs5<C, FA, FB, TE_EPI_ACCUMULATE, TE_FP32, SM>(p, grid, stream);  // fp32 D only
  }
}

template <class C, int SM>
te_status launch_fs2(const GemmParams& p, te_dtype fa, te_dtype fb, te_epilogue epi, te_dtype out, dim3 grid,
                     hipStream_t stream) {
  if (fa == TE_E4M3 && fb == TE_E4M3) return launch_fs3<C, TE_E4M3, TE_E4M3, SM>(p, epi, out, grid, stream);
  if (fa == TE_E5M2 && fb == TE_E4M3) return launch_fs3<C, TE_E5M2, TE_E4M3, SM>(p, epi, out, grid, stream);
  return launch_fs3<C, TE_E4M3, TE_E5M2, SM>(p, epi, out, grid, stream);
}

template <class C>
te_status launch_fs(const GemmParams& p, bool e8m0, int b2d, te_dtype fa, te_dtype fb, te_epilogue epi, te_dtype out,
                    dim3 grid, hipStream_t stream) {
  if (e8m0)
    return b2d ? launch_fs2<C, SM_BE2>(p, fa, fb, epi, out, grid, stream)
               : launch_fs2<C, SM_BE1>(p, fa, fb, epi, out, grid, stream);
  return b2d ? launch_fs2<C, SM_FS2>(p, fa, fb, epi, out, grid, stream)
             : launch_fs2<C, SM_FS1>(p, fa, fb, epi, out, grid, stream);
}

}  // namespace
}  // namespace temx

using namespace temx;

extern "C" size_t te_fp8_block_gemm_workspace_size(int64_t, int64_t, int64_t, te_block_scaling) { return 0; }

extern "C" te_status te_fp8_block_gemm(const uint8_t* a, const float* a_scale_inv, te_dtype a_fmt,
                                       const uint8_t* b, const float* b_scale_inv, te_dtype b_fmt, int b_block_2d,
                                       int64_t M, int64_t N, int64_t K, void* d, te_dtype d_dtype,
                                       te_epilogue epi, const uint16_t* bias, uint16_t* aux,
                                       te_block_scaling mode, void* workspace, size_t workspace_bytes,
                                       hipStream_t stream) {
  TE_REQUIRE(mode == TE_BLOCK_SCALES_E8M0 || mode == TE_BLOCK_SCALES_FP32, TE_ERR_VALUE);
  TE_REQUIRE(b_block_2d == 0 || b_block_2d == 1, TE_ERR_VALUE);
  TE_REQUIRE(M >= 0 && N >= 0 && K >= 0, TE_ERR_SHAPE);
  TE_REQUIRE(K % 128 == 0 && M % 16 == 0 && N % 16 == 0, TE_ERR_SHAPE);
  TE_REQUIRE(M <= ((int64_t)1 << 31) - 256 && N <= ((int64_t)1 << 31) - 256 && K <= ((int64_t)1 << 31) - BK,
             TE_ERR_SHAPE);
  const int64_t big_tiles = ((M + 255) / 256) * ((N + 255) / 256);
  TE_REQUIRE(((M + 127) / 128) * ((N + 127) / 128) < ((int64_t)1 << 31), TE_ERR_SHAPE);
  (void)workspace;
  (void)workspace_bytes;
  const uint8_t* sa = reinterpret_cast<const uint8_t*>(a_scale_inv);
  const uint8_t* sb = reinterpret_cast<const uint8_t*>(b_scale_inv);
  // the scale arrays stand in for the E8M0 ones in the common checks (non-NULL, 4-byte aligned when read)
  te_status st = check_common(a, sa, a_fmt, b, sb, b_fmt, d, d_dtype, epi, bias, aux, M > 0 && N > 0, K > 0);
  if (st != TE_OK) return st;
  if (M == 0 || N == 0) return TE_OK;
  GemmParams p{a, sa, b, sb, d, bias, aux, M, N, K, nullptr, 0};
  const bool e8m0 = mode == TE_BLOCK_SCALES_E8M0;
  if (use_small_tile(big_tiles, K))
    return launch_fs<Small>(p, e8m0, b_block_2d, a_fmt, b_fmt, epi, d_dtype,
                            dim3((unsigned)(((M + 127) / 128) * ((N + 127) / 128))), stream);
  return launch_fs<Big>(p, e8m0, b_block_2d, a_fmt, b_fmt, epi, d_dtype, dim3((unsigned)big_tiles), stream);
}
