// Blockwise FP8 GEMM kernels, FP32 block scales applied in fp32
// (te_fp8_block_gemm with TE_BLOCK_SCALES_FP32).
#include "block_gemm_impl.h"

namespace temx {

te_status launch_block_gemm_fp32(const uint8_t* a, const float* sa, const uint8_t* b, const float* sb, int b2d,
                                 int64_t M, int64_t N, int64_t K, void* d, te_dtype d_dtype, te_epilogue epi,
                                 const uint16_t* bias, uint16_t* aux, float beta, te_dtype fa, te_dtype fb,
                                 hipStream_t stream) {
  return launch_block_modes<SM_FS1, SM_FS2>(a, sa, b, sb, b2d, M, N, K, d, d_dtype, epi, bias, aux, beta, fa, fb,
                                           stream);
}

}  // namespace temx
