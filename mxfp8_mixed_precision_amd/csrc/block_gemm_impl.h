// Launch templates of the blockwise FP8 GEMM, included by block_gemm_e8m0.hip
// and block_gemm_fp32.hip (one scale mode each, so the two compile in
// parallel); the entry point is in block_gemm.hip.
#pragma once

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
  if (out == TE_BF16) return launch_fs5<C, FA, FB, EPI, TE_BF16, SM>(p, grid, stream);
  if (out == TE_FP16) return launch_fs5<C, FA, FB, EPI, TE_FP16, SM>(p, grid, stream);
  return launch_fs5<C, FA, FB, EPI, TE_FP32, SM>(p, grid, stream);
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

// The blockwise GEMM in one scale mode: SM1 for 1-D B blocks, SM2 for 2-D.
template <int SM1, int SM2>
te_status launch_block_modes(const uint8_t* a, const float* sa, const uint8_t* b, const float* sb, int b2d,
                             int64_t M, int64_t N, int64_t K, void* d, te_dtype d_dtype, te_epilogue epi,
                             const uint16_t* bias, uint16_t* aux, float beta, te_dtype fa, te_dtype fb,
                             hipStream_t stream) {
  GemmParams p{a, reinterpret_cast<const uint8_t*>(sa), b, reinterpret_cast<const uint8_t*>(sb), d, bias, aux,
               M, N, K, nullptr, 0};
  p.beta = beta;
  const Tile t = pick_tile(M, N, K);
  const dim3 grid = tile_grid(t, M, N);
  if (t == Tile::SmallDeep)
    return b2d ? launch_fs2<SmallDeep, SM2>(p, fa, fb, epi, d_dtype, grid, stream)
               : launch_fs2<SmallDeep, SM1>(p, fa, fb, epi, d_dtype, grid, stream);
  if (t == Tile::Small)
    return b2d ? launch_fs2<Small, SM2>(p, fa, fb, epi, d_dtype, grid, stream)
               : launch_fs2<Small, SM1>(p, fa, fb, epi, d_dtype, grid, stream);
  return b2d ? launch_fs2<Big, SM2>(p, fa, fb, epi, d_dtype, grid, stream)
             : launch_fs2<Big, SM1>(p, fa, fb, epi, d_dtype, grid, stream);
}

}  // namespace
}  // namespace temx
