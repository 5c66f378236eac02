// Entry points of the MXFP8, MXFP8-output, per-tensor FP8 and grouped GEMMs (kernels in
// gemm_core.h).
#include "gemm_core.h"

namespace temx {
namespace {

// The persistent 4-wave kernel's grid: one workgroup per CU (a multiple of 8, the XCD count, so each
// workgroup stays on the XCD its tiles are rastered for), or one per tile if there are fewer.
inline dim3 persistent_grid(dim3 tiles) {
  const unsigned cap = (unsigned)(device_cu_count() / 8 * 8);
  return dim3(cap >= 8 && tiles.x > cap ? cap : tiles.x);
}

template <class C, bool GROUPED, int FA, int FB, int EPI, int OUT>
te_status launch5(const GemmParams& p, dim3 grid, hipStream_t stream) {
  if constexpr (std::is_same<C, Big4>::value) {
    static_assert(!GROUPED, "the 4-wave tile serves dense GEMMs");
    hipLaunchKernelGGL((mx_gemm4_kernel<FA, FB, EPI, OUT>), persistent_grid(grid), dim3(C::kThreads), 0, stream, p);
  } else if constexpr (GROUPED) {
    hipLaunchKernelGGL((mx_grouped_gemm_kernel<C, FA, FB, EPI, OUT>), grid, dim3(C::kThreads), 0, stream, p);
  } else {
    hipLaunchKernelGGL((mx_gemm_kernel<C, FA, FB, EPI, OUT>), grid, dim3(C::kThreads), 0, stream, p);
  }
  return launch_status();
}

template <class C, bool GROUPED, int FA, int FB, int EPI>
te_status launch4(const GemmParams& p, te_dtype out, dim3 grid, hipStream_t stream) {
  return out == TE_BF16 ? launch5<C, GROUPED, FA, FB, EPI, TE_BF16>(p, grid, stream)
                        : launch5<C, GROUPED, FA, FB, EPI, TE_FP32>(p, grid, stream);
}

template <class C, int FA, int FB, int EPI>
te_status launch_pt4(const GemmParams& p, te_dtype out, dim3 grid, hipStream_t stream) {
  if constexpr (std::is_same<C, Big4>::value) {
    if (out == TE_BF16)
      hipLaunchKernelGGL((mx_gemm4_kernel<FA, FB, EPI, TE_BF16, SM_PT>), persistent_grid(grid), dim3(C::kThreads), 0,
                         stream, p);
    else
      hipLaunchKernelGGL((mx_gemm4_kernel<FA, FB, EPI, TE_FP32, SM_PT>), persistent_grid(grid), dim3(C::kThreads), 0,
                         stream, p);
  } else {
    if (out == TE_BF16)
      hipLaunchKernelGGL((mx_gemm_kernel<C, FA, FB, EPI, TE_BF16, SM_PT>), grid, dim3(C::kThreads), 0, stream, p);
    else
      hipLaunchKernelGGL((mx_gemm_kernel<C, FA, FB, EPI, TE_FP32, SM_PT>), grid, dim3(C::kThreads), 0, stream, p);
  }
  return launch_status();
}

template <class C, int FA, int FB>
te_status launch_pt3(const GemmParams& p, te_epilogue epi, te_dtype out, dim3 grid, hipStream_t stream) {
  switch (epi) {
    case TE_EPI_NONE: return launch_pt4<C, FA, FB, TE_EPI_NONE>(p, out, grid, stream);
    case TE_EPI_BIAS: return launch_pt4<C, FA, FB, TE_EPI_BIAS>(p, out, grid, stream);
    default: return launch_pt4<C, FA, FB, TE_EPI_BIAS_GELU_AUX>(p, out, grid, stream);
  }
}

template <class C>
te_status launch_pt(const GemmParams& p, te_dtype fa, te_dtype fb, te_epilogue epi, te_dtype out, dim3 grid,
                    hipStream_t stream) {
  if (fa == TE_E4M3 && fb == TE_E4M3) return launch_pt3<C, TE_E4M3, TE_E4M3>(p, epi, out, grid, stream);
  if (fa == TE_E5M2 && fb == TE_E4M3) return launch_pt3<C, TE_E5M2, TE_E4M3>(p, epi, out, grid, stream);
  return launch_pt3<C, TE_E4M3, TE_E5M2>(p, epi, out, grid, stream);
}

template <class C, int FA, int FB, int EPI>
te_status launch_mx4(const GemmParams& p, te_dtype out, dim3 grid, hipStream_t stream) {
  return out == TE_E4M3 ? launch5<C, false, FA, FB, EPI, TE_E4M3>(p, grid, stream)
                        : launch5<C, false, FA, FB, EPI, TE_E5M2>(p, grid, stream);
}

template <class C, bool GROUPED, int FA, int FB>
te_status launch3(const GemmParams& p, te_epilogue epi, te_dtype out, dim3 grid, hipStream_t stream) {
  if (out == TE_E4M3 || out == TE_E5M2) {  // MXFP8 output: dense, forward epilogues (validated)
    if constexpr (GROUPED) {
      return TE_ERR_DTYPE;
    } else {
      switch (epi) {
        case TE_EPI_NONE: return launch_mx4<C, FA, FB, TE_EPI_NONE>(p, out, grid, stream);
        case TE_EPI_BIAS: return launch_mx4<C, FA, FB, TE_EPI_BIAS>(p, out, grid, stream);
        default: return launch_mx4<C, FA, FB, TE_EPI_BIAS_GELU_AUX>(p, out, grid, stream);
      }
    }
  }
  switch (epi) {
    case TE_EPI_NONE: return launch4<C, GROUPED, FA, FB, TE_EPI_NONE>(p, out, grid, stream);
    case TE_EPI_BIAS: return launch4<C, GROUPED, FA, FB, TE_EPI_BIAS>(p, out, grid, stream);
    case TE_EPI_BIAS_GELU_AUX: return launch4<C, GROUPED, FA, FB, TE_EPI_BIAS_GELU_AUX>(p, out, grid, stream);
    case TE_EPI_DGELU: return launch4<C, GROUPED, FA, FB, TE_EPI_DGELU>(p, out, grid, stream);
    default: return launch5<C, GROUPED, FA, FB, TE_EPI_ACCUMULATE, TE_FP32>(p, grid, stream);  // fp32 D only
  }
}

template <class C, bool GROUPED>
te_status launch2(const GemmParams& p, te_dtype fa, te_dtype fb, te_epilogue epi, te_dtype out, dim3 grid,
                  hipStream_t stream) {
  if (fa == TE_E4M3 && fb == TE_E4M3) return launch3<C, GROUPED, TE_E4M3, TE_E4M3>(p, epi, out, grid, stream);
  if (fa == TE_E5M2 && fb == TE_E4M3) return launch3<C, GROUPED, TE_E5M2, TE_E4M3>(p, epi, out, grid, stream);
  return launch3<C, GROUPED, TE_E4M3, TE_E5M2>(p, epi, out, grid, stream);
}

}  // namespace

int device_cu_count() {
  static int cached[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 256;
  if (dev < 0 || dev >= 64) return 256;
  if (cached[dev] == 0) {
    int cu = 0;
    if (hipDeviceGetAttribute(&cu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cu <= 0) cu = 256;
    cached[dev] = cu;
  }
  return cached[dev];
}

}  // namespace temx

using namespace temx;

namespace temx {
namespace {

// MXFP8 GEMM on the big tile: the 4-wave kernel when the workspace takes the
// rearranged scales (and the scale arrays allow 16-byte reads), else the
// 8-wave kernel on the scales as they are.
te_status launch_big_mx(GemmParams p, te_dtype a_fmt, te_dtype b_fmt, te_epilogue epi, te_dtype out, dim3 grid,
                        void* workspace, size_t workspace_bytes, hipStream_t stream) {
  const int64_t M = p.M, N = p.N, K = p.K;
  if (four_wave_mx(M, N, K) && workspace != nullptr && workspace_bytes >= scale_blocks_bytes(M, N, K) &&
      ((uintptr_t)workspace & 255u) == 0 && aligned16(p.a_scale) && aligned16(p.b_scale)) {
    uint8_t* ws = static_cast<uint8_t*>(workspace);
    uint8_t* bs = ws + scale_blocks_b_offset(M, K);
    if (launch_scale_blocks(p.a_scale, M, ws, p.b_scale, N, bs, K, stream) != TE_OK) return TE_ERR_HIP;
    p.a_scale = ws;
    p.b_scale = bs;
    return launch2<Big4, false>(p, a_fmt, b_fmt, epi, out, grid, stream);
  }
  return launch2<Big, false>(p, a_fmt, b_fmt, epi, out, grid, stream);
}

}  // namespace
}  // namespace temx

extern "C" size_t te_mxfp8_gemm_workspace_size(int64_t M, int64_t N, int64_t K) {
  if (M <= 0 || N <= 0 || K <= 0 || K % 128 != 0 || !dense_shape_ok(M, N, K)) return 0;
  return four_wave_mx(M, N, K) ? scale_blocks_bytes(M, N, K) : 0;
}

extern "C" te_status te_mxfp8_gemm(const uint8_t* a, const uint8_t* a_scale, te_dtype a_fmt, const uint8_t* b,
                                   const uint8_t* b_scale, te_dtype b_fmt, int64_t M, int64_t N, int64_t K, void* d,
                                   te_dtype d_dtype, te_epilogue epi, const uint16_t* bias, uint16_t* aux,
                                   void* workspace, size_t workspace_bytes, hipStream_t stream) {
  TE_REQUIRE(M >= 0 && N >= 0 && K >= 0, TE_ERR_SHAPE);
  TE_REQUIRE(K % 128 == 0 && M % 16 == 0 && N % 16 == 0, TE_ERR_SHAPE);
  TE_REQUIRE(dense_shape_ok(M, N, K), TE_ERR_SHAPE);
  te_status st = check_common(a, a_scale, a_fmt, b, b_scale, b_fmt, d, d_dtype, epi, bias, aux, M > 0 && N > 0, K > 0);
  if (st != TE_OK) return st;
  if (M == 0 || N == 0) return TE_OK;
  TE_REQUIRE(device_is_gfx950(), TE_ERR_ARCH);
  GemmParams p{a, a_scale, b, b_scale, d, bias, aux, M, N, K, nullptr, 0};
  const Tile t = pick_tile_dense(M, N, K);
  const dim3 grid = tile_grid(t, M, N);
  if (t == Tile::SmallDeep) return launch2<SmallDeep, false>(p, a_fmt, b_fmt, epi, d_dtype, grid, stream);
  if (t == Tile::Small) return launch2<Small, false>(p, a_fmt, b_fmt, epi, d_dtype, grid, stream);
  if (t == Tile::Big192) return launch2<Big192, false>(p, a_fmt, b_fmt, epi, d_dtype, grid, stream);
  return launch_big_mx(p, a_fmt, b_fmt, epi, d_dtype, grid, workspace, workspace_bytes, stream);
}

extern "C" te_status te_mxfp8_gemm_mxout(const uint8_t* a, const uint8_t* a_scale, te_dtype a_fmt, const uint8_t* b,
                                         const uint8_t* b_scale, te_dtype b_fmt, int64_t M, int64_t N, int64_t K,
                                         uint8_t* d, uint8_t* d_scale, te_dtype d_fmt, te_epilogue epi,
                                         const uint16_t* bias, uint16_t* aux, void* workspace, size_t workspace_bytes,
                                         hipStream_t stream) {
  TE_REQUIRE(epi == TE_EPI_NONE || epi == TE_EPI_BIAS || epi == TE_EPI_BIAS_GELU_AUX, TE_ERR_VALUE);
  TE_REQUIRE(d_fmt == TE_E4M3 || d_fmt == TE_E5M2, TE_ERR_DTYPE);
  TE_REQUIRE(M >= 0 && N >= 0 && K >= 0, TE_ERR_SHAPE);
  TE_REQUIRE(K % 128 == 0 && M % 16 == 0 && N % 32 == 0, TE_ERR_SHAPE);
  TE_REQUIRE(dense_shape_ok(M, N, K), TE_ERR_SHAPE);
  // the common checks with the bf16 D this output stands for
  te_status st = check_common(a, a_scale, a_fmt, b, b_scale, b_fmt, d, TE_BF16, epi, bias, aux, M > 0 && N > 0, K > 0);
  if (st != TE_OK) return st;
  if (M == 0 || N == 0) return TE_OK;
  TE_REQUIRE(d_scale != nullptr, TE_ERR_NULL);
  TE_REQUIRE(device_is_gfx950(), TE_ERR_ARCH);
  GemmParams p{a, a_scale, b, b_scale, d, bias, aux, M, N, K, nullptr, 0, d_scale};
  const Tile t = pick_tile_dense(M, N, K);
  const dim3 grid = tile_grid(t, M, N);
  if (t == Tile::SmallDeep) return launch2<SmallDeep, false>(p, a_fmt, b_fmt, epi, d_fmt, grid, stream);
  if (t == Tile::Small) return launch2<Small, false>(p, a_fmt, b_fmt, epi, d_fmt, grid, stream);
  if (t == Tile::Big192) return launch2<Big192, false>(p, a_fmt, b_fmt, epi, d_fmt, grid, stream);
  return launch_big_mx(p, a_fmt, b_fmt, epi, d_fmt, grid, workspace, workspace_bytes, stream);
}

extern "C" te_status te_fp8_gemm(const uint8_t* a, const float* a_scale_inv, te_dtype a_fmt, const uint8_t* b,
                                 const float* b_scale_inv, te_dtype b_fmt, int64_t M, int64_t N, int64_t K, void* d,
                                 te_dtype d_dtype, te_epilogue epi, const uint16_t* bias, uint16_t* aux,
                                 void* workspace, size_t workspace_bytes, hipStream_t stream) {
  (void)workspace;
  (void)workspace_bytes;
  TE_REQUIRE(epi == TE_EPI_NONE || epi == TE_EPI_BIAS || epi == TE_EPI_BIAS_GELU_AUX, TE_ERR_VALUE);
  TE_REQUIRE(M >= 0 && N >= 0 && K >= 0, TE_ERR_SHAPE);
  TE_REQUIRE(K % 128 == 0 && M % 16 == 0 && N % 16 == 0, TE_ERR_SHAPE);
  TE_REQUIRE(dense_shape_ok(M, N, K), TE_ERR_SHAPE);
  // the scale pointers stand in for the block-scale arrays in the common checks
  te_status st = check_common(a, reinterpret_cast<const uint8_t*>(a_scale_inv), a_fmt, b,
                              reinterpret_cast<const uint8_t*>(b_scale_inv), b_fmt, d, d_dtype, epi, bias, aux,
                              M > 0 && N > 0, K > 0);
  if (st != TE_OK) return st;
  if (M == 0 || N == 0) return TE_OK;
  TE_REQUIRE(a_scale_inv != nullptr && b_scale_inv != nullptr, TE_ERR_NULL);
  TE_REQUIRE(device_is_gfx950(), TE_ERR_ARCH);
  // the block-scale descriptors are never read in per-tensor mode; they point at the data
  GemmParams p{a, a, b, b, d, bias, aux, M, N, K, nullptr, 0, nullptr, a_scale_inv, b_scale_inv};
  const Tile t = pick_tile_dense(M, N, K);
  const dim3 grid = tile_grid(t, M, N);
  if (t == Tile::SmallDeep) return launch_pt<SmallDeep>(p, a_fmt, b_fmt, epi, d_dtype, grid, stream);
  if (t == Tile::Small) return launch_pt<Small>(p, a_fmt, b_fmt, epi, d_dtype, grid, stream);
  if (t == Tile::Big192) return launch_pt<Big192>(p, a_fmt, b_fmt, epi, d_dtype, grid, stream);
  if (four_wave(M, N, K)) return launch_pt<Big4>(p, a_fmt, b_fmt, epi, d_dtype, grid, stream);
  return launch_pt<Big>(p, a_fmt, b_fmt, epi, d_dtype, grid, stream);
}

extern "C" te_status te_mxfp8_grouped_gemm(int32_t num_groups, const int32_t* m_splits, int64_t total_m,
                                           const uint8_t* a, const uint8_t* a_scale, te_dtype a_fmt,
                                           const uint8_t* b, const uint8_t* b_scale, te_dtype b_fmt, int64_t N,
                                           int64_t K, void* d, te_dtype d_dtype, te_epilogue epi,
                                           const uint16_t* bias, uint16_t* aux, void* workspace,
                                           size_t workspace_bytes, hipStream_t stream) {
  (void)workspace;
  (void)workspace_bytes;
  TE_REQUIRE(num_groups >= 1 && num_groups <= kMaxGroups, TE_ERR_SHAPE);
  TE_REQUIRE(total_m >= 0 && N > 0 && K > 0, TE_ERR_SHAPE);
  TE_REQUIRE(K % 128 == 0 && N % 16 == 0, TE_ERR_SHAPE);
  TE_REQUIRE(total_m <= ((int64_t)1 << 31) - 256 && N <= ((int64_t)1 << 31) - 256 && K <= ((int64_t)1 << 23),
             TE_ERR_SHAPE);
  TE_REQUIRE((total_m / 128 + num_groups) * ((N + 127) / 128) < ((int64_t)1 << 31), TE_ERR_SHAPE);
  TE_REQUIRE(m_splits != nullptr, TE_ERR_NULL);
  TE_REQUIRE(((uintptr_t)m_splits & 3u) == 0, TE_ERR_ALIGN);
  te_status st = check_common(a, a_scale, a_fmt, b, b_scale, b_fmt, d, d_dtype, epi, bias, aux, total_m > 0, true);
  if (st != TE_OK) return st;
  if (total_m == 0) return TE_OK;
  TE_REQUIRE(device_is_gfx950(), TE_ERR_ARCH);
  GemmParams p{a, a_scale, b, b_scale, d, bias, aux, total_m, N, K, m_splits, num_groups};
  int grid = device_cu_count();
  grid = grid < 8 ? 8 : (grid / 8) * 8;
  // the splits stay on the device: estimate the big-tile count from the total
  // rows, counting one ragged tail tile per group (32 experts x ~512 rows x
  // 1536 columns: big tiles 172 us, small 222 us)
  const int64_t big_tiles = (total_m / 256 + num_groups) * ((N + 255) / 256);
  if (use_small_tile(big_tiles))
    return launch2<Small, true>(p, a_fmt, b_fmt, epi, d_dtype, dim3((unsigned)(2 * grid)), stream);
  return launch2<Big, true>(p, a_fmt, b_fmt, epi, d_dtype, dim3((unsigned)grid), stream);
}
