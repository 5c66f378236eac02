// Blockwise FP8 quantization of bf16 tensors for gfx950: 1 x 128 blocks
// along rows (activations, gradients) or 128 x 128 blocks (weights), one
// FP32 scale inverse per block.
//
// "Transformer Engine On ROCm and AMDGPU", section "Blockwise FP8 GEMM
// support on ROCm (gfx942 and gfx950)": on gfx950 the blockwise recipe makes
// its scales powers of two (the setting that also makes the GEMM cast them
// to E8M0), so the scale inverse of a block with amax a > 0 is the smallest
// power of two p with a / p <= the format's largest value (no element
// saturates), and p = 1 for an all-zero block.  Codes are the saturating
// round-to-nearest-even encodes of x / p.
//
// Both kernels are HBM-bound: 2 bytes read and 1 + 4/128 (1-D) or
// 1 + 4/16384 (2-D) bytes written per element.
#include "temx_device.h"

namespace temx {
namespace {

// 2^e for the block with the given |x| bit pattern maximum (bf16, non-NaN).
// With amax = mant 2^ex (mant in [0.5, 1)) and the format maximum 1.75 2^emax,
// amax / max = (mant / 1.75) 2^(ex - emax) with mant / 1.75 in [0.29, 0.57),
// so the smallest power of two above it is 2^(ex - emax - 1) when
// mant <= 0.875 and 2^(ex - emax) otherwise.  e lies in [-148, 120].
template <int FMT>
__device__ __forceinline__ int block_scale_exp(uint32_t amax_bits) {
  if (amax_bits == 0) return 0;
  const float a = bf16_bits_to_float(amax_bits);
  const int ex = __builtin_amdgcn_frexp_expf(a);
  const float mant = __builtin_amdgcn_frexp_mantf(a);
  return ex - FmtTraits<FMT>::emax - (mant <= 0.875f ? 1 : 0);
}

// Four bf16 pairs times 2^k (k > 0), exactly: the values are small enough
// that the products are normal and keep their 8 significant bits.
__device__ __forceinline__ uint4 scale_up_bf16x8(uint4 v, int k) {
  uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float lo = __builtin_amdgcn_ldexpf(__uint_as_float(w[i] << 16), k);
    const float hi = __builtin_amdgcn_ldexpf(__uint_as_float(w[i] & 0xFFFF0000u), k);
    w[i] = (__float_as_uint(lo) >> 16) | (__float_as_uint(hi) & 0xFFFF0000u);
  }
  return make_uint4(w[0], w[1], w[2], w[3]);
}

// Codes of 8 values of a block with scale inverse 2^e.  The scaled convert
// takes E8M0-range scales (2^-127 and up); a block whose scale is smaller
// (amax below 2^-118 or so) has its values multiplied by 2^(-127 - e) first.
template <int FMT>
__device__ __forceinline__ uint2 encode_block8(uint4 v, int e) {
  if (e < -127) return cvt8_scaled<FMT>(scale_up_bf16x8(v, -127 - e), __builtin_amdgcn_ldexpf(1.0f, -127));
  return cvt8_scaled<FMT>(v, __builtin_amdgcn_ldexpf(1.0f, e));
}

// 1-D: the tensor is a flat run of 128-blocks (cols % 128 == 0).  A lane
// owns a 16-byte chunk (8 bf16); the 16 lanes of a DPP row own one block and
// reduce its amax with quad moves and two row rotations.
constexpr int k1dThreads = 256;
constexpr int k1dUnroll = 4;

template <int FMT>
__global__ __launch_bounds__(k1dThreads) void block_quantize_1d_kernel(const uint4* __restrict__ x,
                                                                       uint2* __restrict__ q,
                                                                       float* __restrict__ s, int64_t nchunks) {
  const int64_t base = (int64_t)blockIdx.x * (k1dThreads * k1dUnroll) + threadIdx.x;
  uint4 v[k1dUnroll];
#pragma unroll
  for (int u = 0; u < k1dUnroll; ++u) {
    const int64_t c = base + (int64_t)u * k1dThreads;
    v[u] = c < nchunks ? load_nt16(x + c) : make_uint4(0, 0, 0, 0);
  }
#pragma unroll
  for (int u = 0; u < k1dUnroll; ++u) {
    const int64_t c = base + (int64_t)u * k1dThreads;
    uint32_t m = quad_max(absmax_bits8(v[u]));
    m = max(m, (uint32_t)__builtin_amdgcn_mov_dpp((int)m, 0x124, 0xF, 0xF, false));  // row_ror:4
    m = max(m, (uint32_t)__builtin_amdgcn_mov_dpp((int)m, 0x128, 0xF, 0xF, false));  // row_ror:8
    const int e = block_scale_exp<FMT>(m);
    const uint2 r = encode_block8<FMT>(v[u], e);
    if (c < nchunks) {
      store_nt8(q + c, r);
      if ((threadIdx.x & 15) == 0) s[c >> 4] = __builtin_amdgcn_ldexpf(1.0f, e);
    }
  }
}

// 2-D: one workgroup per 128 x 128 block.  Lane t of the 256 holds chunk
// t % 16 of rows t / 16 + 16 i, i = 0..7 (each wave reads 4 whole 256-byte
// row segments per load); the block amax is a wave reduction and then a max
// over the 4 waves through LDS.  Rows past the end are neither read nor
// written.
constexpr int k2dThreads = 256;

template <int FMT>
__global__ __launch_bounds__(k2dThreads) void block_quantize_2d_kernel(const uint16_t* __restrict__ x,
                                                                       uint8_t* __restrict__ q,
                                                                       float* __restrict__ s, int64_t rows,
                                                                       int64_t cols) {
  __shared__ uint32_t wave_max[k2dThreads / 64];
  const int64_t kb = cols / 128;
  const int64_t br = blockIdx.x / kb, bc = blockIdx.x - br * kb;
  const int t = threadIdx.x, lane = t & 63;
  const int64_t r0 = br * 128 + t / 16;
  const int64_t col = bc * 128 + (t % 16) * 8;
  uint4 v[8];
  uint32_t m = 0;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int64_t r = r0 + 16 * i;
    v[i] = r < rows ? load_nt16(x + r * cols + col) : make_uint4(0, 0, 0, 0);
    m = max(m, absmax_bits8(v[i]));
  }
  m = quad_max(m);
  m = max(m, (uint32_t)__builtin_amdgcn_mov_dpp((int)m, 0x124, 0xF, 0xF, false));  // row_ror:4
  m = max(m, (uint32_t)__builtin_amdgcn_mov_dpp((int)m, 0x128, 0xF, 0xF, false));  // row_ror:8
  m = max(m, (uint32_t)__builtin_amdgcn_ds_swizzle((int)m, 0x401F));               // lane ^ 16
  m = max(m, (uint32_t)__builtin_amdgcn_ds_bpermute((lane ^ 32) << 2, (int)m));    // lane ^ 32
  if (lane == 0) wave_max[t / 64] = m;
  __syncthreads();
  m = max(max(wave_max[0], wave_max[1]), max(wave_max[2], wave_max[3]));
  const int e = block_scale_exp<FMT>(m);
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int64_t r = r0 + 16 * i;
    const uint2 c = encode_block8<FMT>(v[i], e);
    if (r < rows) store_nt8(q + r * cols + col, c);
  }
  if (t == 0) s[blockIdx.x] = __builtin_amdgcn_ldexpf(1.0f, e);
}

template <int FMT>
te_status launch_block_quantize(const uint16_t* x, int64_t rows, int64_t cols, int block_2d, uint8_t* q,
                                float* s, hipStream_t stream) {
  if (block_2d) {
    const int64_t blocks = ((rows + 127) / 128) * (cols / 128);
    hipLaunchKernelGGL(block_quantize_2d_kernel<FMT>, dim3((unsigned)blocks), dim3(k2dThreads), 0, stream, x, q, s,
                       rows, cols);
  } else {
    const int64_t nchunks = rows * cols / 8;
    const int64_t per_block = (int64_t)k1dThreads * k1dUnroll;
    hipLaunchKernelGGL(block_quantize_1d_kernel<FMT>, dim3((unsigned)((nchunks + per_block - 1) / per_block)),
                       dim3(k1dThreads), 0, stream, reinterpret_cast<const uint4*>(x), reinterpret_cast<uint2*>(q),
                       s, nchunks);
  }
  return launch_status();
}

}  // namespace
}  // namespace temx

using namespace temx;

extern "C" te_status te_fp8_block_quantize(const uint16_t* x, int64_t rows, int64_t cols, te_dtype fmt, int block_2d,
                                           uint8_t* q, float* scale_inv, hipStream_t stream) {
  TE_REQUIRE(is_fp8(fmt), TE_ERR_DTYPE);
  TE_REQUIRE(block_2d == 0 || block_2d == 1, TE_ERR_VALUE);
  TE_REQUIRE(rows >= 0 && cols >= 0 && cols % 128 == 0, TE_ERR_SHAPE);
  // grid sizes: 1-D ceil(rows * cols / 8192) workgroups, 2-D one per block
  TE_REQUIRE(rows <= ((int64_t)1 << 40) && cols <= ((int64_t)1 << 31) &&
                 (rows / 8192 + 1) * cols < ((int64_t)1 << 31) && ((rows + 127) / 128) * (cols / 128) < ((int64_t)1 << 31),
             TE_ERR_SHAPE);
  if (rows == 0 || cols == 0) return TE_OK;
  TE_REQUIRE(x != nullptr && q != nullptr && scale_inv != nullptr, TE_ERR_NULL);
  TE_REQUIRE(aligned16(x) && aligned16(q), TE_ERR_ALIGN);
  TE_REQUIRE(((uintptr_t)scale_inv & 3u) == 0, TE_ERR_ALIGN);
  TE_REQUIRE(device_is_gfx950(), TE_ERR_ARCH);
  return fmt == TE_E4M3 ? launch_block_quantize<TE_E4M3>(x, rows, cols, block_2d, q, scale_inv, stream)
                        : launch_block_quantize<TE_E5M2>(x, rows, cols, block_2d, q, scale_inv, stream);
}
