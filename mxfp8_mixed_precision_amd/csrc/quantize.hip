// MXFP8 1-D block quantization of bf16 tensors for gfx950.
//
// Method: "Transformer Engine On ROCm and AMDGPU", "MXFP8 support on ROCm
// (gfx95x only)" (the MXFP8 recipe) and "Blockwise FP8 GEMM support" (E8M0
// power-of-two scales); E4M3 / E5M2 per "Workflow: NVIDIA TransformerEngine
// FP8 Training Quickstart", Step 4.  Block size 32, scale code
// max(biased_exp(amax) - emax, 0), saturating round-to-nearest-even (OCP MX).
//
// Both kernels are HBM-bound (2 bytes read, 1 + 1/32 bytes written per
// element).  The element encode uses the gfx950 scaled convert
// v_cvt_scalef32_pk_{fp8,bf8}_bf16, which divides a bf16 pair by a power of
// two and rounds to nearest even; it returns the NaN (E4M3) or Inf (E5M2)
// code past the largest finite value, which a byte-wise fix-up turns into
// the saturated code.
#include "temx_device.h"

namespace temx {
namespace {

constexpr int kRowThreads = 256;
constexpr int kRowUnroll = 4;

// Rowwise: the tensor is a flat run of 32-blocks (cols % 32 == 0 keeps every
// block inside one row, and block b's scale lives at s[b]).  A lane owns a
// 16-byte chunk (8 bf16); lanes 4q..4q+3 of a wave own one block and reduce
// its amax with two quad DPP moves.
template <int FMT>
__global__ __launch_bounds__(kRowThreads) void quantize_rowwise_kernel(
    const uint4* __restrict__ x, uint2* __restrict__ q, uint8_t* __restrict__ s, int64_t nchunks) {
  const int64_t base = (int64_t)blockIdx.x * (kRowThreads * kRowUnroll) + threadIdx.x;
  uint4 v[kRowUnroll];
#pragma unroll
  for (int u = 0; u < kRowUnroll; ++u) {
    const int64_t c = base + (int64_t)u * kRowThreads;
    v[u] = c < nchunks ? load_nt16(x + c) : make_uint4(0, 0, 0, 0);
  }
#pragma unroll
  for (int u = 0; u < kRowUnroll; ++u) {
    const int64_t c = base + (int64_t)u * kRowThreads;
    const uint32_t amax_bits = quad_max(absmax_bits8(v[u]));
    const uint32_t code = e8m0_code_from_amax_bits<FMT>(amax_bits);
    const uint2 r = cvt8_scaled<FMT>(v[u], e8m0_to_float(code));
    if (c < nchunks) {
      q[c] = r;
      if ((threadIdx.x & 3) == 0) s[c >> 2] = (uint8_t)code;
    }
  }
}

// Columnwise (transposed): a 128-row x 64-column bf16 tile is staged through
// LDS with coalesced 16-byte loads; wave w then encodes rows 32w..32w+31 of
// the tile (one block) and lane l owns column l, so each lane writes the 32
// codes of its block contiguously into row c of the transposed output.
constexpr int kColTileR = 128;
constexpr int kColTileC = 64;
constexpr int kColPitch = kColTileC + 8;  // bf16 elements; 144-byte rows keep 16-byte stores aligned

template <int FMT>
__global__ __launch_bounds__(256) void quantize_colwise_kernel(
    const uint16_t* __restrict__ x, uint8_t* __restrict__ qc, uint8_t* __restrict__ sc,
    int64_t rows, int64_t cols) {
  __shared__ __attribute__((aligned(16))) uint16_t tile[kColTileR * kColPitch];
  const int64_t r0 = (int64_t)blockIdx.y * kColTileR;
  const int64_t c0 = (int64_t)blockIdx.x * kColTileC;
  // 128 rows x 8 chunks of 16 bytes; 256 threads x 4
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int idx = threadIdx.x + 256 * i;
    const int r = idx >> 3, ch = idx & 7;
    const int64_t gr = r0 + r, gc = c0 + ch * 8;
    uint4 v = make_uint4(0, 0, 0, 0);
    if (gr < rows && gc < cols) v = load_nt16(x + gr * cols + gc);
    *reinterpret_cast<uint4*>(&tile[r * kColPitch + ch * 8]) = v;
  }
  __syncthreads();
  const int w = threadIdx.x >> 6, l = threadIdx.x & 63;
  const int64_t gc = c0 + l;
  const int64_t gr = r0 + 32 * w;
  if (gr >= rows || gc >= cols) return;
  uint4 v[4];
  uint32_t* vw = reinterpret_cast<uint32_t*>(v);
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const uint32_t lo = tile[(32 * w + 2 * i) * kColPitch + l];
    const uint32_t hi = tile[(32 * w + 2 * i + 1) * kColPitch + l];
    vw[i] = lo | (hi << 16);
  }
  const uint32_t amax_bits = max(max(absmax_bits8(v[0]), absmax_bits8(v[1])), max(absmax_bits8(v[2]), absmax_bits8(v[3])));
  const uint32_t code = e8m0_code_from_amax_bits<FMT>(amax_bits);
  const float scale = e8m0_to_float(code);
  const uint2 a = cvt8_scaled<FMT>(v[0], scale), b = cvt8_scaled<FMT>(v[1], scale);
  const uint2 c = cvt8_scaled<FMT>(v[2], scale), d = cvt8_scaled<FMT>(v[3], scale);
  uint4* out = reinterpret_cast<uint4*>(qc + gc * rows + gr);
  out[0] = make_uint4(a.x, a.y, b.x, b.y);
  out[1] = make_uint4(c.x, c.y, d.x, d.y);
  sc[gc * (rows / 32) + gr / 32] = (uint8_t)code;
}

template <int FMT>
te_status launch_quantize(const uint16_t* x, int64_t rows, int64_t cols, te_qdir dir, uint8_t* q_row,
                          uint8_t* s_row, uint8_t* q_col, uint8_t* s_col, hipStream_t stream) {
  if (dir & TE_ROWWISE) {
    const int64_t nchunks = rows * cols / 8;
    const int64_t per_block = (int64_t)kRowThreads * kRowUnroll;
    const int64_t grid = (nchunks + per_block - 1) / per_block;
    hipLaunchKernelGGL(quantize_rowwise_kernel<FMT>, dim3((unsigned)grid), dim3(kRowThreads), 0, stream,
                       reinterpret_cast<const uint4*>(x), reinterpret_cast<uint2*>(q_row), s_row, nchunks);
    if (launch_status() != TE_OK) return TE_ERR_HIP;
  }
  if (dir & TE_COLWISE) {
    dim3 grid((unsigned)((cols + kColTileC - 1) / kColTileC), (unsigned)((rows + kColTileR - 1) / kColTileR));
    hipLaunchKernelGGL(quantize_colwise_kernel<FMT>, grid, dim3(256), 0, stream, x, q_col, s_col, rows, cols);
    if (launch_status() != TE_OK) return TE_ERR_HIP;
  }
  return TE_OK;
}

}  // namespace
}  // namespace temx

using namespace temx;

extern "C" te_status te_mxfp8_quantize(const uint16_t* x, int64_t rows, int64_t cols, te_dtype fmt, te_qdir dir,
                                       uint8_t* q_row, uint8_t* s_row, uint8_t* q_col, uint8_t* s_col,
                                       hipStream_t stream) {
  TE_REQUIRE(dir == TE_ROWWISE || dir == TE_COLWISE || dir == TE_BOTH, TE_ERR_VALUE);
  TE_REQUIRE(is_fp8(fmt), TE_ERR_DTYPE);
  TE_REQUIRE(rows >= 0 && cols >= 0, TE_ERR_SHAPE);
  TE_REQUIRE(rows <= (int64_t)1 << 31 && cols <= (int64_t)1 << 31, TE_ERR_SHAPE);
  const bool row = dir & TE_ROWWISE, col = dir & TE_COLWISE;
  TE_REQUIRE(!row || cols % 32 == 0, TE_ERR_SHAPE);
  TE_REQUIRE(!col || (rows % 32 == 0 && cols % 8 == 0), TE_ERR_SHAPE);
  TE_REQUIRE(row == (q_row != nullptr) && row == (s_row != nullptr), TE_ERR_NULL);
  TE_REQUIRE(col == (q_col != nullptr) && col == (s_col != nullptr), TE_ERR_NULL);
  if (rows == 0 || cols == 0) return TE_OK;
  TE_REQUIRE(x != nullptr, TE_ERR_NULL);
  TE_REQUIRE(aligned16(x), TE_ERR_ALIGN);
  TE_REQUIRE(!row || aligned16(q_row), TE_ERR_ALIGN);
  TE_REQUIRE(!col || aligned16(q_col), TE_ERR_ALIGN);
  return fmt == TE_E4M3 ? launch_quantize<TE_E4M3>(x, rows, cols, dir, q_row, s_row, q_col, s_col, stream)
                        : launch_quantize<TE_E5M2>(x, rows, cols, dir, q_row, s_row, q_col, s_col, stream);
}
