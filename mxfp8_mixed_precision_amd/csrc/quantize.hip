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
      store_nt8(q + c, r);
      if ((threadIdx.x & 3) == 0) s[c >> 2] = (uint8_t)code;
    }
  }
}

// Columnwise (transposed), without an LDS round trip for the input.
//
// A workgroup of 8 waves covers 256 columns, as 4 strips of 64 columns x 2
// row groups: wave w takes strip w % 4 and row group w / 4.  The workgroup
// spans cpw x 256 rows; its chunk c covers rows 256 c .. 256 c + 255, and row
// group r takes rows 128 r .. 128 r + 127 of each chunk, so the 8 waves work
// on one 256 x 256 tile at a time.  At any moment a workgroup thus reads
// 512-byte runs of 256 consecutive rows (measured on MI355X, 8192^2: 36 us,
// against 38-40 us for 128 columns x 4 row groups of 256 consecutive rows
// each; the backward shapes 14336 x 4096 and 4096 x 14336 gain 8-10% too).
// Lane (rq, g) = (lane >> 3,
// lane & 7) loads rows 4rq..4rq+3 of each 32-row block straight into
// registers, 8 columns (16 bytes) each, so every load instruction still
// covers eight whole 128-byte row segments.  The block amax of a column is
// the max over the 8 lanes with the same g (DPP row rotate by 8, a swizzle
// across 16 lanes, a permute across 32).  Each lane then packs the values of
// one column from row pairs, converts them with that column's scale, and
// holds 4 codes (rows 4rq..4rq+3) per column.
//
// Codes go through a wave-private LDS stage of 64 output rows x 128 bytes
// (one 128-row chunk): a lane writes 4 bytes per column at row offset
// (32 (block & 3) + 4 rq) XOR (16 g), which spreads the 64 lanes over the
// banks (2-way at most) and leaves every 16-byte piece whole, so the stage
// drains with 16-byte stores covering whole 128-byte lines.  These stores
// are ordinary (cached) ones: measured on gfx950, streaming stores of this
// scattered line pattern are ~10% slower, while the input loads, read once,
// are streaming.  The
// E8M0 codes of the workgroup's 256 columns collect in LDS and leave after
// one barrier as runs of 8 or 16 bytes per column (cpw 1 or 2).  Staging a
// whole 512-row tile in a workgroup-shared LDS buffer, so that every output
// row is written as one 512-byte run, measured no faster.
constexpr int kColWaves = 8;
constexpr int kColThreads = 64 * kColWaves;
constexpr int kColStrip = 64;          // columns per wave
constexpr int kColStrips = 4;          // column strips per workgroup
constexpr int kColGroups = kColWaves / kColStrips;  // row groups per workgroup
constexpr int kColWgCols = kColStrips * kColStrip;
constexpr int kColChunk = 128;         // rows per staged chunk
constexpr int kColMaxChunks = 2;       // chunks per wave at most
constexpr int kColScaleRun = kColGroups * kColMaxChunks * 4;  // scale codes per column and workgroup, at most

__device__ __forceinline__ uint32_t pk_max_u16(uint32_t a, uint32_t b) {
  return __builtin_bit_cast(uint32_t, __builtin_elementwise_max(__builtin_bit_cast(u16x2, a), __builtin_bit_cast(u16x2, b)));
}

// max over the 8 lanes l, l^8, l^16, ..., l^56 (packed u16 halves)
__device__ __forceinline__ uint32_t max_over_row_quads(uint32_t v, int lane) {
  v = pk_max_u16(v, (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x128, 0xF, 0xF, false));   // row_ror:8 = lane ^ 8
  v = pk_max_u16(v, (uint32_t)__builtin_amdgcn_ds_swizzle((int)v, 0x401F));                // lane ^ 16
  v = pk_max_u16(v, (uint32_t)__builtin_amdgcn_ds_bpermute((lane ^ 32) << 2, (int)v));      // lane ^ 32
  return v;
}

// sum over the 8 lanes l, l^8, l^16, ..., l^56 in a fixed butterfly order
// (a + b == b + a in fp32, so every lane of the group ends with the same bits)
__device__ __forceinline__ float sum_over_row_quads(float v, int lane) {
  v += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x128, 0xF, 0xF, false));   // lane ^ 8
  v += __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(v), 0x401F));                // lane ^ 16
  v += __int_as_float(__builtin_amdgcn_ds_bpermute((lane ^ 32) << 2, __float_as_int(v)));      // lane ^ 32
  return v;
}

template <int FMT>
__device__ __forceinline__ uint32_t cvt4_scaled(uint32_t rows01, uint32_t rows23, float scale) {
  v2s r = {0, 0};
  if constexpr (FMT == TE_E4M3) {
    r = __builtin_amdgcn_cvt_scalef32_pk_fp8_bf16(r, __builtin_bit_cast(v2bf, rows01), scale, false);
    r = __builtin_amdgcn_cvt_scalef32_pk_fp8_bf16(r, __builtin_bit_cast(v2bf, rows23), scale, true);
  } else {
    r = __builtin_amdgcn_cvt_scalef32_pk_bf8_bf16(r, __builtin_bit_cast(v2bf, rows01), scale, false);
    r = __builtin_amdgcn_cvt_scalef32_pk_bf8_bf16(r, __builtin_bit_cast(v2bf, rows23), scale, true);
  }
  return saturate_bytes<FMT>(__builtin_bit_cast(uint32_t, r));
}

// ROW: the same pass also writes the rowwise copy (both directions from one
// read of x).  Lane (rq, g) holds, for each of its 4 rows, 8 consecutive
// columns, so the 4 lanes g = 4h .. 4h+3 (a DPP quad) hold one row's 32-block:
// its amax is a quad max, and each lane encodes and stores its 8 codes.
// These are plain stores: a wave writes 64 of each 128-byte line, the wave of
// the neighbouring strip the other 64, and L2 merges them.
// BGRAD: also the column sums of x in fp32 (the bias gradient when x is an
// output gradient), per workgroup into ws[blockIdx.y][cols]: each lane adds
// its 4 rows per block in block order, the 8 lanes of a column combine in a
// fixed butterfly, then the two row groups in LDS; deterministic.
template <int FMT, bool ROW, bool BGRAD>
__global__ __launch_bounds__(kColThreads) __attribute__((amdgpu_waves_per_eu(4))) void quantize_colwise_kernel(
    const uint16_t* __restrict__ x, uint8_t* __restrict__ qc, uint8_t* __restrict__ sc,
    uint8_t* __restrict__ qr, uint8_t* __restrict__ sr, float* __restrict__ ws,
    int64_t rows, int64_t cols, int cpw) {
  __shared__ __attribute__((aligned(16))) uint8_t stage_all[kColWaves][kColStrip * kColChunk];
  __shared__ uint8_t scodes[kColWgCols * kColScaleRun];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int cs = wave % kColStrips, rg = wave / kColStrips;
  const int rq = lane >> 3, g = lane & 7;
  const int64_t wg_rows = kColGroups * (int64_t)cpw * kColChunk;
  const int64_t R0 = (int64_t)blockIdx.y * wg_rows;
  const int64_t c0 = (int64_t)blockIdx.x * kColWgCols;
  const int64_t c0w = c0 + kColStrip * cs;                   // first column of this wave
  const int64_t gcol = c0w + 8 * g;                           // this lane's 8 columns
  const bool col_ok = gcol < cols;
  // first row of this wave's part of chunk c; the wave's blocks k = 4 c + b
  // (b < 4) run up the rows, so the valid ones are a prefix
  auto chunk_row = [&](int c) { return R0 + (int64_t)c * kColGroups * kColChunk + (int64_t)rg * kColChunk; };
  int nblocks = 0;
  for (int k = 0; k < cpw * 4; ++k) nblocks += (chunk_row(k >> 2) + 32 * (k & 3) + 32 <= rows) ? 1 : 0;
  if (c0w >= cols) nblocks = 0;
  uint8_t* stage = stage_all[wave];
  float csum[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};

  auto load = [&](u32x4 (&v)[4], int k) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
      v[i] = col_ok ? __builtin_nontemporal_load(
                          reinterpret_cast<const u32x4*>(x + (chunk_row(k >> 2) + 32 * (k & 3) + 4 * rq + i) * cols + gcol))
                    : u32x4{0, 0, 0, 0};
  };

  auto process = [&](const u32x4 (&v)[4], int k) {
    if constexpr (ROW) {
      const int64_t row0 = chunk_row(k >> 2) + 32 * (k & 3) + 4 * rq;
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const uint4 xv = {v[u][0], v[u][1], v[u][2], v[u][3]};
        const uint32_t code = e8m0_code_from_amax_bits<FMT>(quad_max(absmax_bits8(xv)));
        const uint2 r = cvt8_scaled<FMT>(xv, e8m0_to_float(code));
        if (col_ok) {
          *reinterpret_cast<uint2*>(qr + (row0 + u) * cols + gcol) = r;
          if ((g & 3) == 0) sr[(row0 + u) * (cols / 32) + gcol / 32] = (uint8_t)code;
        }
      }
    }
    if constexpr (BGRAD) {
#pragma unroll
      for (int u = 0; u < 4; ++u)
#pragma unroll
        for (int d = 0; d < 4; ++d) {
          csum[2 * d] += bf16_bits_to_float(v[u][d] & 0xFFFFu);
          csum[2 * d + 1] += bf16_bits_to_float(v[u][d] >> 16);
        }
    }
    uint32_t m[4];
#pragma unroll
    for (int d = 0; d < 4; ++d) {
      m[d] = pk_max_u16(pk_max_u16(v[0][d] & 0x7FFF7FFFu, v[1][d] & 0x7FFF7FFFu),
                        pk_max_u16(v[2][d] & 0x7FFF7FFFu, v[3][d] & 0x7FFF7FFFu));
      m[d] = max_over_row_quads(m[d], lane);
    }
    const int row_off = (32 * (k & 3) + 4 * rq) ^ (16 * g);
    uint32_t my_code = 0;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int d = j >> 1;
      const uint32_t amax_bits = (j & 1) ? (m[d] >> 16) : (m[d] & 0xFFFFu);
      const uint32_t code = e8m0_code_from_amax_bits<FMT>(amax_bits);
      const float scale = e8m0_to_float(code);
      const uint32_t sel = (j & 1) ? 0x07060302u : 0x05040100u;  // high or low bf16 halves of two rows
      const uint32_t q = cvt4_scaled<FMT>(__builtin_amdgcn_perm(v[1][d], v[0][d], sel),
                                          __builtin_amdgcn_perm(v[3][d], v[2][d], sel), scale);
      *reinterpret_cast<uint32_t*>(&stage[(8 * g + j) * kColChunk + row_off]) = q;
      my_code = rq == j ? code : my_code;
    }
    scodes[(kColStrip * cs + 8 * g + rq) * kColScaleRun + (k >> 2) * kColGroups * 4 + rg * 4 + (k & 3)] =
        (uint8_t)my_code;
    if ((k & 3) == 3 || k == nblocks - 1) {
      // drain the chunk: 64 output rows, 16-byte pieces, 8 lanes per 128-byte segment
      const int valid = 32 * ((k & 3) + 1);
      const int64_t out_row0 = chunk_row(k >> 2);
      __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): this wave's stage writes have landed
      asm volatile("" ::: "memory");
#pragma unroll
      for (int kk = 0; kk < 8; ++kk) {
        const int piece = lane + 64 * kk;
        const int orow = piece >> 3, seg = piece & 7;
        const uint4 val = *reinterpret_cast<const uint4*>(&stage[orow * kColChunk + ((16 * seg) ^ (16 * (orow >> 3)))]);
        if (16 * seg < valid && c0w + orow < cols)
          *reinterpret_cast<uint4*>(qc + (c0w + orow) * rows + out_row0 + 16 * seg) = val;
      }
      asm volatile("" ::: "memory");  // the next chunk's stage writes stay after these reads
    }
  };

  u32x4 va[4], vb[4];
  if (nblocks > 0) load(va, 0);
  for (int k = 0; k < nblocks; k += 2) {
    if (k + 1 < nblocks) load(vb, k + 1);
    process(va, k);
    if (k + 1 < nblocks) {
      if (k + 2 < nblocks) load(va, k + 2);
      process(vb, k + 1);
    }
  }

  __syncthreads();
  // the workgroup's scale codes: column c, blocks R0/32 .. R0/32 + nbw - 1, consecutive threads on consecutive bytes
  const int nbw = (int)max((int64_t)0, min(wg_rows, rows - R0) / 32);
  const int64_t sstride = rows / 32;
  for (int idx = threadIdx.x; idx < kColWgCols * nbw; idx += kColThreads) {
    const int c = idx / nbw, b = idx - c * nbw;
    if (c0 + c < cols) sc[(c0 + c) * sstride + R0 / 32 + b] = scodes[c * kColScaleRun + b];
  }

  if constexpr (BGRAD) {
    __shared__ float group_sums[kColGroups][kColWgCols];
#pragma unroll
    for (int j = 0; j < 8; ++j) csum[j] = sum_over_row_quads(csum[j], lane);
    if (rq == 0) {
#pragma unroll
      for (int j = 0; j < 8; ++j) group_sums[rg][kColStrip * cs + 8 * g + j] = csum[j];
    }
    __syncthreads();
    for (int c = threadIdx.x; c < kColWgCols; c += kColThreads) {
      float t = group_sums[0][c];
#pragma unroll
      for (int r = 1; r < kColGroups; ++r) t += group_sums[r][c];
      if (c0 + c < cols) ws[(int64_t)blockIdx.y * cols + c0 + c] = t;
    }
  }
}

// Both directions in one pass with 128 columns per wave (the rowwise copy's
// stores then cover whole 128-byte lines).  A workgroup of 4 waves covers
// 256 columns as 2 strips x 2 row groups; wave w takes strip w % 2 and row
// group w / 2, and spans cpw chunks of 128 rows per row group, as in the
// colwise kernel.  Lane (rr, cg) = (lane >> 4, lane & 15) loads rows
// 8 rr .. 8 rr + 7 of each 32-row block, columns 8 cg .. 8 cg + 7 (16 bytes):
// one load instruction covers four whole 256-byte row segments.
// * colwise: the amax of a column is a max over the lane's 8 rows, then over
//   the 4 lanes holding the column (lane ^ 16, lane ^ 32); each lane encodes
//   its 8 rows of each of its 8 columns (8 bytes per output row) into a
//   wave-private LDS stage of 128 output rows x 128 bytes (one chunk), 8-byte
//   slots XOR-swizzled by cg, drained with 16-byte stores as in the colwise
//   kernel;
// * rowwise: the 4 lanes of a DPP quad hold one row's 32-column block; each
//   store instruction writes 4 rows x 128 bytes;
// * BGRAD: 8 fp32 column sums per lane in row order, combined over the 4
//   lanes of a column in a fixed order, then over the 2 row groups.
constexpr int kB128Waves = 4;
constexpr int kB128Threads = 64 * kB128Waves;
constexpr int kB128Strip = 128;
constexpr int kB128Strips = 2;
constexpr int kB128Groups = kB128Waves / kB128Strips;
constexpr int kB128WgCols = kB128Strips * kB128Strip;
constexpr int kB128Chunk = 128;
constexpr int kB128MaxChunks = 2;
constexpr int kB128ScaleRun = kB128Groups * kB128MaxChunks * 4;  // codes per column and workgroup, at most

template <int FMT, bool BGRAD>
__global__ __launch_bounds__(kB128Threads) void quantize_both128_kernel(
    const uint16_t* __restrict__ x, uint8_t* __restrict__ qc, uint8_t* __restrict__ sc,
    uint8_t* __restrict__ qr, uint8_t* __restrict__ sr, float* __restrict__ ws,
    int64_t rows, int64_t cols, int cpw) {
  __shared__ __attribute__((aligned(16))) uint8_t stage_all[kB128Waves][kB128Strip * kB128Chunk];
  __shared__ uint8_t scodes[kB128WgCols * kB128ScaleRun];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int cs = wave % kB128Strips, rg = wave / kB128Strips;
  const int rr = lane >> 4, cg = lane & 15;
  const int64_t wg_rows = kB128Groups * (int64_t)cpw * kB128Chunk;
  const int64_t R0 = (int64_t)blockIdx.y * wg_rows;
  const int64_t c0 = (int64_t)blockIdx.x * kB128WgCols;
  const int64_t c0w = c0 + kB128Strip * cs;
  const int64_t gcol = c0w + 8 * cg;
  const bool col_ok = gcol < cols;
  auto chunk_row = [&](int c) { return R0 + (int64_t)c * kB128Groups * kB128Chunk + (int64_t)rg * kB128Chunk; };
  int nblocks = 0;
  for (int k = 0; k < cpw * 4; ++k) nblocks += (chunk_row(k >> 2) + 32 * (k & 3) + 32 <= rows) ? 1 : 0;
  if (c0w >= cols) nblocks = 0;
  uint8_t* stage = stage_all[wave];
  float csum[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};

  auto load = [&](u32x4 (&v)[8], int k) {
#pragma unroll
    for (int i = 0; i < 8; ++i)
      v[i] = col_ok ? __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(
                          x + (chunk_row(k >> 2) + 32 * (k & 3) + 8 * rr + i) * cols + gcol))
                    : u32x4{0, 0, 0, 0};
  };

  auto process = [&](const u32x4 (&v)[8], int k) {
    const int64_t row0 = chunk_row(k >> 2) + 32 * (k & 3) + 8 * rr;
    // rowwise: row i of the lane, its quad's 32-column block
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const uint4 xv = {v[i][0], v[i][1], v[i][2], v[i][3]};
      const uint32_t code = e8m0_code_from_amax_bits<FMT>(quad_max(absmax_bits8(xv)));
      const uint2 r = cvt8_scaled<FMT>(xv, e8m0_to_float(code));
      if (col_ok) {
        *reinterpret_cast<uint2*>(qr + (row0 + i) * cols + gcol) = r;
        if ((cg & 3) == 0) sr[(row0 + i) * (cols / 32) + gcol / 32] = (uint8_t)code;
      }
    }
    if constexpr (BGRAD) {
#pragma unroll
      for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int d = 0; d < 4; ++d) {
          csum[2 * d] += bf16_bits_to_float(v[i][d] & 0xFFFFu);
          csum[2 * d + 1] += bf16_bits_to_float(v[i][d] >> 16);
        }
    }
    // colwise: column amax over the lane's 8 rows, then the 4 lanes of the column
    uint32_t m[4];
#pragma unroll
    for (int d = 0; d < 4; ++d) {
      uint32_t t = v[0][d] & 0x7FFF7FFFu;
#pragma unroll
      for (int i = 1; i < 8; ++i) t = pk_max_u16(t, v[i][d] & 0x7FFF7FFFu);
      t = pk_max_u16(t, (uint32_t)__builtin_amdgcn_ds_swizzle((int)t, 0x401F));               // lane ^ 16
      t = pk_max_u16(t, (uint32_t)__builtin_amdgcn_ds_bpermute((lane ^ 32) << 2, (int)t));    // lane ^ 32
      m[d] = t;
    }
    const int slot = (4 * (k & 3) + rr) ^ cg;  // 8-byte slot of this lane's rows in a 128-byte output row
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int d = j >> 1;
      const uint32_t amax_bits = (j & 1) ? (m[d] >> 16) : (m[d] & 0xFFFFu);
      const uint32_t code = e8m0_code_from_amax_bits<FMT>(amax_bits);
      const float scale = e8m0_to_float(code);
      const uint32_t sel = (j & 1) ? 0x07060302u : 0x05040100u;  // high or low bf16 halves of two rows
      const uint32_t lo = cvt4_scaled<FMT>(__builtin_amdgcn_perm(v[1][d], v[0][d], sel),
                                           __builtin_amdgcn_perm(v[3][d], v[2][d], sel), scale);
      const uint32_t hi = cvt4_scaled<FMT>(__builtin_amdgcn_perm(v[5][d], v[4][d], sel),
                                           __builtin_amdgcn_perm(v[7][d], v[6][d], sel), scale);
      *reinterpret_cast<uint2*>(&stage[(8 * cg + j) * kB128Chunk + 8 * slot]) = make_uint2(lo, hi);
      if ((j >> 1) == rr)
        scodes[(kB128Strip * cs + 8 * cg + j) * kB128ScaleRun + (k >> 2) * kB128Groups * 4 + rg * 4 + (k & 3)] =
            (uint8_t)code;
    }
    if ((k & 3) == 3 || k == nblocks - 1) {
      // drain the chunk: 128 output rows, 16-byte pieces, 8 lanes per 128-byte row
      const int valid = 32 * ((k & 3) + 1);
      const int64_t out_row0 = chunk_row(k >> 2);
      __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): this wave's stage writes have landed
      asm volatile("" ::: "memory");
#pragma unroll
      for (int kk = 0; kk < 16; ++kk) {
        const int piece = lane + 64 * kk;
        const int orow = piece >> 3, seg = piece & 7;
        const int ocg = orow >> 3;  // the cg whose lanes wrote this output row
        // logical 8-byte slots 2 seg, 2 seg + 1 sit at (2 seg) ^ ocg and (2 seg + 1) ^ ocg: one
        // 16-byte pair, its halves swapped when ocg is odd
        const uint4 raw = *reinterpret_cast<const uint4*>(&stage[orow * kB128Chunk + 16 * (seg ^ (ocg >> 1))]);
        const uint4 val = (ocg & 1) ? make_uint4(raw.z, raw.w, raw.x, raw.y) : raw;
        if (16 * seg < valid && c0w + orow < cols)
          *reinterpret_cast<uint4*>(qc + (c0w + orow) * rows + out_row0 + 16 * seg) = val;
      }
      asm volatile("" ::: "memory");  // the next chunk's stage writes stay after these reads
    }
  };

  u32x4 va[8], vb[8];
  if (nblocks > 0) load(va, 0);
  for (int k = 0; k < nblocks; k += 2) {
    if (k + 1 < nblocks) load(vb, k + 1);
    process(va, k);
    if (k + 1 < nblocks) {
      if (k + 2 < nblocks) load(va, k + 2);
      process(vb, k + 1);
    }
  }

  __syncthreads();
  const int nbw = (int)max((int64_t)0, min(wg_rows, rows - R0) / 32);
  const int64_t sstride = rows / 32;
  for (int idx = threadIdx.x; idx < kB128WgCols * nbw; idx += kB128Threads) {
    const int c = idx / nbw, b = idx - c * nbw;
    if (c0 + c < cols) sc[(c0 + c) * sstride + R0 / 32 + b] = scodes[c * kB128ScaleRun + b];
  }

  if constexpr (BGRAD) {
    __shared__ float group_sums[kB128Groups][kB128WgCols];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      float t = csum[j];
      t += __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(t), 0x401F));                // lane ^ 16
      t += __int_as_float(__builtin_amdgcn_ds_bpermute((lane ^ 32) << 2, __float_as_int(t)));     // lane ^ 32
      csum[j] = t;
    }
    if (rr == 0) {
#pragma unroll
      for (int j = 0; j < 8; ++j) group_sums[rg][kB128Strip * cs + 8 * cg + j] = csum[j];
    }
    __syncthreads();
    for (int c = threadIdx.x; c < kB128WgCols; c += kB128Threads) {
      float t = group_sums[0][c];
#pragma unroll
      for (int r = 1; r < kB128Groups; ++r) t += group_sums[r][c];
      if (c0 + c < cols) ws[(int64_t)blockIdx.y * cols + c0 + c] = t;
    }
  }
}

// bgrad[c] = sum over the workgroup row tiles t (in order) of ws[t][c].
template <int OUT>
__global__ __launch_bounds__(256) void bgrad_final_kernel(const float* __restrict__ ws, int tiles, int64_t cols,
                                                          void* __restrict__ out) {
  const int64_t c = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (c >= cols) return;
  // loads issued 8 at a time, added in tile order (the same sums as one at a time)
  float s = 0.f;
  int t = 0;
  for (; t + 8 <= tiles; t += 8) {
    float v[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] = ws[(int64_t)(t + i) * cols + c];
#pragma unroll
    for (int i = 0; i < 8; ++i) s += v[i];
  }
  for (; t < tiles; ++t) s += ws[(int64_t)t * cols + c];
  if constexpr (OUT == TE_FP32)
    static_cast<float*>(out)[c] = s;
  else
    static_cast<uint16_t*>(out)[c] = __builtin_bit_cast(uint16_t, (__bf16)s);
}

// Chunks of 128 rows per colwise wave: two (16-byte scale runs per column)
// when that grid still has 1.5 workgroups per CU, else one.  Measured on
// MI355X: 8192^2 36.0 vs 36.4 us, 14336 x 4096 33.5 vs 35.3 us, 4096 x 14336
// 34.4 vs 35.3 us with two; 4096^2 12.6 vs 17.3 us with one.
int colwise_chunks_per_wave(int64_t rows, int64_t cols) {
  const int64_t col_tiles = (cols + kColWgCols - 1) / kColWgCols;
  const int64_t row_tiles_2 = (rows + kColGroups * 2 * kColChunk - 1) / (kColGroups * 2 * kColChunk);
  return 2 * col_tiles * row_tiles_2 >= 3 * (int64_t)device_cu_count() ? 2 : 1;
}

// The colwise kernel over [rows, cols] (rows, cols > 0); `tiles` receives
// the number of workgroup row tiles (the rows of the bgrad workspace).
template <int FMT, bool ROW, bool BGRAD>
te_status launch_colwise(const uint16_t* x, int64_t rows, int64_t cols, uint8_t* q_row, uint8_t* s_row,
                         uint8_t* q_col, uint8_t* s_col, float* ws, hipStream_t stream, int* tiles) {
  const int cpw = colwise_chunks_per_wave(rows, cols);
  const int64_t rows_per_wg = kColGroups * (int64_t)cpw * kColChunk;
  dim3 grid((unsigned)((cols + kColWgCols - 1) / kColWgCols), (unsigned)((rows + rows_per_wg - 1) / rows_per_wg));
  if (tiles) *tiles = (int)grid.y;
  hipLaunchKernelGGL((quantize_colwise_kernel<FMT, ROW, BGRAD>), grid, dim3(kColThreads), 0, stream, x, q_col, s_col,
                     q_row, s_row, ws, rows, cols, cpw);
  return launch_status();
}

// Fewest rows a colwise workgroup covers (one chunk per wave): the bgrad
// workspace is sized for the largest number of row tiles.
constexpr int64_t kColMinWgRows = (int64_t)kColGroups * kColChunk;

// Both kernels that make the two copies tile the columns and the rows alike,
// so the chunk heuristic and the bgrad workspace size hold for either.
static_assert(kB128WgCols == kColWgCols && kB128Groups == kColGroups && kB128Chunk == kColChunk &&
                  kB128MaxChunks == kColMaxChunks,
              "the fused kernels differ in their workgroup tiles");

// Both directions (and with BGRAD the column sums) from one read of x.  The
// 128-column kernel runs where the grid takes two chunks per wave; smaller
// grids run the colwise kernel with its rowwise copy, whose 8-wave
// workgroups keep more loads in flight per CU.  Measured on MI355X
// (both directions / with column sums, us):
//   8192^2         59.3 / 64.3  ->  54.6 / 59.6
//   4096 x 14336   59.8 / 63.0  ->  53.3 / 57.1
//   14336 x 4096   54.7 / 58.7  ->  50.3 / 55.7
//   2048 x 14336   31.8 / 34.7  ->  31.2 / 34.7   (one chunk per wave: colwise kernel)
//   4096^2         19.1 / 22.9  ->  20.3 / 23.9   (one chunk per wave: colwise kernel)
template <int FMT, bool BGRAD>
te_status launch_both(const uint16_t* x, int64_t rows, int64_t cols, uint8_t* q_row, uint8_t* s_row,
                      uint8_t* q_col, uint8_t* s_col, float* ws, hipStream_t stream, int* tiles) {
  const int cpw = colwise_chunks_per_wave(rows, cols);
  if (cpw < 2) return launch_colwise<FMT, true, BGRAD>(x, rows, cols, q_row, s_row, q_col, s_col, ws, stream, tiles);
  const int64_t rows_per_wg = kB128Groups * (int64_t)cpw * kB128Chunk;
  dim3 grid((unsigned)((cols + kB128WgCols - 1) / kB128WgCols), (unsigned)((rows + rows_per_wg - 1) / rows_per_wg));
  if (tiles) *tiles = (int)grid.y;
  hipLaunchKernelGGL((quantize_both128_kernel<FMT, BGRAD>), grid, dim3(kB128Threads), 0, stream, x, q_col, s_col,
                     q_row, s_row, ws, rows, cols, cpw);
  return launch_status();
}

template <int FMT>
te_status launch_quantize(const uint16_t* x, int64_t rows, int64_t cols, te_qdir dir, uint8_t* q_row,
                          uint8_t* s_row, uint8_t* q_col, uint8_t* s_col, hipStream_t stream) {
  // both directions: one pass, x read once
  if (dir == TE_BOTH) return launch_both<FMT, false>(x, rows, cols, q_row, s_row, q_col, s_col, nullptr, stream,
                                                     nullptr);
  if (dir & TE_ROWWISE) {
    const int64_t nchunks = rows * cols / 8;
    const int64_t per_block = (int64_t)kRowThreads * kRowUnroll;
    const int64_t grid = (nchunks + per_block - 1) / per_block;
    hipLaunchKernelGGL(quantize_rowwise_kernel<FMT>, dim3((unsigned)grid), dim3(kRowThreads), 0, stream,
                       reinterpret_cast<const uint4*>(x), reinterpret_cast<uint2*>(q_row), s_row, nchunks);
    if (launch_status() != TE_OK) return TE_ERR_HIP;
  }
  if (dir & TE_COLWISE) return launch_colwise<FMT, false, false>(x, rows, cols, nullptr, nullptr, q_col, s_col, nullptr,
                                                                stream, nullptr);
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
  TE_REQUIRE(device_is_gfx950(), TE_ERR_ARCH);
  return fmt == TE_E4M3 ? launch_quantize<TE_E4M3>(x, rows, cols, dir, q_row, s_row, q_col, s_col, stream)
                        : launch_quantize<TE_E5M2>(x, rows, cols, dir, q_row, s_row, q_col, s_col, stream);
}

extern "C" size_t te_mxfp8_quantize_bgrad_workspace_size(int64_t rows, int64_t cols) {
  if (rows <= 0 || cols <= 0) return 0;
  const int64_t tiles = (rows + kColMinWgRows - 1) / kColMinWgRows;
  return (size_t)(tiles * cols) * sizeof(float);
}

extern "C" te_status te_mxfp8_quantize_bgrad(const uint16_t* x, int64_t rows, int64_t cols, te_dtype fmt,
                                             uint8_t* q_row, uint8_t* s_row, uint8_t* q_col, uint8_t* s_col,
                                             void* bgrad, te_dtype bgrad_dtype, void* workspace,
                                             size_t workspace_bytes, hipStream_t stream) {
  TE_REQUIRE(is_fp8(fmt), TE_ERR_DTYPE);
  TE_REQUIRE(bgrad_dtype == TE_FP32 || bgrad_dtype == TE_BF16, TE_ERR_DTYPE);
  TE_REQUIRE(rows >= 0 && cols >= 0, TE_ERR_SHAPE);
  TE_REQUIRE(rows <= (int64_t)1 << 31 && cols <= (int64_t)1 << 31, TE_ERR_SHAPE);
  TE_REQUIRE(rows % 32 == 0 && cols % 32 == 0, TE_ERR_SHAPE);
  if (cols == 0) return TE_OK;
  TE_REQUIRE(bgrad != nullptr, TE_ERR_NULL);
  TE_REQUIRE(((uintptr_t)bgrad & (bgrad_dtype == TE_FP32 ? 3u : 1u)) == 0, TE_ERR_ALIGN);
  if (rows > 0) {
    TE_REQUIRE(x && q_row && s_row && q_col && s_col && workspace, TE_ERR_NULL);
    TE_REQUIRE(aligned16(x) && aligned16(q_row) && aligned16(q_col), TE_ERR_ALIGN);
    TE_REQUIRE(((uintptr_t)workspace & 3u) == 0, TE_ERR_ALIGN);
    TE_REQUIRE(workspace_bytes >= te_mxfp8_quantize_bgrad_workspace_size(rows, cols), TE_ERR_WORKSPACE);
  }
  TE_REQUIRE(device_is_gfx950(), TE_ERR_ARCH);
  int tiles = 0;
  float* ws = static_cast<float*>(workspace);
  if (rows > 0) {
    const te_status st =
        fmt == TE_E4M3
            ? launch_both<TE_E4M3, true>(x, rows, cols, q_row, s_row, q_col, s_col, ws, stream, &tiles)
            : launch_both<TE_E5M2, true>(x, rows, cols, q_row, s_row, q_col, s_col, ws, stream, &tiles);
    if (st != TE_OK) return st;
  }
  const dim3 grid((unsigned)((cols + 255) / 256));
  if (bgrad_dtype == TE_FP32)
    hipLaunchKernelGGL(bgrad_final_kernel<TE_FP32>, grid, dim3(256), 0, stream, ws, tiles, cols, bgrad);
  else
    hipLaunchKernelGGL(bgrad_final_kernel<TE_BF16>, grid, dim3(256), 0, stream, ws, tiles, cols, bgrad);
  return launch_status();
}
