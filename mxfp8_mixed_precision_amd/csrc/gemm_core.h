// The GEMM kernels of the library ("TN": A [M, K], B [N, K], D = A . B^T) for
// gfx950: MXFP8, per-tensor FP8 and blockwise FP8 operands (template scaling
// modes, see SM_* below), bias / GELU(tanh) / GELU-aux / dgelu / accumulate
// epilogues and an MXFP8-output epilogue, dense and grouped.  Entry points:
// gemm.hip (MXFP8, per-tensor, grouped) and block_gemm*.hip (blockwise).
//
// Method: "HipKittens MXFP8 GEMM Support" (ROCm/TransformerEngine PR #566):
// an MXFP8 GEMM with BIAS and GELU AUX epilogues; review threads: 1-D MXFP8
// scaling, K % 128 == 0, M % 16 == 0, N % 16 == 0, "TN" operands.  GELU is
// the tanh approximation ("Getting Started", TE JAX quickstart).  The grouped
// form is the single-launch grouped GEMM of "Transformer Engine On ROCm and
// AMDGPU" ("Grouped GEMM using CK_Tile"); the blockwise modes follow its
// section "Blockwise FP8 GEMM support on ROCm (gfx942 and gfx950)".
//
// Design for CDNA4:
// * v_mfma_scale_f32_16x16x128_f8f6f4 consumes the fp8 codes and the E8M0
//   block scales directly.  Its operand layout (lane l = 16 g + r holds row r,
//   bytes 0-15 = K 16g..16g+15 and bytes 16-31 = K 64+16g..; the scale byte
//   of K-block kb comes from lane r + 16 kb) means a lane loads two 16-byte
//   chunks of one row and supplies the scale of block g of that row.
// * The MFMA's A operand is a B-tile row (n) and its B operand an A-tile row
//   (m), so each lane ends with 4 consecutive output columns of one row: the
//   epilogue stores 8 bytes (bf16) per lane straight from registers.
// * 256 x 256 workgroup tile, 8 waves in 4 x 2 (two per SIMD), 64 x 128 per
//   wave (4 x 8 MFMA tiles = 128 fp32 accumulators per lane), K step 128;
//   a 256 x 192 tile (8 waves of 64 x 96) where that fills the CUs the
//   256 x 256 grid leaves idle; a 128 x 128 tile (4 waves of 64 x 64) for
//   grids the big tile cannot fill, with 2 or 4 LDS stages (see Cfg); and for
//   long-K grids the 4-wave 256 x 256 tile (Big4, mainloop4: one wave per
//   SIMD, 128 x 128 per wave, 256 accumulators in AGPRs), persistent over its
//   tiles.
// * A, B and their scale tiles are copied global -> LDS with direct-to-LDS
//   buffer loads (buffer_load_dwordx4 / _dword ... lds) into a ring of
//   stages, issued by one wave per SIMD.
// * Workgroup -> tile mapping is XCD-aware: workgroups are dealt round-robin
//   to the 8 XCDs, so each XCD is given a contiguous run of tiles (grouped in
//   bands of 4 row-tiles) and its L2 sees the reuse.
// * Ragged M / N tails: each tile's copies go through buffer resources that
//   cover only its valid rows, so rows past the end read as zeros; stores are
//   masked.  Only the 4-wave MXFP8 path takes a workspace: (M + N) K / 32
//   bytes, the operands' scales rearranged by scale_blocks_kernel.
#pragma once

#include "temx_device.h"

namespace temx {
namespace {

constexpr int BK = 128;

// How the operands are scaled (a template parameter of the kernels):
//   SM_MX   MXFP8: E8M0 scale bytes [rows, K/32], applied by the MFMA itself.
//   SM_PT   per-tensor: no block scales; the MFMA scales are 2^0 and the
//           accumulators are multiplied by a_scale_inv * b_scale_inv at the end.
//   SM_FS1  blockwise FP8 with FP32 scale inverses, one per 1 x 128 block
//           ([rows, K/128] floats) for both operands: each 128-deep MFMA is
//           one K block, computed with unit scales and added to the
//           accumulators times sa[m, kb] * sb[n, kb].
//   SM_FS2  as SM_FS1, but B has one scale per 128 x 128 block
//           ([ceil(N/128), K/128] floats).
//   SM_BE1, SM_BE2  blockwise FP8 as SM_FS1 / SM_FS2, with each FP32 scale
//           cast to E8M0 (the smallest power of two >= s) as it is read from
//           LDS and handed to the MFMA as the scale of all four 32-blocks of
//           its 128-block: the MXFP8 arithmetic on the cast scales.
// A [rows, K/128] float array has the row stride of a [rows, K/32] byte
// array and holds block kt of a row at byte 4 kt, where the E8M0 bytes of
// step kt sit: the stage copies move either kind of scale unchanged, and in
// LDS each tile row has 4 scale bytes per stage (four E8M0 codes, or one float).
constexpr int SM_MX = 0, SM_PT = 1, SM_FS1 = 2, SM_FS2 = 3, SM_BE1 = 4, SM_BE2 = 5;
constexpr bool fp32_scales(int sm) { return sm == SM_FS1 || sm == SM_FS2; }
constexpr bool block_scales(int sm) { return sm == SM_FS1 || sm == SM_FS2 || sm == SM_BE1 || sm == SM_BE2; }
constexpr bool b_2d(int sm) { return sm == SM_FS2 || sm == SM_BE2; }

// Workgroup tile configurations.  A BM x BN tile is computed by NWM x NWN
// waves, each a (BM / NWM) x (BN / NWN) block of FRM x FRN MFMA tiles of
// 16 x 16; the last NCOPY waves issue the stage copies.  One stage in LDS is
// A data [BM][128], B data [BN][128], and (SB = 1) A scales [BM][4], B scales
// [BN][4]; NSTAGE stages form a ring.
//   Big:   256 x 256, 8 waves of 64 x 128 (two per SIMD, 128 accumulators),
//          waves 4-7 copy; scales in 4-step blocks; 144 KB of LDS, one
//          workgroup per CU.  A copy instruction holds up its SIMD for
//          ~70-90 clocks whatever its size, so one 16-byte scale copy per
//          row and 4 steps replaces four 4-byte ones (measured on MI355X,
//          bit-identical results: 8192^3 460 -> 444 us, 4096 x 4096 x 14336
//          199 -> 191 us, the 32-expert grouped GEMM 170 -> 160 us).  The
//          blockwise modes' FP32 scales ([rows, K/128], 4 bytes per row and
//          step) travel in the same 16-byte blocks.
//   Small: 128 x 128, 4 waves of 64 x 64 (64 accumulators), all four copy;
//          66 KB of LDS, two workgroups per CU.  For grids the big tile
//          cannot fill (few or ragged row tiles).
//   SmallDeep: the small tile with 4 stages (132 KB of LDS, one workgroup
//          per CU), for grids of at most one small tile per CU and long K.
//          A 128 x 128 x 128 step computes for ~0.25 us, far less than the
//          latency of its copies from L2 / MALL; three stages in flight
//          cover it where one does not (measured on MI355X: 4096 x 1024 x
//          4096 33.8 -> 28.3 us, 2048 x 2048 x 8192 55.3 -> 45.2 us; with
//          K = 1024 the longer prologue costs a few percent).
template <int BM_, int BN_, int NWM_, int NWN_, int NCOPY_, int NSTAGE_ = 2, int SB_ = 1>
struct Cfg {
  static constexpr int BM = BM_, BN = BN_, NWM = NWM_, NWN = NWN_, NW = NWM * NWN, kThreads = 64 * NW;
  static constexpr int NCOPY = NCOPY_, NSTAGE = NSTAGE_;
  static constexpr int WTM = BM / NWM, WTN = BN / NWN;
  static constexpr int FRM = WTM / 16, FRN = WTN / 16;
  static constexpr int kAData = BM * BK, kBData = BN * BK, kAScale = BM * 4, kBScale = BN * 4;
  static constexpr int kOffBData = kAData;
  static constexpr int kOffAScale = kAData + kBData;
  static constexpr int kOffBScale = kOffAScale + kAScale;
  // SB = 1: each stage holds its step's scales (4 bytes per row).  SB = 4:
  // the scales of 4 steps (16 bytes per row: A rows, then B rows) sit in a
  // separate pair of buffers after the stage ring, one copy per 64 rows and
  // 4 steps instead of per step.
  static constexpr int SB = SB_;
  static constexpr int kStage = SB == 1 ? kOffBScale + kBScale : kAData + kBData;
  static constexpr int kScaleBuf = (BM + BN) * 16;
  static constexpr int kOffScaleBuf = NSTAGE * kStage;
  static constexpr int kLds = NSTAGE * kStage + (SB == 1 ? 0 : 2 * kScaleBuf);
  static_assert(SB == 1 || (SB == 4 && NSTAGE == 2 && BM % 64 == 0 && BN % 64 == 0 && (BM + BN) / 64 <= 2 * NCOPY),
                "scale blocks: at most two 64-row slices per copier wave");
  // SB = 1: scale slices (64 rows of one operand) per copier wave; every
  // copier issues the same number of copies per stage
  static constexpr int kScaleSlicesPerCopier = 2 * (BM / 64) / NCOPY;
  static_assert(SB == 4 || (BM == BN && 2 * (BM / 64) % NCOPY == 0), "per-step scale slices split evenly");
  static_assert(NCOPY % 2 == 0 && (BM / 8) % NCOPY == 0 && (BN / 8) % NCOPY == 0 && (BM / 64) <= NCOPY,
                "copy slices per copier wave");
};
using Big = Cfg<256, 256, 4, 2, 4, 2, 4>;
// 256 x 192 (8 waves of 64 x 96): for grids whose 256 x 256 tiles leave CUs
// idle and whose 256 x 192 tiles fill them without a second round (the
// decoder's QKV, 4096 x 3072: 192 tiles of 256 x 256, 256 of 256 x 192).
using Big192 = Cfg<256, 192, 4, 2, 4, 2, 4>;
using Small = Cfg<128, 128, 2, 2, 4>;
using SmallDeep = Cfg<128, 128, 2, 2, 4, 4>;

// The 4-wave big tile (mainloop4): 256 x 256, one wave per SIMD in 2 x 2,
// each 128 x 128 (8 x 8 MFMA tiles, 256 fp32 accumulators held in AGPRs).
// LDS: two 64-KB stages (A codes [256][128], then B codes), then two scale
// buffers of 4 K steps each (16 E8M0 bytes per tile row: A rows, then B
// rows), 144 KB in all.  For K % 1024 == 0: the loop runs 8 steps a turn.
struct Big4 {
  static constexpr int BM = 256, BN = 256, NWM = 2, NWN = 2, NW = 4, kThreads = 256;
  static constexpr int WTM = 128, WTN = 128, FRM = 8, FRN = 8;
  static constexpr int kHalf = BM * 128;              // A codes of a stage; B codes follow
  static constexpr int kStage = 2 * kHalf;
  static constexpr int kScaleSteps = 4;
  static constexpr int kScaleRow = 4 * kScaleSteps;   // bytes per tile row and scale block
  static constexpr int kScaleBuf = (BM + BN) * kScaleRow;
  static constexpr int kOffScale = 2 * kStage;
  static constexpr int kLds = kOffScale + 2 * kScaleBuf;
  static constexpr int kKAlign = 1024;                // K must be a multiple of this
};
static_assert(Big4::kLds == 144 * 1024, "the 4-wave tile's LDS");

constexpr int kGroupM = 4;      // row-tile band of the raster order
constexpr int kMaxGroups = 1024;

// LDS data tile of one operand and stage: [BM rows][128 bytes] (the step's
// 128 K bytes of each row).  The eight 16-byte chunks of row r are permuted
// by chunk ^ swz(r).  A fragment read has lane 16 g + r fetch logical chunks
// g and g + 4 of row r; with swz(r) = (r >> 1) & 7 these ds_read_b128 run
// without bank conflicts on gfx950 (measured: 4.2 clocks per wave
// instruction, the same as a linear 1-KB read; unswizzled 128-byte rows take
// 14.5).  Chunk g + 4 is at chunk g's address XOR 64.
__device__ __forceinline__ int swz(int row) { return (row >> 1) & 7; }

template <int F> struct MfmaFmt;  // cbsz / blgp operand format codes
template <> struct MfmaFmt<TE_E4M3> { static constexpr int v = 0; };
template <> struct MfmaFmt<TE_E5M2> { static constexpr int v = 1; };

// An operand tile as two buffer resources: rows [row0, row0 + rows) of the
// data [*, K] and of the scales [*, K/32].  Reads past the valid rows (ragged
// M / N / expert tails) return zeros from the buffer range check.
typedef int i32x4 __attribute__((ext_vector_type(4)));
struct Operand {
  i32x4 data;
  i32x4 scale;
};

constexpr int kRsrcWord3 = 0x00020000;  // raw byte buffer, 32-bit data format (gfx9 descriptor word 3)

// The descriptor must live in SGPRs; its inputs are uniform over the wave
// (tile coordinates), which readfirstlane states for the compiler.
__device__ __forceinline__ i32x4 make_rsrc(const void* base, int64_t bytes) {
  const uint64_t a = reinterpret_cast<uint64_t>(base);
  return i32x4{__builtin_amdgcn_readfirstlane((int)(uint32_t)a),
               __builtin_amdgcn_readfirstlane((int)((uint32_t)(a >> 32) & 0xFFFFu)),
               __builtin_amdgcn_readfirstlane((int)bytes), kRsrcWord3};
}

__device__ __forceinline__ Operand make_operand(const uint8_t* data, const uint8_t* scale, int64_t row0,
                                                int64_t rows, int64_t K, int64_t tile_rows) {
  rows = rows < 0 ? 0 : (rows > tile_rows ? tile_rows : rows);
  return Operand{make_rsrc(data + row0 * K, rows * K), make_rsrc(scale + row0 * (K / 32), rows * (K / 32))};
}

// B of SM_FS2: one scale row (K/128 floats = K/32 bytes) per 128 data rows;
// row0 is a multiple of 128.
__device__ __forceinline__ Operand make_operand_2d(const uint8_t* data, const uint8_t* scale, int64_t row0,
                                                   int64_t rows, int64_t K, int64_t tile_rows) {
  rows = rows < 0 ? 0 : (rows > tile_rows ? tile_rows : rows);
  return Operand{make_rsrc(data + row0 * K, rows * K),
                 make_rsrc(scale + (row0 / 128) * (K / 32), ((rows + 127) / 128) * (K / 32))};
}

// Direct-to-LDS buffer loads (buffer_load_dword{,x4} ... lds): lane l's
// bytes land at LDS address m0 + size * l.  They are issued from inline asm
// so that the compiler, which cannot tell the stage being filled from the
// stage being read, does not wait for them before every LDS read; the K loop
// orders them itself (s_waitcnt vmcnt(0) + barrier before a stage is read).
// m0 is saved and restored around the copy (the LDS base is read at issue).
__device__ __forceinline__ void lds_dma16(const i32x4& rsrc, uint32_t lds_addr, int voff, int soff) {
  int saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %1\n\t"
      "buffer_load_dwordx4 %2, %3, %4 offen lds\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "s"(lds_addr), "v"(voff), "s"(rsrc), "s"(soff)
      : "memory");
}

__device__ __forceinline__ void lds_dma4(const i32x4& rsrc, uint32_t lds_addr, int voff, int soff) {
  int saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %1\n\t"
      "buffer_load_dword %2, %3, %4 offen lds\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "s"(lds_addr), "v"(voff), "s"(rsrc), "s"(soff)
      : "memory");
}

// Per-lane byte offsets of the tile copies.  A copy instruction fills one
// 1-KB slice: rows 8 q .. 8 q + 7, lane l landing at LDS byte 16 l, i.e. row
// 8 q + l/8, physical chunk l % 8, which holds logical chunk
// (l % 8) ^ swz(8 q + l/8) = (l % 8) ^ (l / 16) ^ (4 if q is odd).  Each
// instruction reads 8 whole 128-byte lines.  The BM/8 slices of an operand
// tile are dealt to the NCOPY copier waves as q = c + NCOPY i; with NCOPY
// even, q has copier c's parity, so one per-lane offset plus the uniform
// 8 NCOPY i K + 128 kt serves every copy.  Scale slices are rows
// 64 s .. 64 s + 63 of the BM x 4-byte scale tile; copier c < BM/64 copies
// scale slice c of both operands.
struct CopyOffsets {
  int data;
  int scale;  // lane l's row of a 64-row scale slice: l * (K/32)
};

__device__ __forceinline__ CopyOffsets copy_offsets(int64_t K, int c, int lane) {
  const int chunk = (lane & 7) ^ (lane >> 4) ^ ((c & 1) << 2);
  CopyOffsets o;
  o.data = (int)((8 * c + (lane >> 3)) * K) + chunk * 16;
  o.scale = (int)(lane * (K / 32));
  return o;
}

template <class C, int SM = SM_MX>
__device__ __forceinline__ void load_stage(uint32_t stage, const Operand& A, const Operand& B,
                                           const CopyOffsets& off, int64_t K, int kt, int c) {
  constexpr int kA = C::BM / 8 / C::NCOPY, kB = C::BN / 8 / C::NCOPY;  // slices per copier
#pragma unroll
  for (int i = 0; i < (kA > kB ? kA : kB); ++i) {
    const int q = c + C::NCOPY * i;
    const int so = (int)(8 * C::NCOPY * i * K) + kt * BK;
    if (i < kA) lds_dma16(A.data, stage + q * 1024, off.data, so);
    if (i < kB) lds_dma16(B.data, stage + C::kOffBData + q * 1024, off.data, so);
  }
  if constexpr (SM != SM_PT && C::SB == 1) {
#pragma unroll
    for (int i = 0; i < C::kScaleSlicesPerCopier; ++i) {
      const int q = c + C::NCOPY * i, s64 = q >> 1;  // slice q: operand q & 1, rows 64 s64 .. 64 s64 + 63
      const int slice_off = (int)(64 * s64 * (K / 32)) + kt * 4;
      if (q & 1) {
        if constexpr (b_2d(SM))  // the 64 rows lie in 128-row block s64 / 2: one scale row for all lanes
          lds_dma4(B.scale, stage + C::kOffBScale + s64 * 256, 0, (int)((s64 >> 1) * (K / 32)) + kt * 4);
        else
          lds_dma4(B.scale, stage + C::kOffBScale + s64 * 256, off.scale, slice_off);
      } else {
        lds_dma4(A.scale, stage + C::kOffAScale + s64 * 256, off.scale, slice_off);
      }
    }
  }
}

// SB = 4: the 16 scale bytes of steps 4 blk .. 4 blk + 3 of each tile row
// (A rows 0 .. BM-1, then B rows) into scale buffer sbuf; 64-row slice q of
// the 2 BM / 64 is copied by copier q % NCOPY, lane l landing at row 64 s + l.
// With 2-D B blocks (b_2d) a B slice's 64 rows all take their 128-row block
// row's scales.
template <class C, int SM>
__device__ __forceinline__ void load_scale_block(uint32_t sbuf, const Operand& A, const Operand& B,
                                                 const CopyOffsets& off, int64_t K, int blk, int c) {
  constexpr int kSa = C::BM / 64, kSb = C::BN / 64;  // slices of A, then of B
#pragma unroll
  for (int i = 0; i < (kSa + kSb + C::NCOPY - 1) / C::NCOPY; ++i) {
    const int q = c + C::NCOPY * i;
    if (q >= kSa + kSb) break;
    const int s64 = q < kSa ? q : q - kSa;
    const int soff = (int)(64 * s64 * (K / 32)) + 16 * blk;
    if (q < kSa) {
      lds_dma16(A.scale, sbuf + s64 * 1024, off.scale, soff);
    } else if constexpr (b_2d(SM)) {
      lds_dma16(B.scale, sbuf + C::BM * 16 + s64 * 1024, 0, (int)((s64 >> 1) * (K / 32)) + 16 * blk);
    } else {
      lds_dma16(B.scale, sbuf + C::BM * 16 + s64 * 1024, off.scale, soff);
    }
  }
}

struct Frag {
  v8i v;
  int s;
};

// Per-lane LDS read offsets of a wave, computed once.  Fragment j of a
// wave's 128 rows is 16 j rows further (1 KB of data, 64 B of scales), which
// the reads take as immediate offsets.  The empty asm statement keeps each
// offset a single opaque VGPR so that the compiler does not re-associate it
// into per-fragment address registers.
struct ReadOffsets {
  int a_data, a_data2, b_data, b_data2, a_scale, b_scale;
};

// With FP32 scales, a_scale is the float of row r (fragment j: + 64 bytes)
// and b_scale the four floats of columns 4 g .. 4 g + 3 (SM_FS1; fragment i:
// + 64 bytes) or the one float of the wave's 128-row block of B (SM_FS2:
// a wave's columns never straddle a 128 boundary).  With E8M0-cast blockwise
// scales a_scale is the float of row r, whose code serves every lane g, and
// b_scale likewise (SM_BE1) or the wave's one block-row float (SM_BE2).
template <class LY, int SM = SM_MX>
__device__ __forceinline__ ReadOffsets read_offsets(int wm, int wn, int lane) {  // LY: a Cfg
  const int g = lane >> 4, r = lane & 15;
  const int lane_off = r * BK + ((g ^ swz(r)) << 4);
  ReadOffsets o;
  o.a_data = wm * LY::WTM * BK + lane_off;
  o.a_data2 = o.a_data ^ 64;
  o.b_data = LY::kOffBData + wn * LY::WTN * BK + lane_off;
  o.b_data2 = o.b_data ^ 64;
  if constexpr (LY::SB == 4 && block_scales(SM)) {  // blockwise scales in 4-step blocks: 16 bytes per row
    static_assert(128 % LY::WTN == 0, "a wave's columns stay inside one 128-row block of B");
    o.a_scale = (wm * LY::WTM + r) * 16;
    o.b_scale = LY::BM * 16 + (wn * LY::WTN + ((SM == SM_FS1) ? 4 * g : (SM == SM_BE1) ? r : 0)) * 16;
  } else if constexpr (fp32_scales(SM)) {
    static_assert(128 % LY::WTN == 0, "a wave's columns stay inside one 128-row block of B");
    o.a_scale = LY::kOffAScale + (wm * LY::WTM + r) * 4;
    o.b_scale = LY::kOffBScale + (wn * LY::WTN + (SM == SM_FS1 ? 4 * g : 0)) * 4;
  } else if constexpr (block_scales(SM)) {
    static_assert(128 % LY::WTN == 0, "a wave's columns stay inside one 128-row block of B");
    o.a_scale = LY::kOffAScale + (wm * LY::WTM + r) * 4;
    o.b_scale = LY::kOffBScale + (wn * LY::WTN + (SM == SM_BE1 ? r : 0)) * 4;
  } else if constexpr (LY::SB == 4) {  // MXFP8: offsets inside a scale buffer; + 4 (kt % 4) per step
    o.a_scale = (wm * LY::WTM + r) * 16 + g;
    o.b_scale = LY::BM * 16 + (wn * LY::WTN + r) * 16 + g;
  } else {
    o.a_scale = LY::kOffAScale + (wm * LY::WTM + r) * 4 + g;
    o.b_scale = LY::kOffBScale + (wn * LY::WTN + r) * 4 + g;
  }
  asm volatile("" : "+v"(o.a_data), "+v"(o.a_data2), "+v"(o.b_data), "+v"(o.b_data2), "+v"(o.a_scale),
               "+v"(o.b_scale));
  return o;
}

// Fragment j: two 16-byte chunks (K 16g.. and 64 + 16g.. of the step) of row
// 16 j + r of the wave's rows, and the E8M0 byte of block g of that row,
// read on its own (ds_read_u8; the four lanes of a row share one dword, a
// broadcast).  No ALU work depends on the scale read, so its wait lands at the
// MFMA that uses it (measured: 2-12% faster across the GEMM shapes than
// shifting the byte out of the row's scale word).  Rows 16 j further are 2 KB
// further (an immediate offset).
// Scale kinds of a fragment read: the E8M0 byte of block g, 2^0, or the
// E8M0 cast of the row's FP32 block scale.
constexpr int kScaleByte = 0, kScaleUnit = 1, kScaleCast = 2;

template <int SK = kScaleByte, int SSTRIDE = 64>
__device__ __forceinline__ Frag read_frag(const uint8_t* stage, int data_off, int data_off2, int scale_off, int j,
                                          const uint8_t* sstage = nullptr) {
  const uint4 lo = *reinterpret_cast<const uint4*>(stage + data_off + j * 16 * BK);
  const uint4 hi = *reinterpret_cast<const uint4*>(stage + data_off2 + j * 16 * BK);
  Frag f;
  f.v = v8i{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
  if constexpr (SK == kScaleUnit) f.s = 127;
  else if constexpr (SK == kScaleCast)
    f.s = (int)e8m0_at_least(*reinterpret_cast<const float*>((SSTRIDE == 64 ? stage : sstage) + scale_off + j * SSTRIDE));
  else f.s = (int)(SSTRIDE == 64 ? stage : sstage)[scale_off + j * SSTRIDE];
  return f;
}

template <class LY, int FA, int FB, int SM = SM_MX>
__device__ __forceinline__ void compute(const uint8_t* stage, v4f (&acc)[LY::FRN][LY::FRM], const ReadOffsets& ro,
                                        const uint8_t* sstage = nullptr) {
  constexpr int SK = SM == SM_MX ? kScaleByte : (SM == SM_BE1 || SM == SM_BE2) ? kScaleCast : kScaleUnit;
  constexpr int SST = LY::SB == 4 ? 256 : 64;  // scale bytes between fragments (16 rows)
  const uint8_t* sbase = LY::SB == 4 ? sstage : stage;
  Frag bop[LY::FRM];
#pragma unroll
  for (int j = 0; j < LY::FRM; ++j) bop[j] = read_frag<SK, SST>(stage, ro.a_data, ro.a_data2, ro.a_scale, j, sstage);
  if constexpr (fp32_scales(SM)) {
    // one K block per step: P = the block's unit-scale product, then
    // acc += (sa[m] * sb[n]) * P with one rounding (fma)
    float sa[LY::FRM];
#pragma unroll
    for (int j = 0; j < LY::FRM; ++j) sa[j] = *reinterpret_cast<const float*>(sbase + ro.a_scale + j * SST);
    float sab[LY::FRM];
    if constexpr (SM == SM_FS2) {
      const float sb = *reinterpret_cast<const float*>(sbase + ro.b_scale);
#pragma unroll
      for (int j = 0; j < LY::FRM; ++j) sab[j] = sa[j] * sb;
    }
    // The products of fragment i are added one fragment later, so the FRM MFMAs of fragment i + 1 issue
    // between an MFMA and the FMAs that read its result.  With the FMAs right after their MFMA the
    // compiler filled the gap with wait states once the register assignment left it no independent
    // work (measured on MI355X, 8192^3 with 1-D x 2-D FP32 scales: 543 us that way, 488 us this way).
    // Each accumulator still takes its K blocks' products in K order.
    v4f t[2][LY::FRM];
    float4 sb4[2] = {make_float4(0.f, 0.f, 0.f, 0.f), make_float4(0.f, 0.f, 0.f, 0.f)};
    auto add = [&](int i) {
      const int h = i & 1;
#pragma unroll
      for (int j = 0; j < LY::FRM; ++j) {
        if constexpr (SM == SM_FS2) {
#pragma unroll
          for (int e = 0; e < 4; ++e) acc[i][j][e] = __builtin_fmaf(sab[j], t[h][j][e], acc[i][j][e]);
        } else {
          acc[i][j][0] = __builtin_fmaf(sa[j] * sb4[h].x, t[h][j][0], acc[i][j][0]);
          acc[i][j][1] = __builtin_fmaf(sa[j] * sb4[h].y, t[h][j][1], acc[i][j][1]);
          acc[i][j][2] = __builtin_fmaf(sa[j] * sb4[h].z, t[h][j][2], acc[i][j][2]);
          acc[i][j][3] = __builtin_fmaf(sa[j] * sb4[h].w, t[h][j][3], acc[i][j][3]);
        }
      }
    };
#pragma unroll
    for (int i = 0; i < LY::FRN; ++i) {
      const int h = i & 1;
      const Frag aop = read_frag<kScaleUnit>(stage, ro.b_data, ro.b_data2, 0, i);
      if constexpr (SM == SM_FS1 && LY::SB == 1) {
        sb4[h] = *reinterpret_cast<const float4*>(stage + ro.b_scale + i * 64);
      } else if constexpr (SM == SM_FS1) {  // the four rows' floats are 16 bytes apart
        const float* f = reinterpret_cast<const float*>(sbase + ro.b_scale + i * SST);
        sb4[h] = make_float4(f[0], f[4], f[8], f[12]);
      }
#pragma unroll
      for (int j = 0; j < LY::FRM; ++j)
        t[h][j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(aop.v, bop[j].v, v4f{0.f, 0.f, 0.f, 0.f},
                                                                   MfmaFmt<FB>::v, MfmaFmt<FA>::v, 0, 127, 0, 127);
      if (i > 0) add(i - 1);
    }
    add(LY::FRN - 1);
    return;
  }
  int sb_code = 0;  // SM_BE2: one E8M0 code for all of the wave's columns
  if constexpr (SM == SM_BE2) sb_code = (int)e8m0_at_least(*reinterpret_cast<const float*>(sbase + ro.b_scale));
#pragma unroll
  for (int i = 0; i < LY::FRN; ++i) {
    Frag aop;
    if constexpr (SM == SM_BE2) {
      aop = read_frag<kScaleUnit>(stage, ro.b_data, ro.b_data2, 0, i);
      aop.s = sb_code;
    } else {
      aop = read_frag<SK, SST>(stage, ro.b_data, ro.b_data2, ro.b_scale, i, sstage);
    }
#pragma unroll
    for (int j = 0; j < LY::FRM; ++j)
      acc[i][j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(aop.v, bop[j].v, acc[i][j], MfmaFmt<FB>::v,
                                                                   MfmaFmt<FA>::v, 0, aop.s, 0, bop[j].s);
  }
}

// s_waitcnt vmcnt(N) lgkmcnt(0) expcnt(0) (gfx9 encoding: vmcnt bits 3:0 and 15:14).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14));
}

// K loop over a ring of NSTAGE stages: the copies of steps kt+1 ..
// kt+NSTAGE-1 are in flight while step kt computes.  Stage kt is read only
// after each copier has waited until no more than the later stages' copies
// are outstanding (vmcnt counts a wave's copies, which complete in issue
// order) and a barrier; a stage is refilled only after the barrier that
// follows its last read.  With two stages this is plain double buffering.
//
// Only the last NCOPY waves issue the copies.  A direct-to-LDS buffer load
// holds up the wave that issues it for ~70-90 clocks (measured on gfx950,
// whether the data is in L2 or not), so a wave issuing many of them stalls
// for much of a step.  In the big tile the copiers are waves 4-7, one per
// SIMD, and the other wave of each SIMD keeps the MFMA pipe busy meanwhile
// (measured: 8192^3 GEMM ~10% faster than with all 8 waves copying).
template <class LY, int FA, int FB, int SM = SM_MX>
__device__ __forceinline__ void mainloop(uint8_t* lds, v4f (&acc)[LY::FRN][LY::FRM], const Operand& A,
                                         const Operand& B, int64_t K, int wave, int lane) {
  const int wm = wave / LY::NWN, wn = wave % LY::NWN;
#pragma unroll
  for (int i = 0; i < LY::FRN; ++i)
#pragma unroll
    for (int j = 0; j < LY::FRM; ++j) acc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};
  const int kt_n = (int)(K / BK);
  if (kt_n == 0) return;
  const int c = wave - (LY::NW - LY::NCOPY);
  const bool copier = c >= 0;
  const CopyOffsets off = copy_offsets(K, copier ? c : 0, lane);
  const ReadOffsets ro = read_offsets<LY, SM>(wm, wn, lane);
  const uint32_t lds_addr = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) uint8_t*)lds;
  constexpr int S = LY::NSTAGE;
  static_assert(S >= 2 && S <= 4, "the waits below cover up to two later stages in flight");
  // copies per copier wave and stage (the same for every copier)
  constexpr int kPerStage = (LY::BM + LY::BN) / 8 / LY::NCOPY + (SM == SM_PT || LY::SB == 4 ? 0 : LY::kScaleSlicesPerCopier);
  constexpr bool kBlk = LY::SB == 4 && SM != SM_PT;
  if (copier) {
#pragma unroll
    for (int s = 0; s < S - 1; ++s)
      if (s < kt_n) load_stage<LY, SM>(lds_addr + s * LY::kStage, A, B, off, K, s, c);
    if constexpr (kBlk) load_scale_block<LY, SM>(lds_addr + LY::kOffScaleBuf, A, B, off, K, 0, c);
  }
  for (int kt = 0; kt < kt_n; ++kt) {
    // stage kt has landed once at most `ahead` later stages' copies are outstanding
    const int ahead = min(S - 2, kt_n - 1 - kt);
    if (S > 2 && ahead >= 2) wait_vmcnt<2 * kPerStage>();
    else if (S > 2 && ahead == 1) wait_vmcnt<kPerStage>();
    else __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (copier && kt + S - 1 < kt_n)
      load_stage<LY, SM>(lds_addr + ((kt + S - 1) % S) * LY::kStage, A, B, off, K, kt + S - 1, c);
    if constexpr (kBlk) {
      // block kt / 4 + 1 goes into the buffer block kt / 4 - 1 used, whose last reads precede this barrier
      const int nb = (kt >> 2) + 1;
      if (copier && (kt & 3) == 0 && 4 * nb < kt_n)
        load_scale_block<LY, SM>(lds_addr + LY::kOffScaleBuf + (nb & 1) * LY::kScaleBuf, A, B, off, K, nb, c);
      compute<LY, FA, FB, SM>(lds + (kt % S) * LY::kStage, acc, ro,
                              lds + LY::kOffScaleBuf + ((kt >> 2) & 1) * LY::kScaleBuf + 4 * (kt & 3));
    } else {
      compute<LY, FA, FB, SM>(lds + (kt % S) * LY::kStage, acc, ro);
    }
  }
}

// ---- The 4-wave big tile ----------------------------------------------------
//
// With one wave per SIMD a wave's MFMA stream is all its SIMD has, so every
// memory operation sits between two MFMAs and the MFMA pipe keeps issuing.
// K step kt (its codes in stage kt % 2, landed and visible):
//  * column group j = 0..7 issues the 8 MFMAs acc[i][j] += B_i x A_j;
//  * B fragments 0..2 and A fragment 0 were read during the previous step,
//    B 3..7 are read in group 0 three MFMAs ahead of their use, A j+1 in
//    group j;
//  * the wave's 16 copies of step kt + 1 (8 slices of A, 8 of B) go between
//    the MFMAs of groups 0..2, into the other stage, whose reads every wave
//    finished before the previous step's barrier;
//  * before group 7 the wave waits for its copies and meets the others at a
//    barrier: step kt + 1's stage is complete and every read of stage kt is
//    done (group 7 reads none of it);
//  * group 7 reads step kt + 1's first fragments.
// One m0 write serves four copies: a copy's immediate offset moves both its
// global and its LDS address (the soffset takes the global part back).
// Scales: blocks of 4 K steps in the layout scale_blocks_kernel writes (a
// tile row's 16 bytes of a block contiguous, rows consecutive, each row
// [32-block][step]), so a scale copy reads 64 rows' bytes as 1 KB in a row,
// and a lane reads its block's bytes for the 4 steps with one dword read,
// the MFMA selecting the step's byte.  Block b + 1 is copied during steps 4b
// and 4b + 1 (one 64-row slice per wave and step) into the buffer block
// b - 1 used.  Measured on MI355X (8192^3, clocks per K step): scales as
// [rows, K/32] in 4-step blocks 2,700, in 8-step blocks 2,600 (a copy of
// 16-byte pieces of 64 or 32 rows costs several times one of whole lines,
// and each step took 16 byte reads); rearranged 2,350-2,390, where no scale
// traffic at all gives 2,350.
// The MFMAs are inline asm on AGPR accumulators ("+a"): with the builtin the
// compiler's register allocation rotated the 256 accumulators through copies
// and spilled.  The asm keeps the MFMAs out of the compiler's hazard checks,
// so the loop itself orders the accumulators' other accesses behind wait
// states: the zeroing before the first MFMA and the reads after the last.

// acc += B fragment x A fragment with their E8M0 scales; SEL picks the scale
// byte of the two scale registers (op_sel / op_sel_hi of the scale operands).
#define TEMX_MFMA_ASM(MODS)                                                                          \
  asm volatile("v_mfma_scale_f32_16x16x128_f8f6f4 %0, %1, %2, %0, %3, %4 " MODS                     \
               : "+a"(acc) : "v"(bv), "v"(av), "v"(bs), "v"(as))
#define TEMX_MFMA_FMT(SELMODS)                                                                       \
  if constexpr (FA == TE_E4M3 && FB == TE_E4M3) TEMX_MFMA_ASM(SELMODS);                             \
  else if constexpr (FA == TE_E4M3) TEMX_MFMA_ASM(SELMODS " cbsz:1"); /* B (the first operand) E5M2 */ \
  else if constexpr (FB == TE_E4M3) TEMX_MFMA_ASM(SELMODS " blgp:1"); /* A E5M2 */                   \
  else TEMX_MFMA_ASM(SELMODS " cbsz:1 blgp:1");

template <int FA, int FB, int SEL = 0>
__device__ __forceinline__ void mfma_acc(v4f& acc, const v8i& bv, int bs, const v8i& av, int as) {
  if constexpr (SEL == 0) {
    TEMX_MFMA_FMT("op_sel_hi:[0,0,0]")
  } else if constexpr (SEL == 1) {
    TEMX_MFMA_FMT("op_sel:[1,1,0] op_sel_hi:[0,0,0]")
  } else if constexpr (SEL == 2) {
    TEMX_MFMA_FMT("op_sel_hi:[1,1,0]")
  } else {
    TEMX_MFMA_FMT("op_sel:[1,1,0] op_sel_hi:[1,1,0]")
  }
}
#undef TEMX_MFMA_FMT
#undef TEMX_MFMA_ASM

// m0 <- an LDS address, for the direct-to-LDS copies that follow
__device__ __forceinline__ void set_m0(uint32_t lds_addr) { asm volatile("s_mov_b32 m0, %0" ::"s"(lds_addr) : "memory"); }

// buffer_load_dwordx4 ... lds with an immediate offset, which moves the LDS
// address too (lane l lands at m0 + IMM + 16 l).  A VALU write of an SGPR
// (v_readlane, v_readfirstlane) that a vector memory instruction reads needs 5
// wait states, which the compiler cannot insert ahead of an asm statement:
// WAIT puts them in, for code where the compiler may reload the resource or
// offset SGPRs from VGPR lanes right before (measured: without it, copies
// after such reloads read rows at stale offsets).
template <int IMM, bool WAIT = false>
__device__ __forceinline__ void lds_dma16_imm(const i32x4& rsrc, int voff, int soff) {
  if constexpr (WAIT)
    asm volatile("s_nop 4\n\tbuffer_load_dwordx4 %0, %1, %2 offen offset:%3 lds" ::"v"(voff), "s"(rsrc), "s"(soff),
                 "i"(IMM) : "memory");
  else
    asm volatile("buffer_load_dwordx4 %0, %1, %2 offen offset:%3 lds" ::"v"(voff), "s"(rsrc), "s"(soff), "i"(IMM)
                 : "memory");
}

#define TEMX_SCHED_BARRIER() __builtin_amdgcn_sched_barrier(0)

// The lane index, computed afresh where this is called (opaque to the
// compiler): after the 4-wave main loop the epilogue derives its per-lane
// offsets from it instead of keeping the prologue's values live through the
// loop, which has no VGPR to spare.
__device__ __forceinline__ int lane_id_fresh() {
  int l;
  asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(l));
  return l;
}

// The 4-wave tile's direct-to-LDS copies.  Wave w fills slices 8w .. 8w+7
// of A and of B (slice q = rows 8q .. 8q+7, 1 KB); copy t takes slice 8w + t:
// lane l lands at row 8q + l/8, physical chunk l%8, which holds logical chunk
// (l%8) ^ swz(row) = (l%8) ^ (l/16) ^ 4 (t & 1).  vo_e / vo_o: the lane's
// global offsets for even / odd t; vo_s: its offset in a 1-KB scale slice
// (64 rows of 16 bytes).
struct Copy4 {
  int vo_e, vo_o, vo_s;
};
__device__ __forceinline__ Copy4 copy4_offsets(int K, int wave, int lane) {
  const int chunk_e = (lane & 7) ^ (lane >> 4);
  Copy4 co;
  co.vo_e = (64 * wave + (lane >> 3)) * K + chunk_e * 16;
  co.vo_o = (64 * wave + (lane >> 3)) * K + (chunk_e ^ 4) * 16;
  co.vo_s = 16 * lane;
  return co;
}
// data copy c (0..15: A slices, then B) of the K step at byte kbase into the stage at l_stage; copies
// 0, 4, 8 and 12 set m0, the next three add their immediate offset to it (WAIT: see lds_dma16_imm)
template <bool WAIT = false>
__device__ __forceinline__ void copy4_data(const Operand& A, const Operand& B, const Copy4& co, int c, int K,
                                           int kbase, uint32_t l_stage, int wave) {
  const int t = c & 7;
  const bool isb = c >= 8;
  if ((t & 3) == 0)
    set_m0((uint32_t)__builtin_amdgcn_readfirstlane((int)(l_stage + (isb ? Big4::kHalf : 0) + (8 * wave + t) * 1024)));
  const int so = __builtin_amdgcn_readfirstlane(8 * t * K - (t & 3) * 1024) + kbase;
  const int vo = (t & 1) ? co.vo_o : co.vo_e;
  const i32x4& rs = isb ? B.data : A.data;
  switch (t & 3) {
    case 0: lds_dma16_imm<0, WAIT>(rs, vo, so); break;
    case 1: lds_dma16_imm<1024, WAIT>(rs, vo, so); break;
    case 2: lds_dma16_imm<2048, WAIT>(rs, vo, so); break;
    default: lds_dma16_imm<3072, WAIT>(rs, vo, so); break;
  }
}
// scale slice s = wave + 4k of block blk (1 KB: 64 rows of 16 bytes) into the scale buffer at l_sbuf:
// k = 0 A rows 64 w .., k = 1 B rows 64 w ..  (a_blk / b_blk: the byte offset of one block)
template <bool WAIT = false>
__device__ __forceinline__ void copy4_scales(const Operand& A, const Operand& B, const Copy4& co, int blk,
                                             uint32_t l_sbuf, int k, int wave, int a_blk, int b_blk) {
  const int s = wave + 4 * k;
  blk = __builtin_amdgcn_readfirstlane(blk);
  asm volatile("" : "+s"(blk));
  set_m0((uint32_t)__builtin_amdgcn_readfirstlane((int)(l_sbuf + s * 1024)));
  const int so = __builtin_amdgcn_readfirstlane(1024 * wave) + blk * (k == 0 ? a_blk : b_blk);
  if (k == 0) lds_dma16_imm<0, WAIT>(A.scale, co.vo_s, so);
  else lds_dma16_imm<0, WAIT>(B.scale, co.vo_s, so);
}

// A tile's K step 0 into stage 0, and (MXFP8) its scale block 0 into scale
// buffer 0; mainloop4 waits for these copies.  The persistent kernel issues
// them for its next tile as soon as the current tile's main loop is done: the
// last step reads stage 1 and scale buffer 1 only (K / 128 is a multiple of
// 8), and every wave is past the step before it.  Its copies take the wait
// states of lds_dma16_imm: between tiles the compiler reloads their offsets.
template <int SM>
__device__ __forceinline__ void prologue4(uint8_t* lds, const Operand& A, const Operand& B, int64_t K64, int wave,
                                          int a_blk, int b_blk) {
  const int K = (int)K64;
  const Copy4 co = copy4_offsets(K, wave, lane_id_fresh());
  const uint32_t l0 = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) uint8_t*)lds;
  int m0_saved;
  asm volatile("s_mov_b32 %0, m0" : "=s"(m0_saved));
#pragma unroll
  for (int c = 0; c < 16; ++c) copy4_data<true>(A, B, co, c, K, 0, l0, wave);
  if constexpr (SM == SM_MX) {
#pragma unroll
    for (int k = 0; k < 2; ++k) copy4_scales<true>(A, B, co, 0, l0 + Big4::kOffScale, k, wave, a_blk, b_blk);
  }
  asm volatile("s_mov_b32 m0, %0" ::"s"(m0_saved) : "memory");
}

// MXFP8 scales come in the layout of scale_blocks_kernel (a_blk / b_blk: the
// byte offset of one scale block of A / B, rows x 16).  Step 0's copies were
// issued by prologue4.
template <int FA, int FB, int SM>
__device__ __forceinline__ void mainloop4(uint8_t* lds, v4f (&acc)[8][8], const Operand& A, const Operand& B,
                                          int64_t K64, int wave, int a_blk = 0, int b_blk = 0) {
  static_assert(SM == SM_MX || SM == SM_PT, "E8M0 block scales or none");
  using LY = Big4;
  // the per-lane offsets below start from a fresh lane index, so none of them is computed ahead of
  // this function and kept live through it
  const int lane = lane_id_fresh();
  constexpr int kNcg = 3;                            // column groups that carry the copies
  constexpr int kScaleSlot = (4 * 8 * kNcg) / 16;    // the slot of data copy 4, which sets m0 again
  const int K = (int)K64;
  const int kt_n = K / BK;  // a multiple of 8, > 0
  const int wm = wave >> 1, wn = wave & 1;
  // zeros into the AGPRs, and wait states after them: the compiler cannot see the MFMAs read them (a
  // VALU write read as an MFMA's accumulator input needs a gap)
  // (the zero comes from an opaque move here, so the compiler keeps no copy of it live from elsewhere)
  float zero;
  asm volatile("v_mov_b32 %0, 0" : "=v"(zero));
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      acc[i][j] = v4f{zero, zero, zero, zero};
      asm volatile("" : "+a"(acc[i][j]));
    }
  asm volatile("s_nop 7" ::: "memory");
  const uint32_t l0 = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) uint8_t*)lds;

  Copy4 co = copy4_offsets(K, wave, lane);
  // fragment reads: lane 16 g + r reads logical chunks g and g + 4 of row r of each fragment
  const int g = lane >> 4, r = lane & 15;
  const int lane_off = r * BK + ((g ^ swz(r)) << 4);
  int ra_off = wm * 128 * BK + lane_off;                                  // + 2 KB j
  int rb_off = LY::kHalf + wn * 128 * BK + lane_off;                      // + 2 KB i
  // a scale read: lane (g, r) takes the dword of block g of row r for the 4 steps (a row's 16 bytes
  // are [block][step]); the MFMA picks the step's byte
  int sa_off = (wm * 128 + r) * LY::kScaleRow + 4 * g;                        // + 256 j
  int sb_off = LY::BM * LY::kScaleRow + (wn * 128 + r) * LY::kScaleRow + 4 * g;  // + 256 i
  asm volatile("" : "+v"(co.vo_e), "+v"(co.vo_o), "+v"(co.vo_s), "+v"(ra_off), "+v"(rb_off), "+v"(sa_off),
               "+v"(sb_off));

  auto copy = [&](int c, int kbase, uint32_t l_stage) __attribute__((always_inline)) {
    copy4_data(A, B, co, c, K, kbase, l_stage, wave);
  };
  auto copy_scales = [&](int blk, uint32_t l_sbuf, int k) __attribute__((always_inline)) {
    copy4_scales(A, B, co, blk, l_sbuf, k, wave, a_blk, b_blk);
  };
  int held[16];  // each fragment's scale dword of the current 4 steps (A 0..7, B 8..15)
  auto rd = [&](const uint8_t* stg, const uint8_t* sbuf, int off, int soff, int f, int sub, int h)
                __attribute__((always_inline)) {
    Frag fr;
    const uint4 lo = *reinterpret_cast<const uint4*>(stg + off + f * 16 * BK);
    const uint4 hi = *reinterpret_cast<const uint4*>(stg + (off ^ 64) + f * 16 * BK);
    fr.v = v8i{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
    if constexpr (SM == SM_PT) {
      fr.s = 127;  // 2^0 in every byte the MFMA may pick
    } else {
      if ((sub & 3) == 0) held[h] = *reinterpret_cast<const int*>(sbuf + soff + f * 16 * LY::kScaleRow);
      fr.s = held[h];
    }
    return fr;
  };

  int m0_saved;
  asm volatile("s_mov_b32 %0, m0" : "=s"(m0_saved));
  // step 0's stage and scale block 0 (prologue4) have landed, and every wave is done with the LDS
  // (a previous tile's epilogue stages its output in stage 1)
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  Frag Af0, Bf[3];  // the step's first fragments, read during the previous step
  Af0 = rd(lds, lds + LY::kOffScale, ra_off, sa_off, 0, 0, 0);
#pragma unroll
  for (int i = 0; i < 3; ++i) Bf[i] = rd(lds, lds + LY::kOffScale, rb_off, sb_off, i, 0, 8 + i);

  auto step = [&](int kt, auto s8c, auto more_c) __attribute__((always_inline)) {
    constexpr int S8 = decltype(s8c)::value;  // kt % 8
    constexpr bool MORE = decltype(more_c)::value;
    const uint8_t* cur = lds + (S8 & 1) * LY::kStage;
    const uint8_t* nxt = lds + ((S8 & 1) ^ 1) * LY::kStage;
    const uint32_t l_nxt = l0 + ((S8 & 1) ^ 1) * LY::kStage;
    const uint8_t* sbuf = lds + LY::kOffScale + ((kt >> 2) & 1) * LY::kScaleBuf;
    const uint8_t* sbuf_n = lds + LY::kOffScale + (((kt + 1) >> 2) & 1) * LY::kScaleBuf;
    // opaque, so that the copies' offsets are a few hoisted constants plus this
    int kbase_n = __builtin_amdgcn_readfirstlane((kt + 1) * BK);
    asm volatile("" : "+s"(kbase_n));
    Frag Bv[8], Av[2];
    Bv[0] = Bf[0];
    Bv[1] = Bf[1];
    Bv[2] = Bf[2];
    Av[0] = Af0;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      if (j == 7) {
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
        TEMX_SCHED_BARRIER();
      }
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int slot = 8 * j + i;
        mfma_acc<FA, FB, SM == SM_MX ? (S8 & 3) : 0>(acc[i][j], Bv[i].v, Bv[i].s, Av[j & 1].v, Av[j & 1].s);
        if (j == 0 && i + 3 < 8) Bv[i + 3] = rd(cur, sbuf, rb_off, sb_off, i + 3, S8, 8 + i + 3);
        if (j < 7 && i == 4) Av[(j + 1) & 1] = rd(cur, sbuf, ra_off, sa_off, j + 1, S8, j + 1);
        if (SM == SM_MX && (S8 & 3) < 2 && slot == kScaleSlot)
          copy_scales((kt >> 2) + 1, l0 + LY::kOffScale + ((((kt >> 2) + 1) & 1) * LY::kScaleBuf), S8 & 3);
        if (MORE) {
#pragma unroll
          for (int c = 0; c < 16; ++c)
            if ((c * 8 * kNcg) / 16 == slot) copy(c, kbase_n, l_nxt);
        }
        if (MORE && j == 7) {
          if (i == 0) Af0 = rd(nxt, sbuf_n, ra_off, sa_off, 0, (S8 + 1) & 7, 0);
          if (i >= 1 && i <= 3) Bf[i - 1] = rd(nxt, sbuf_n, rb_off, sb_off, i - 1, (S8 + 1) & 7, 8 + i - 1);
        }
        TEMX_SCHED_BARRIER();
      }
    }
  };
  using T = std::true_type;
  using F = std::false_type;
  auto eight = [&](int k0, auto last) __attribute__((always_inline)) {
    step(k0, std::integral_constant<int, 0>{}, T{});
    step(k0 + 1, std::integral_constant<int, 1>{}, T{});
    step(k0 + 2, std::integral_constant<int, 2>{}, T{});
    step(k0 + 3, std::integral_constant<int, 3>{}, T{});
    step(k0 + 4, std::integral_constant<int, 4>{}, T{});
    step(k0 + 5, std::integral_constant<int, 5>{}, T{});
    step(k0 + 6, std::integral_constant<int, 6>{}, T{});
    step(k0 + 7, std::integral_constant<int, 7>{}, last);
  };
  int kt = 0;
  for (; kt < kt_n - 8; kt += 8) eight(kt, T{});
  eight(kt, F{});
  // the last MFMAs' results: wait states before anything reads them (an MFMA result read by another
  // instruction needs at most 19 on gfx950), and the copies' m0 back.  The empty asm statements tie
  // every accumulator to a point after the wait states, so the compiler cannot read one earlier.
  asm volatile("s_nop 15\n\ts_nop 15\n\ts_mov_b32 m0, %0" ::"s"(m0_saved) : "memory");
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int j = 0; j < 8; ++j) asm volatile("" : "+a"(acc[i][j]));
}

// Epilogue from registers.  acc[i][j][e] is D[m][n] with
// m = m0 + WTM wm + 16 j + (lane & 15), n = n0 + WTN wn + 16 i + 4 (lane >> 4) + e.
// A store instruction writes 32 bytes of each of 16 rows; the row fragments
// are the outer loop, so the pieces of one row's line leave in consecutive
// stores and meet in L2 before it writes the line back (measured: 4096 x
// 4096 x 1024 with GELU aux 42.2 -> 37.8 us, against the column-fragment
// order, whose scattered partial lines doubled the bytes written).
// a * b rounded on its own: never contracted into an FMA with a later add
__device__ __forceinline__ float mul_rn(float a, float b) {
#pragma clang fp contract(off)
  return a * b;
}

// SCALE: each result is first multiplied by alpha (its own rounding, no FMA
// with the bias add), fragment by fragment: the per-tensor mode of the
// 4-wave tile, whose 256 accumulators cannot all pass through VGPRs at once.
template <class LY, int EPI, int OUT, bool SCALE = false>
__device__ __forceinline__ void epilogue(v4f (&acc)[LY::FRN][LY::FRM], void* d, uint16_t* aux,
                                         const uint16_t* bias, int64_t m0, int64_t m_end, int64_t n0, int64_t N,
                                         int wave, int lane, float beta = 1.0f, float alpha = 1.0f) {
  const int wm = wave / LY::NWN, wn = wave % LY::NWN;
  const int g = lane >> 4, r = lane & 15;
  // bias of the lane's columns, all fragments (columns past N, never stored, read column 0's)
  float bv[LY::FRN][4];
#pragma unroll
  for (int i = 0; i < LY::FRN; ++i) {
    const int64_t n = n0 + wn * LY::WTN + 16 * i + 4 * g;
    if constexpr (EPI == TE_EPI_BIAS || EPI == TE_EPI_BIAS_GELU_AUX) {
      const uint2 bb = *reinterpret_cast<const uint2*>(bias + (n < N ? n : 0));
      bv[i][0] = bf16_bits_to_float(bb.x & 0xFFFFu);
      bv[i][1] = bf16_bits_to_float(bb.x >> 16);
      bv[i][2] = bf16_bits_to_float(bb.y & 0xFFFFu);
      bv[i][3] = bf16_bits_to_float(bb.y >> 16);
    } else {
      bv[i][0] = bv[i][1] = bv[i][2] = bv[i][3] = 0.f;
    }
  }
  // row fragments outermost: a row's pieces of the wave's columns leave in consecutive stores
#pragma unroll
  for (int j = 0; j < LY::FRM; ++j) {
    const int64_t m = m0 + wm * LY::WTM + 16 * j + r;
    if (m >= m_end) continue;
#pragma unroll
    for (int i = 0; i < LY::FRN; ++i) {
      const int64_t n = n0 + wn * LY::WTN + 16 * i + 4 * g;
      if (n >= N) continue;
      // 4-wave tile: the fragment's AGPRs are read here and not hoisted above the row / column checks
      // (256 accumulators do not all fit in VGPRs at once)
      if constexpr (LY::FRN * LY::FRM > 32) asm volatile("" : "+a"(acc[i][j]));
      float v0 = acc[i][j][0], v1 = acc[i][j][1], v2 = acc[i][j][2], v3 = acc[i][j][3];
      if constexpr (SCALE) {
        v0 = mul_rn(v0, alpha);
        v1 = mul_rn(v1, alpha);
        v2 = mul_rn(v2, alpha);
        v3 = mul_rn(v3, alpha);
      }
      if constexpr (EPI == TE_EPI_BIAS || EPI == TE_EPI_BIAS_GELU_AUX) {
        v0 += bv[i][0];
        v1 += bv[i][1];
        v2 += bv[i][2];
        v3 += bv[i][3];
      }
      if constexpr (EPI == TE_EPI_BIAS_GELU_AUX) {
        *reinterpret_cast<uint2*>(aux + m * N + n) = make_uint2(pack_bf16x2(v0, v1), pack_bf16x2(v2, v3));
        v0 = gelu_tanh(v0);
        v1 = gelu_tanh(v1);
        v2 = gelu_tanh(v2);
        v3 = gelu_tanh(v3);
      }
      if constexpr (EPI == TE_EPI_DGELU) {  // aux holds the saved bf16 pre-activation
        const uint2 pa = *reinterpret_cast<const uint2*>(aux + m * N + n);
        v0 *= dgelu_tanh(bf16_bits_to_float(pa.x & 0xFFFFu));
        v1 *= dgelu_tanh(bf16_bits_to_float(pa.x >> 16));
        v2 *= dgelu_tanh(bf16_bits_to_float(pa.y & 0xFFFFu));
        v3 *= dgelu_tanh(bf16_bits_to_float(pa.y >> 16));
      }
      if constexpr (EPI == TE_EPI_ACCUMULATE) {  // fp32 D is read, scaled by beta and added to (one rounding)
        const float4 c = *reinterpret_cast<const float4*>(static_cast<float*>(d) + m * N + n);
        v0 = __builtin_fmaf(beta, c.x, v0);
        v1 = __builtin_fmaf(beta, c.y, v1);
        v2 = __builtin_fmaf(beta, c.z, v2);
        v3 = __builtin_fmaf(beta, c.w, v3);
      }
      if constexpr (OUT == TE_BF16) {
        *reinterpret_cast<uint2*>(static_cast<uint16_t*>(d) + m * N + n) =
            make_uint2(pack_bf16x2(v0, v1), pack_bf16x2(v2, v3));
      } else if constexpr (OUT == TE_FP16) {
        *reinterpret_cast<uint2*>(static_cast<uint16_t*>(d) + m * N + n) =
            make_uint2(pack_f16x2(v0, v1), pack_f16x2(v2, v3));
      } else {
        *reinterpret_cast<float4*>(static_cast<float*>(d) + m * N + n) = make_float4(v0, v1, v2, v3);
      }
    }
  }
}

// Epilogue of the 2-byte outputs (bf16 / fp16 D, and the bf16 GELU aux)
// through LDS.  Stored straight from the MFMA layout, a wave store writes 32
// bytes into each of 16 rows: 16 partial lines per instruction, which left
// the store path the slowest part of a decoder-sized GEMM.  Here each wave
// writes blocks of up to 64 rows x WTN of 2-byte results to a region of LDS
// of its own (row q at q * 2 WTN bytes, 16-byte chunk c at chunk c ^ (q % CH),
// CH chunks per row: the 8-byte writes and the 16-byte reads are both free of
// bank conflicts), then reads each back row-major, 16 bytes per lane, and
// stores 2 WTN contiguous bytes of each of 64 / CH rows per instruction.
// The LDS is free once every wave has finished the last step's reads (the
// barrier below); the region is reused by the next block (and with the GELU
// aux, aux first, then D), since LDS accesses of one wave complete in issue
// order.  The regions of all waves take staged_bytes<LY>() from lds.
// A staged row's bytes: 2 WTN, rounded up to a power of two (96-column waves
// use 12 of 16 chunks), so the chunk swizzle stays an XOR.
template <class LY>
constexpr int staged_row_bytes() {
  int rb = 16;
  while (rb < 2 * LY::WTN) rb *= 2;
  return rb;
}

template <class LY, int ROWS>
__device__ __forceinline__ void store_region(const uint8_t* region, uint16_t* out, int64_t mb, int64_t m_end,
                                             int64_t nb, int64_t N, int lane) {
  constexpr int RB = staged_row_bytes<LY>(), CHP = RB / 16, CH = LY::WTN * 2 / 16;
  static_assert(ROWS * CH % 64 == 0, "whole store instructions");
#pragma unroll
  for (int t = 0; t < ROWS * CH / 64; ++t) {
    const int q = (64 * t + lane) / CH, c = (64 * t + lane) % CH;
    const uint4 v = *reinterpret_cast<const uint4*>(region + q * RB + ((c ^ (q & (CHP - 1))) << 4));
    const int64_t m = mb + q, n = nb + 8 * c;  // N % 16 == 0: a chunk of 8 columns is all in or all out
    if (m < m_end && n < N) *reinterpret_cast<uint4*>(out + m * N + n) = v;
  }
}

constexpr bool staged_epilogue(int epi, int out) {
  return (out == TE_BF16 || out == TE_FP16) &&
         (epi == TE_EPI_NONE || epi == TE_EPI_BIAS || epi == TE_EPI_BIAS_GELU_AUX);
}
template <class LY>
constexpr int staged_row_frags() { return LY::FRM < 4 ? LY::FRM : 4; }  // row fragments per staged block
template <class LY>
constexpr int staged_bytes() { return LY::NW * 16 * staged_row_frags<LY>() * staged_row_bytes<LY>(); }
// LDS of a dense 8- or 4-wave kernel: its stages and scale buffers, or the
// staged epilogue's regions if those are larger (256 x 192: 128 KB against 126)
template <class LY>
constexpr int lds_bytes() { return LY::kLds > staged_bytes<LY>() ? LY::kLds : staged_bytes<LY>(); }

template <class LY, int EPI, int OUT, bool SCALE = false>
__device__ __forceinline__ void epilogue_lds(v4f (&acc)[LY::FRN][LY::FRM], uint8_t* lds, void* d,
                                             uint16_t* aux, const uint16_t* bias, int64_t m0, int64_t m_end,
                                             int64_t n0, int64_t N, int wave, int lane, float alpha = 1.0f) {
  static_assert(OUT == TE_BF16 || OUT == TE_FP16, "2-byte outputs");
  static_assert(EPI == TE_EPI_NONE || EPI == TE_EPI_BIAS || EPI == TE_EPI_BIAS_GELU_AUX, "forward epilogues");
  constexpr int FRH = staged_row_frags<LY>(), RB = staged_row_bytes<LY>(), CH = RB / 16, kRegion = 16 * FRH * RB;
  static_assert(CH <= 16 && LY::FRM % FRH == 0 && staged_bytes<LY>() <= lds_bytes<LY>(), "staging layout");
  const int wm = wave / LY::NWN, wn = wave % LY::NWN;
  const int g = lane >> 4, r = lane & 15;
  uint8_t* region = lds + wave * kRegion;
  const int64_t mb = m0 + wm * LY::WTM, nb = n0 + wn * LY::WTN;
  // With up to 32 fragments the bias is added in place (the accumulators are not needed afterwards):
  // fewer live registers than keeping the bias beside them through both passes.  The 4-wave tile's
  // 256 accumulators live in AGPRs, where an in-place add would pull them all into VGPRs: there each
  // pass adds the bias (held, 4 values per column fragment) fragment by fragment.
  constexpr bool kHasBias = EPI == TE_EPI_BIAS || EPI == TE_EPI_BIAS_GELU_AUX;
  constexpr bool kInPlace = LY::FRN * LY::FRM <= 32;
  float bv[kInPlace ? 1 : LY::FRN][4];
  if constexpr (kHasBias && !kInPlace) {
#pragma unroll
    for (int i = 0; i < LY::FRN; ++i) {
      // columns past N (never stored) read column 0's bias: no zero defaults, whose registers the
      // compiler may set up ahead of the main loop and keep live through it
      const int64_t n = nb + 16 * i + 4 * g;
      const uint2 bb = *reinterpret_cast<const uint2*>(bias + (n < N ? n : 0));
      bv[i][0] = bf16_bits_to_float(bb.x & 0xFFFFu);
      bv[i][1] = bf16_bits_to_float(bb.x >> 16);
      bv[i][2] = bf16_bits_to_float(bb.y & 0xFFFFu);
      bv[i][3] = bf16_bits_to_float(bb.y >> 16);
    }
  }
  if constexpr (kHasBias && kInPlace) {
#pragma unroll
    for (int i = 0; i < LY::FRN; ++i) {
      const int64_t n = nb + 16 * i + 4 * g;
      if (n < N) {
        const uint2 bb = *reinterpret_cast<const uint2*>(bias + n);
        const float b0 = bf16_bits_to_float(bb.x & 0xFFFFu), b1 = bf16_bits_to_float(bb.x >> 16);
        const float b2 = bf16_bits_to_float(bb.y & 0xFFFFu), b3 = bf16_bits_to_float(bb.y >> 16);
#pragma unroll
        for (int j = 0; j < LY::FRM; ++j) {
          if constexpr (SCALE) {
            acc[i][j][0] = mul_rn(acc[i][j][0], alpha) + b0;
            acc[i][j][1] = mul_rn(acc[i][j][1], alpha) + b1;
            acc[i][j][2] = mul_rn(acc[i][j][2], alpha) + b2;
            acc[i][j][3] = mul_rn(acc[i][j][3], alpha) + b3;
          } else {
            acc[i][j][0] += b0;
            acc[i][j][1] += b1;
            acc[i][j][2] += b2;
            acc[i][j][3] += b3;
          }
        }
      }
    }
  }
  __syncthreads();  // every wave's reads of the last stage are done: the LDS is free
  // lane (g, r) of fragment (i, j): row 16 j + r, 8 bytes at byte 32 i + 8 g = chunk 2 i + g / 2, half g % 2
  const int wr_off = r * RB + ((g & 1) << 3);
  constexpr int kPasses = EPI == TE_EPI_BIAS_GELU_AUX ? 2 : 1;
#pragma unroll
  for (int pass = 0; pass < kPasses; ++pass) {
    const bool to_aux = kPasses == 2 && pass == 0;
#pragma unroll
    for (int h = 0; h < LY::FRM / FRH; ++h) {
#pragma unroll
      for (int jj = 0; jj < FRH; ++jj) {
        const int j = FRH * h + jj;
#pragma unroll
        for (int i = 0; i < LY::FRN; ++i) {
          // 4-wave tile: the fragment's AGPRs are read here, one fragment at a time through VGPRs
          if constexpr (!kInPlace) asm volatile("" : "+a"(acc[i][j]));
          float v0 = acc[i][j][0], v1 = acc[i][j][1], v2 = acc[i][j][2], v3 = acc[i][j][3];
          if constexpr (SCALE && !(kHasBias && kInPlace)) {  // in place with the bias, alpha went in above
            v0 = mul_rn(v0, alpha);
            v1 = mul_rn(v1, alpha);
            v2 = mul_rn(v2, alpha);
            v3 = mul_rn(v3, alpha);
          }
          if constexpr (kHasBias && !kInPlace) {
            v0 += bv[i][0];
            v1 += bv[i][1];
            v2 += bv[i][2];
            v3 += bv[i][3];
          }
          uint2 w;
          if (EPI == TE_EPI_BIAS_GELU_AUX && !to_aux) {
            v0 = gelu_tanh(v0);
            v1 = gelu_tanh(v1);
            v2 = gelu_tanh(v2);
            v3 = gelu_tanh(v3);
          }
          if (OUT == TE_FP16 && !to_aux)
            w = make_uint2(pack_f16x2(v0, v1), pack_f16x2(v2, v3));
          else
            w = make_uint2(pack_bf16x2(v0, v1), pack_bf16x2(v2, v3));
          const int q = 16 * jj + r, chunk = 2 * i + (g >> 1);
          *reinterpret_cast<uint2*>(region + wr_off + 16 * jj * RB + ((chunk ^ (q & (CH - 1))) << 4)) = w;
        }
      }
      asm volatile("" ::: "memory");
      store_region<LY, 16 * FRH>(region, to_aux ? aux : static_cast<uint16_t*>(d), mb + 16 * FRH * h, m_end, nb, N,
                                 lane);
      asm volatile("" ::: "memory");
    }
    if constexpr (!kInPlace && kPasses == 2) {
      // the second pass reads the AGPRs again: without this the compiler keeps the first pass's
      // 256 VGPR copies live between the passes
      if (pass == 0) {
#pragma unroll
        for (int i = 0; i < LY::FRN; ++i)
#pragma unroll
          for (int j = 0; j < LY::FRM; ++j) asm volatile("" : "+a"(acc[i][j]));
      }
    }
  }
}

// MXFP8 rowwise output.  The epilogue's fp32 results are rounded to bf16
// exactly as for a bf16 D and then quantized in 32-column blocks (one E8M0
// scale each, as the rowwise quantize kernel does), so the codes equal the
// rowwise quantization of the bf16 D this GEMM writes otherwise: the next
// GEMM sees the same operand without a bf16 round trip through memory.
// Lane 16 g + r holds columns 16 i + 4 g .. +3 of row r, so the block
// 32 b .. 32 b + 31 (i = 2b, 2b+1) sits in lanes r, r+16, r+32, r+48: the
// block amax is a max over the lane's 8 values and then across those 4 lanes.
template <class LY, int EPI, int FMT>
__device__ __forceinline__ void epilogue_mx(const v4f (&acc)[LY::FRN][LY::FRM], uint8_t* d, uint8_t* d_scale,
                                            uint16_t* aux, const uint16_t* bias, int64_t m0, int64_t m_end,
                                            int64_t n0, int64_t N, int wave, int lane) {
  static_assert(EPI == TE_EPI_NONE || EPI == TE_EPI_BIAS || EPI == TE_EPI_BIAS_GELU_AUX, "forward epilogues only");
  const int wm = wave / LY::NWN, wn = wave % LY::NWN;
  const int g = lane >> 4, r = lane & 15;
  constexpr int NB = LY::FRN / 2;  // 32-column blocks of the wave
  float bv[NB][8];
#pragma unroll
  for (int b = 0; b < NB; ++b) {
    const int64_t nb = n0 + wn * LY::WTN + 32 * b;
#pragma unroll
    for (int k = 0; k < 8; ++k) bv[b][k] = 0.f;
    if constexpr (EPI != TE_EPI_NONE) {
      if (nb < N) {
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const uint2 bb = *reinterpret_cast<const uint2*>(bias + nb + 16 * h + 4 * g);
          bv[b][4 * h + 0] = bf16_bits_to_float(bb.x & 0xFFFFu);
          bv[b][4 * h + 1] = bf16_bits_to_float(bb.x >> 16);
          bv[b][4 * h + 2] = bf16_bits_to_float(bb.y & 0xFFFFu);
          bv[b][4 * h + 3] = bf16_bits_to_float(bb.y >> 16);
        }
      }
    }
  }
  // row fragments outermost, as in the bf16 epilogue: a row's pieces leave in consecutive stores
#pragma unroll
  for (int j = 0; j < LY::FRM; ++j) {
    const int64_t m = m0 + wm * LY::WTM + 16 * j + r;
    const bool row_ok = m < m_end;
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      const int64_t nb = n0 + wn * LY::WTN + 32 * b;  // wave-uniform; with N % 32 == 0 a block is all in or all out
      if (nb >= N) continue;
      float v[8];
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int e = 0; e < 4; ++e) v[4 * h + e] = acc[2 * b + h][j][e] + bv[b][4 * h + e];
      if constexpr (EPI == TE_EPI_BIAS_GELU_AUX) {
        if (row_ok) {
#pragma unroll
          for (int h = 0; h < 2; ++h)
            *reinterpret_cast<uint2*>(aux + m * N + nb + 16 * h + 4 * g) =
                make_uint2(pack_bf16x2(v[4 * h], v[4 * h + 1]), pack_bf16x2(v[4 * h + 2], v[4 * h + 3]));
        }
#pragma unroll
        for (int k = 0; k < 8; ++k) v[k] = gelu_tanh(v[k]);
      }
      const uint4 bits = {pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]), pack_bf16x2(v[4], v[5]),
                          pack_bf16x2(v[6], v[7])};
      uint32_t amax = absmax_bits8(bits);  // every lane takes part in the exchanges
      amax = max(amax, (uint32_t)__builtin_amdgcn_ds_swizzle((int)amax, 0x401F));               // lane ^ 16
      amax = max(amax, (uint32_t)__builtin_amdgcn_ds_bpermute((lane ^ 32) << 2, (int)amax));    // lane ^ 32
      const uint32_t code = e8m0_code_from_amax_bits<FMT>(amax);
      const uint2 q = cvt8_scaled<FMT>(bits, e8m0_to_float(code));
      // lane g holds bytes 4g .. 4g+3 (q.x) and 16+4g .. 16+4g+3 (q.y) of the row's block; lane G
      // stores bytes 8G .. 8G+7, field G >> 1 of lanes 2 (G & 1) and 2 (G & 1) + 1 of the same row
      // (8-byte pieces: measured 38.3 -> 34.8 us on 4096 x 4096 x 1024 with GELU aux)
      const int src_lo = ((2 * (g & 1)) << 4 | r) << 2, src_hi = ((2 * (g & 1) + 1) << 4 | r) << 2;
      const uint32_t xlo = (uint32_t)__builtin_amdgcn_ds_bpermute(src_lo, (int)q.x);
      const uint32_t xhi = (uint32_t)__builtin_amdgcn_ds_bpermute(src_hi, (int)q.x);
      const uint32_t ylo = (uint32_t)__builtin_amdgcn_ds_bpermute(src_lo, (int)q.y);
      const uint32_t yhi = (uint32_t)__builtin_amdgcn_ds_bpermute(src_hi, (int)q.y);
      if (row_ok) {
        *reinterpret_cast<uint2*>(d + m * N + nb + 8 * g) = (g >> 1) ? make_uint2(ylo, yhi) : make_uint2(xlo, xhi);
        if (g == 0) d_scale[m * (N / 32) + nb / 32] = (uint8_t)code;
      }
    }
  }
}

struct GemmParams {
  const uint8_t* a;
  const uint8_t* a_scale;
  const uint8_t* b;
  const uint8_t* b_scale;
  void* d;
  const uint16_t* bias;
  uint16_t* aux;
  int64_t M, N, K;
  const int32_t* m_splits;  // grouped only
  int32_t groups;           // grouped only
  uint8_t* d_scale;         // MXFP8 output only: E8M0 scales [M, N/32]
  const float* alpha_a;     // per-tensor FP8 only: a_scale_inv and b_scale_inv (device scalars)
  const float* alpha_b;
  float beta = 1.0f;        // accumulate epilogue: D = fl32(beta D + acc)
};

// Workgroup b's tile: workgroups are dealt round-robin to the 8 XCDs, so
// each XCD is given a contiguous run of tiles, rastered in bands of kGroupM
// row-tiles.
__device__ __forceinline__ void raster_tile(int bid, int ntm, int ntn, int& tm, int& tn) {
  const int ntiles = ntm * ntn;
  const int per = ntiles / 8;
  const int t = bid < 8 * per ? (bid % 8) * per + bid / 8 : bid;
  const int band = t / (kGroupM * ntn);
  const int first_tm = band * kGroupM;
  const int band_rows = min(ntm - first_tm, kGroupM);
  const int in_band = t % (kGroupM * ntn);
  tm = first_tm + in_band % band_rows;
  tn = in_band / band_rows;
}

// A dense tile's accumulators to D (and aux / MXFP8 scales), per the epilogue
// and scaling mode.
template <class LY, int EPI, int OUT, int SM>
__device__ __forceinline__ void finish_tile(v4f (&acc)[LY::FRN][LY::FRM], uint8_t* lds, const GemmParams& p,
                                            int64_t m0, int64_t n0, int wave, int lane) {
  if constexpr (SM == SM_PT && LY::FRM * LY::FRN > 32) {
    // alpha goes in fragment by fragment inside the epilogue (per-tensor mode: bf16 or fp32 D)
    static_assert(OUT == TE_BF16 || OUT == TE_FP32, "per-tensor outputs");
    const float alpha = *p.alpha_a * *p.alpha_b;
    if constexpr (staged_epilogue(EPI, OUT))
      epilogue_lds<LY, EPI, OUT, true>(acc, lds, p.d, p.aux, p.bias, m0, p.M, n0, p.N, wave, lane, alpha);
    else
      epilogue<LY, EPI, OUT, true>(acc, p.d, p.aux, p.bias, m0, p.M, n0, p.N, wave, lane, p.beta, alpha);
    return;
  }
  if constexpr (SM == SM_PT) {
    // these products are rounded on their own: with contraction off here the
    // epilogue's bias add stays a second rounding instead of becoming an FMA
#pragma clang fp contract(off)
    const float alpha = *p.alpha_a * *p.alpha_b;
#pragma unroll
    for (int i = 0; i < LY::FRN; ++i)
#pragma unroll
      for (int j = 0; j < LY::FRM; ++j) acc[i][j] *= alpha;
  }
  if constexpr (OUT == TE_E4M3 || OUT == TE_E5M2)
    epilogue_mx<LY, EPI, OUT>(acc, static_cast<uint8_t*>(p.d), p.d_scale, p.aux, p.bias, m0, p.M, n0, p.N, wave,
                              lane);
  else if constexpr (staged_epilogue(EPI, OUT))
    epilogue_lds<LY, EPI, OUT>(acc, lds, p.d, p.aux, p.bias, m0, p.M, n0, p.N, wave, lane);
  else
    epilogue<LY, EPI, OUT>(acc, p.d, p.aux, p.bias, m0, p.M, n0, p.N, wave, lane, p.beta);
}

// Dense: one workgroup per tile, operands scaled as SM says (SM_PT: the
// accumulators are multiplied by alpha = a_scale_inv * b_scale_inv before the
// epilogue).
template <class LY, int FA, int FB, int EPI, int OUT, int SM = SM_MX>
__global__ __launch_bounds__(LY::kThreads) void mx_gemm_kernel(GemmParams p) {
  constexpr int BM = LY::BM, BN = LY::BN;
  __shared__ __attribute__((aligned(1024))) uint8_t lds[lds_bytes<LY>()];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  int tm, tn;
  raster_tile(blockIdx.x, (int)((p.M + BM - 1) / BM), (int)((p.N + BN - 1) / BN), tm, tn);
  const int64_t m0 = (int64_t)tm * BM, n0 = (int64_t)tn * BN;
  const Operand A = make_operand(p.a, p.a_scale, m0, p.M - m0, p.K, BM);
  const Operand B = b_2d(SM) ? make_operand_2d(p.b, p.b_scale, n0, p.N - n0, p.K, BN)
                                 : make_operand(p.b, p.b_scale, n0, p.N - n0, p.K, BN);
  v4f acc[LY::FRN][LY::FRM];
  mainloop<LY, FA, FB, SM>(lds, acc, A, B, p.K, wave, lane);
  finish_tile<LY, EPI, OUT, SM>(acc, lds, p, m0, n0, wave, lane);
}

// The E8M0 scales of an operand [rows, K/32] rearranged for the 4-wave tile:
// blocks of 4 K steps (16 scale bytes of a row), block-major, each row's 16
// bytes ordered [32-block g][step s] (byte 4 g + s) instead of [s][g]:
//   out[blk][row][4 g + s] = in[row][4 (4 blk + s) + g].
// A tile's scale block is then one contiguous run per operand (its copies
// read 8 whole lines per instruction instead of 64 partial ones), and a lane
// reads the scales of the block's 4 steps with one dword read, the MFMA
// picking the step's byte.  One launch for both operands: threads
// [0, rows_a * nblk) take A's (row, block) pairs, the rest B's.
__global__ __launch_bounds__(256) void scale_blocks_kernel(const uint8_t* __restrict__ a_in, int64_t rows_a,
                                                           uint8_t* __restrict__ a_out,
                                                           const uint8_t* __restrict__ b_in, int64_t rows_b,
                                                           uint8_t* __restrict__ b_out, int64_t ks) {
  const int64_t nblk = ks / 16;
  int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const uint8_t* in = a_in;
  uint8_t* out = a_out;
  int64_t rows = rows_a;
  if (idx >= rows_a * nblk) {
    idx -= rows_a * nblk;
    in = b_in;
    out = b_out;
    rows = rows_b;
    if (idx >= rows_b * nblk) return;
  }
  const int64_t row = idx / nblk, blk = idx - row * nblk;
  const uint4 v = *reinterpret_cast<const uint4*>(in + row * ks + blk * 16);
  const uint32_t d[4] = {v.x, v.y, v.z, v.w};  // d[s]: blocks 0..3 of step s
  uint32_t o[4];
#pragma unroll
  for (int gb = 0; gb < 4; ++gb) {
    uint32_t w = 0;
#pragma unroll
    for (int t = 0; t < 4; ++t) w |= ((d[t] >> (8 * gb)) & 0xFFu) << (8 * t);
    o[gb] = w;
  }
  *reinterpret_cast<uint4*>(out + blk * rows * 16 + row * 16) = make_uint4(o[0], o[1], o[2], o[3]);
}

// Dense on the 4-wave big tile (K % 1024 == 0): one wave per SIMD, so the
// whole register file is the wave's.  MXFP8 operands come with their scales
// in the layout of scale_blocks_kernel (p.a_scale / p.b_scale point at the
// rearranged copies); per-tensor operands have none.  Persistent: workgroup
// w takes the tiles of workgroups w, w + G, w + 2G, ... (G = gridDim.x, a
// multiple of 8 when it is below the tile count), so the XCD-aware tile order
// is unchanged.  Once a tile's main loop is done, the next tile's first
// copies are issued before its epilogue, whose staging then uses stage 1 only:
// the next tile's first stage lands while this one's results are stored.
template <int FA, int FB, int EPI, int OUT, int SM = SM_MX>
__global__ __launch_bounds__(Big4::kThreads, 1) void mx_gemm4_kernel(GemmParams p) {
  using LY = Big4;
  static_assert(staged_bytes<LY>() <= LY::kStage, "the staged epilogue fits in stage 1");
  __shared__ __attribute__((aligned(1024))) uint8_t lds[LY::kLds];
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int ntm = (int)((p.M + LY::BM - 1) / LY::BM), ntn = (int)((p.N + LY::BN - 1) / LY::BN);
  const int ntiles = ntm * ntn;
  const int a_blk = (int)(p.M * 16), b_blk = (int)(p.N * 16);
  auto tile = [&](int v, int64_t& m0, int64_t& n0, Operand& A, Operand& B) __attribute__((always_inline)) {
    int tm, tn;
    raster_tile(v, ntm, ntn, tm, tn);
    m0 = (int64_t)tm * LY::BM;
    n0 = (int64_t)tn * LY::BN;
    A = make_operand(p.a, p.a_scale, m0, p.M - m0, p.K, LY::BM);
    B = make_operand(p.b, p.b_scale, n0, p.N - n0, p.K, LY::BN);
    if constexpr (SM == SM_MX) {
      // the tile's rows of every block: block blk at + blk * rows * 16 (the soffset), rows past the
      // operand's end read the next block (never stored) or zeros past the array
      const int64_t nblk = p.K / 512;
      A.scale = make_rsrc(p.a_scale + m0 * 16, (nblk * p.M - m0) * 16);
      B.scale = make_rsrc(p.b_scale + n0 * 16, (nblk * p.N - n0) * 16);
    }
  };
  int v = blockIdx.x;
  int64_t m0, n0;
  Operand A, B;
  tile(v, m0, n0, A, B);
  prologue4<SM>(lds, A, B, p.K, wave, a_blk, b_blk);
  for (;;) {
    v4f acc[LY::FRN][LY::FRM];
    mainloop4<FA, FB, SM>(lds, acc, A, B, p.K, wave, a_blk, b_blk);
    const int vn = v + (int)gridDim.x;
    int64_t m0n = 0, n0n = 0;
    Operand An = A, Bn = B;
    if (vn < ntiles) {
      tile(vn, m0n, n0n, An, Bn);
      prologue4<SM>(lds, An, Bn, p.K, wave, a_blk, b_blk);
    }
    finish_tile<LY, EPI, OUT, SM>(acc, lds + LY::kStage, p, m0, n0, wave, lane_id_fresh());
    if (vn >= ntiles) break;
    v = vn;
    m0 = m0n;
    n0 = n0n;
    A = An;
    B = Bn;
  }
}

// Grouped: a persistent grid walks the flat list of (expert row-tile,
// n-tile) pairs, built in LDS from the device-resident splits.
template <class LY, int FA, int FB, int EPI, int OUT>
__global__ __launch_bounds__(LY::kThreads) void mx_grouped_gemm_kernel(GemmParams p) {
  constexpr int BM = LY::BM, BN = LY::BN;
  __shared__ __attribute__((aligned(1024))) uint8_t lds[LY::kLds];
  __shared__ int tile_prefix[kMaxGroups + 1];
  __shared__ int64_t row_off[kMaxGroups + 1];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int G = p.groups;
  const int64_t total_m = p.M;
  // the splits are loaded all at once (one thread each), then scanned by one thread from LDS: a serial
  // pass over global memory waited on each load in turn (~4 us for 32 experts)
  for (int e = threadIdx.x; e < G; e += LY::kThreads) row_off[e + 1] = p.m_splits[e];
  __syncthreads();
  if (threadIdx.x == 0) {
    int tiles = 0;
    int64_t off = 0;
    tile_prefix[0] = 0;
    row_off[0] = 0;
    for (int e = 0; e < G; ++e) {
      int64_t me = row_off[e + 1];
      me = me < 0 ? 0 : me;
      int64_t end = off + me;
      end = end > total_m ? total_m : end;
      tiles += (int)((end - off + BM - 1) / BM);
      off = end;
      tile_prefix[e + 1] = tiles;
      row_off[e + 1] = off;
    }
  }
  __syncthreads();
  const int ntn = (int)((p.N + BN - 1) / BN);
  const int total = tile_prefix[G] * ntn;
  const int xcd = blockIdx.x % 8, slot = blockIdx.x / 8, nslots = gridDim.x / 8;
  const int chunk = (total + 7) / 8;
  const int t_end = min((xcd + 1) * chunk, total);
  for (int t = xcd * chunk + slot; t < t_end; t += nslots) {
    const int rt = t / ntn, tn = t % ntn;
    int lo = 0, hi = G;  // find e with tile_prefix[e] <= rt < tile_prefix[e + 1]
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (tile_prefix[mid] <= rt) lo = mid; else hi = mid;
    }
    const int e = lo;
    const int64_t m0 = row_off[e] + (int64_t)(rt - tile_prefix[e]) * BM;
    const int64_t m_end = row_off[e + 1];
    const int64_t n0 = (int64_t)tn * BN;
    const Operand A = make_operand(p.a, p.a_scale, m0, m_end - m0, p.K, BM);
    const Operand B = make_operand(p.b + (int64_t)e * p.N * p.K, p.b_scale + (int64_t)e * p.N * (p.K / 32), n0,
                                   p.N - n0, p.K, BN);
    v4f acc[LY::FRN][LY::FRM];
    __syncthreads();  // the previous tile's last reads of stage 0/1 are done
    mainloop<LY, FA, FB>(lds, acc, A, B, p.K, wave, lane);
    const bool has_bias = EPI == TE_EPI_BIAS || EPI == TE_EPI_BIAS_GELU_AUX;
    const uint16_t* bias = has_bias ? p.bias + (int64_t)e * p.N : nullptr;
    if constexpr (staged_epilogue(EPI, OUT))
      epilogue_lds<LY, EPI, OUT>(acc, lds, p.d, p.aux, bias, m0, m_end, n0, p.N, wave, lane);
    else
      epilogue<LY, EPI, OUT>(acc, p.d, p.aux, bias, m0, m_end, n0, p.N, wave, lane);
  }
}

// The big tile unless its grid leaves most CUs idle.  Measured on MI355X
// (256 CUs, bf16 D through the LDS-staged epilogue; big / small tile):
// 4096 x 3072 x 1024 (192 big tiles) 21.1 / 23.1 us, 4096 x 2560 x 2048
// (160) 31.2 / 34.9, 4096 x 4096 x 1024 + GELU aux (256) 30.6 / 34.3,
// 8192 x 4096 x 1024 (512) 46.9 / 55.0, but 4096 x 2048 x 1024 (128)
// 18.9 / 14.7 and 4096 x 1024 x 4096 (64) 46.9 / 31.5: below about 5/8 of a
// big tile per CU the small tile's 4x finer grid wins.
inline bool use_small_tile(int64_t big_tiles) {
  return 8 * big_tiles < 5 * (int64_t)device_cu_count();
}

// Tile configuration of a dense GEMM: SmallDeep for grids of at most one
// small tile per CU with K >= 2048 (16 or more K steps; 4096 x 1024 x 4096:
// 26.7 us against 31.5 for Small), else as above.
enum class Tile { Big, Small, SmallDeep, Big192 };

inline Tile pick_tile(int64_t M, int64_t N, int64_t K) {
  const int64_t small_tiles = ((M + 127) / 128) * ((N + 127) / 128);
  if (small_tiles <= (int64_t)device_cu_count() && K >= 2048) return Tile::SmallDeep;
  return use_small_tile(((M + 255) / 256) * ((N + 255) / 256)) ? Tile::Small : Tile::Big;
}

inline dim3 tile_grid(Tile t, int64_t M, int64_t N) {
  if (t == Tile::Big) return dim3((unsigned)(((M + 255) / 256) * ((N + 255) / 256)));
  if (t == Tile::Big192) return dim3((unsigned)(((M + 255) / 256) * ((N + 191) / 192)));
  return dim3((unsigned)(((M + 127) / 128) * ((N + 127) / 128)));
}

// The 4-wave tile instead of the 8-wave big tile: K % 1024 == 0 (the loop's
// 8-step turns) and enough K steps per CU that its faster main loop outweighs
// its single-wave prologue and epilogue: K >= 2048 and at least 32 steps per
// CU over the whole grid.  Measured on MI355X (4-wave against 8-wave, us, the
// MXFP8 path with its scale rearrangement): 4096 x 3072 x 1024 26.7 / 24.0,
// 4096 x 4096 x 1024 with GELU aux 37.2 / 30.2, 4096 x 4096 x 2048 38.2 /
// 36.6, 8192 x 8192 x 1024 82.0 / 81.8; 4096 x 4096 x 4096 59.8 / 61.9,
// 8192 x 8192 x 2048 120.5 / 132.3, 14336 x 4096 x 4096 199.5 / 224.3,
// 4096 x 4096 x 14336 170.9 / 193.5, 8192^3 386.7 / 437.9.
inline bool four_wave(int64_t M, int64_t N, int64_t K) {
  if (pick_tile(M, N, K) != Tile::Big || K % Big4::kKAlign != 0 || K < 2048) return false;
  const int64_t cus = device_cu_count(), tiles = ((M + 255) / 256) * ((N + 255) / 256);
  return (K / BK) * ((tiles + cus - 1) / cus) >= 32;
}
// The 4-wave MXFP8 path: the above, and each operand's rearranged scales fit
// 32-bit offsets.  Its workspace holds the rearranged scales of A, then
// (256-byte aligned) of B.
inline bool four_wave_mx(int64_t M, int64_t N, int64_t K) {
  const int64_t lim = ((int64_t)1 << 31) - 4096;
  return four_wave(M, N, K) && M * (K / 32) < lim && N * (K / 32) < lim;
}
// Tile of a dense MXFP8 or per-tensor GEMM (the blockwise GEMMs keep
// pick_tile: their FP32-scale modes take 128-column wave tiles): the
// 256 x 192 tile where the big-tile grid is one partial round, the 256 x 192
// grid fits in one and the 4-wave tile does not apply.
inline Tile pick_tile_dense(int64_t M, int64_t N, int64_t K) {
  const Tile t = pick_tile(M, N, K);
  if (t != Tile::Big || four_wave(M, N, K)) return t;
  const int64_t cus = device_cu_count(), rows = (M + 255) / 256;
  return rows * ((N + 255) / 256) < cus && rows * ((N + 191) / 192) <= cus ? Tile::Big192 : Tile::Big;
}
inline size_t scale_blocks_b_offset(int64_t M, int64_t K) { return (size_t)((M * (K / 32) + 255) / 256 * 256); }
inline size_t scale_blocks_bytes(int64_t M, int64_t N, int64_t K) {
  return scale_blocks_b_offset(M, K) + (size_t)(N * (K / 32));
}

inline te_status launch_scale_blocks(const uint8_t* a_scale, int64_t M, uint8_t* a_out, const uint8_t* b_scale,
                                     int64_t N, uint8_t* b_out, int64_t K, hipStream_t stream) {
  const int64_t threads = (M + N) * (K / 512);
  hipLaunchKernelGGL(scale_blocks_kernel, dim3((unsigned)((threads + 255) / 256)), dim3(256), 0, stream, a_scale, M,
                     a_out, b_scale, N, b_out, K / 32);
  return launch_status();
}

// Shape limits of the dense GEMMs beyond the divisibility rules: tile copies
// use 32-bit buffer offsets (up to 225 K bytes) and a tile's rows x K bytes
// must fit a buffer resource, so K <= 2^23; M, N and the tile count fit int.
inline bool dense_shape_ok(int64_t M, int64_t N, int64_t K) {
  return M <= ((int64_t)1 << 31) - 256 && N <= ((int64_t)1 << 31) - 256 && K <= ((int64_t)1 << 23) &&
         ((M + 127) / 128) * ((N + 127) / 128) < ((int64_t)1 << 31);
}

inline te_status check_common(const uint8_t* a, const uint8_t* a_scale, te_dtype a_fmt, const uint8_t* b,
                       const uint8_t* b_scale, te_dtype b_fmt, void* d, te_dtype d_dtype, te_epilogue epi,
                       const uint16_t* bias, uint16_t* aux, bool any_rows, bool any_k, bool allow_fp16 = false) {
  TE_REQUIRE(epi == TE_EPI_NONE || epi == TE_EPI_BIAS || epi == TE_EPI_BIAS_GELU_AUX || epi == TE_EPI_DGELU ||
                 epi == TE_EPI_ACCUMULATE,
             TE_ERR_VALUE);
  TE_REQUIRE(is_fp8(a_fmt) && is_fp8(b_fmt), TE_ERR_DTYPE);
  TE_REQUIRE(!(a_fmt == TE_E5M2 && b_fmt == TE_E5M2), TE_ERR_DTYPE);
  TE_REQUIRE(d_dtype == TE_BF16 || d_dtype == TE_FP32 || (allow_fp16 && d_dtype == TE_FP16), TE_ERR_DTYPE);
  TE_REQUIRE(epi != TE_EPI_ACCUMULATE || d_dtype == TE_FP32, TE_ERR_DTYPE);
  TE_REQUIRE((epi == TE_EPI_BIAS || epi == TE_EPI_BIAS_GELU_AUX) == (bias != nullptr), TE_ERR_NULL);
  TE_REQUIRE((epi == TE_EPI_BIAS_GELU_AUX || epi == TE_EPI_DGELU) == (aux != nullptr), TE_ERR_NULL);
  if (!any_rows) return TE_OK;
  TE_REQUIRE(d != nullptr, TE_ERR_NULL);
  TE_REQUIRE(aligned16(d), TE_ERR_ALIGN);
  if (any_k) {  // with K == 0 the operands are never read
    TE_REQUIRE(a && a_scale && b && b_scale, TE_ERR_NULL);
    TE_REQUIRE(aligned16(a) && aligned16(b), TE_ERR_ALIGN);
    TE_REQUIRE(((uintptr_t)a_scale & 3u) == 0 && ((uintptr_t)b_scale & 3u) == 0, TE_ERR_ALIGN);
  }
  TE_REQUIRE(bias == nullptr || ((uintptr_t)bias & 7u) == 0, TE_ERR_ALIGN);
  TE_REQUIRE(aux == nullptr || aligned16(aux), TE_ERR_ALIGN);
  return TE_OK;
}

}  // namespace
}  // namespace temx
