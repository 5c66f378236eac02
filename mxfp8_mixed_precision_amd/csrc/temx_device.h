// Device-side helpers shared by the gfx950 kernels of the MXFP8 Linear path.
//
// Encoding conventions (OCP FP8 / OCP MX, the readings stated in temx.h):
// E4M3 "FN" (max 448), E5M2 (max 57344), E8M0 scale code
// max(biased_exp(amax) - emax, 0), saturating round-to-nearest-even.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "temx_internal.h"

namespace temx {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef short v2s __attribute__((ext_vector_type(2)));
typedef __bf16 v2bf __attribute__((ext_vector_type(2)));

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(1))) void global_void_t;

// 16-byte streaming load (non-temporal: the data is read once).
__device__ __forceinline__ uint4 load_nt16(const void* p) {
  const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
  return make_uint4(v[0], v[1], v[2], v[3]);
}

// Streaming stores (non-temporal: the output is not read again by this kernel).
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ void store_nt16(void* p, uint4 v) {
  __builtin_nontemporal_store(u32x4{v.x, v.y, v.z, v.w}, reinterpret_cast<u32x4*>(p));
}
__device__ __forceinline__ void store_nt8(void* p, uint2 v) {
  __builtin_nontemporal_store(u32x2{v.x, v.y}, reinterpret_cast<u32x2*>(p));
}

// Exponent of the largest finite value of the element format.
template <int FMT> struct FmtTraits;
template <> struct FmtTraits<TE_E4M3> {
  static constexpr int emax = 8;
  static constexpr float max_value = 448.0f;
  static constexpr uint32_t overflow_code = 0x7F;  // what the hardware convert gives past the max
};
template <> struct FmtTraits<TE_E5M2> {
  static constexpr int emax = 15;
  static constexpr float max_value = 57344.0f;
  static constexpr uint32_t overflow_code = 0x7C;
};

// E8M0 code of a 32-block from the bit pattern of its amax (|x| bits, 0..0x7FFF).
// Non-finite blocks (amax bits >= 0x7F80) get 255.
template <int FMT>
__device__ __forceinline__ uint32_t e8m0_code_from_amax_bits(uint32_t amax_bits) {
  int bexp = (int)(amax_bits >> 7);
  int code = bexp - FmtTraits<FMT>::emax;
  code = code < 0 ? 0 : code;
  return amax_bits >= 0x7F80u ? 255u : (uint32_t)code;
}

// 2^(code - 127) as an fp32 bit pattern, for code in [0, 254]
// (code 0 is the subnormal 2^-127).
__device__ __forceinline__ float e8m0_to_float(uint32_t code) {
  uint32_t bits = code == 0 ? 0x00400000u : (code << 23);
  return __uint_as_float(bits);
}

// E8M0 code of the smallest E8M0 value >= s (the cast of an FP32 block
// scale inverse): saturates at 2^127 (+inf included); +-0 and positive values
// up to 2^-127 give code 0 (2^-127); NaN and negative values give 255.
// Selects only, no branches: it runs inside the GEMM's MFMA loop.
__device__ __forceinline__ uint32_t e8m0_at_least(float s) {
  const uint32_t u = __float_as_uint(s);
  const uint32_t mag = u & 0x7FFFFFFFu;
  const uint32_t e = mag >> 23, m = mag & 0x7FFFFFu;
  // above 2^(e-127) rounds up; a subnormal rounds up only past 2^-127 (m = 0x400000)
  const uint32_t c = min(e + (m > (e == 0 ? 0x400000u : 0u) ? 1u : 0u), 254u);
  const bool bad = mag > 0x7F800000u || (u != mag && mag != 0);  // NaN, or negative non-zero
  return bad ? 255u : c;
}

// Byte-wise saturation fix-up: the hardware converts give 0x7F (E4M3 NaN) or
// 0x7C (E5M2 Inf) with the sign bit for magnitudes past the largest finite
// value; those bytes are replaced by the largest finite code (one less).
template <int FMT>
__device__ __forceinline__ uint32_t saturate_bytes(uint32_t q) {
  constexpr uint32_t ov = FmtTraits<FMT>::overflow_code * 0x01010101u;
  uint32_t t = (q & 0x7F7F7F7Fu) ^ ov;                    // zero byte <=> overflow code
  uint32_t nonzero = ((t + 0x7F7F7F7Fu) | t) & 0x80808080u;  // bit 7 set <=> byte != 0
  uint32_t hit = (~nonzero) & 0x80808080u;
  return q - (hit >> 7);
}

// Four bf16 pairs (8 elements) -> 8 codes, dividing by the power-of-two scale.
template <int FMT>
__device__ __forceinline__ uint2 cvt8_scaled(uint4 x, float scale) {
  v2s lo = {0, 0}, hi = {0, 0};
  if constexpr (FMT == TE_E4M3) {
    lo = __builtin_amdgcn_cvt_scalef32_pk_fp8_bf16(lo, __builtin_bit_cast(v2bf, x.x), scale, false);
    lo = __builtin_amdgcn_cvt_scalef32_pk_fp8_bf16(lo, __builtin_bit_cast(v2bf, x.y), scale, true);
    hi = __builtin_amdgcn_cvt_scalef32_pk_fp8_bf16(hi, __builtin_bit_cast(v2bf, x.z), scale, false);
    hi = __builtin_amdgcn_cvt_scalef32_pk_fp8_bf16(hi, __builtin_bit_cast(v2bf, x.w), scale, true);
  } else {
    lo = __builtin_amdgcn_cvt_scalef32_pk_bf8_bf16(lo, __builtin_bit_cast(v2bf, x.x), scale, false);
    lo = __builtin_amdgcn_cvt_scalef32_pk_bf8_bf16(lo, __builtin_bit_cast(v2bf, x.y), scale, true);
    hi = __builtin_amdgcn_cvt_scalef32_pk_bf8_bf16(hi, __builtin_bit_cast(v2bf, x.z), scale, false);
    hi = __builtin_amdgcn_cvt_scalef32_pk_bf8_bf16(hi, __builtin_bit_cast(v2bf, x.w), scale, true);
  }
  uint2 r;
  r.x = saturate_bytes<FMT>(__builtin_bit_cast(uint32_t, lo));
  r.y = saturate_bytes<FMT>(__builtin_bit_cast(uint32_t, hi));
  return r;
}

// Max of |x| bit patterns over 8 bf16 values, as a 15-bit integer
// (for non-NaN values the integer order of |x| bits is the magnitude order).
typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t absmax_bits8(uint4 x) {
  u16x2 a = __builtin_bit_cast(u16x2, x.x & 0x7FFF7FFFu), b = __builtin_bit_cast(u16x2, x.y & 0x7FFF7FFFu);
  u16x2 c = __builtin_bit_cast(u16x2, x.z & 0x7FFF7FFFu), d = __builtin_bit_cast(u16x2, x.w & 0x7FFF7FFFu);
  u16x2 m = __builtin_elementwise_max(__builtin_elementwise_max(a, b), __builtin_elementwise_max(c, d));
  return max((uint32_t)m[0], (uint32_t)m[1]);
}

// Max across the 4 lanes of a DPP quad (lanes 4q .. 4q+3).
__device__ __forceinline__ uint32_t quad_max(uint32_t v) {
  // quad_perm [1,0,3,2] then [2,3,0,1]
  uint32_t t = (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0xB1, 0xF, 0xF, false);
  v = max(v, t);
  t = (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x4E, 0xF, 0xF, false);
  return max(v, t);
}

// Round-to-nearest-even fp32 -> bf16 of two values, packed (lo = a).
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  v2bf r = {(__bf16)a, (__bf16)b};
  return __builtin_bit_cast(uint32_t, r);
}

__device__ __forceinline__ float bf16_bits_to_float(uint32_t h) { return __uint_as_float(h << 16); }

// Round-to-nearest-even fp32 -> IEEE half of two values, packed (lo = a);
// magnitudes beyond the half range become +-inf.
typedef _Float16 v2h __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack_f16x2(float a, float b) {
  v2h r = {(_Float16)a, (_Float16)b};
  return __builtin_bit_cast(uint32_t, r);
}

// GELU, tanh form: 0.5 x (1 + tanh(u)) with u = sqrt(2/pi) (x + 0.044715 x^3),
// evaluated as x / (1 + 2^(-2 u log2 e)) (the same function; no cancellation
// for negative x).
__device__ __forceinline__ float gelu_tanh(float x) {
  constexpr float kC = -2.0f * 0.7978845608028654f * 1.4426950408889634f;  // -2 sqrt(2/pi) log2(e)
  float t = x * (kC + (kC * 0.044715f) * (x * x));
  float e = __builtin_amdgcn_exp2f(t);
  return x * __builtin_amdgcn_rcpf(1.0f + e);
}

// d/dx gelu_tanh(x) = s + 2 x s (1 - s) u' with s = 1 / (1 + e), e = 2^(-2 u log2 e)
// and u' = sqrt(2/pi) (1 + 3 * 0.044715 x^2).  s (1 - s) is evaluated as
// 1 / (2 + e + 1/e): no cancellation as s -> 0 or 1, and the right limit 0
// when e overflows or underflows (the derivative then keeps its relative
// accuracy down to where it leaves the fp32 range).  The product term is
// taken as 0 once that factor is 0, so huge |x| (x^2 = inf) cannot give 0 * inf.
__device__ __forceinline__ float dgelu_tanh(float x) {
  constexpr float kC = -2.0f * 0.7978845608028654f * 1.4426950408889634f;  // -2 sqrt(2/pi) log2(e)
  constexpr float kK = 0.7978845608028654f;                                 // sqrt(2/pi)
  const float x2 = x * x;
  const float e = __builtin_amdgcn_exp2f(x * (kC + (kC * 0.044715f) * x2));
  const float s = __builtin_amdgcn_rcpf(1.0f + e);
  const float sd = __builtin_amdgcn_rcpf(2.0f + e + __builtin_amdgcn_rcpf(e));
  const float t = 2.0f * x * sd * (kK + (kK * 3.0f * 0.044715f) * x2);
  return s + (sd == 0.0f ? 0.0f : t);
}

}  // namespace temx
