// Host-side helpers of the C ABI: argument checks and launch-error mapping.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/temx.h"

namespace temx {

inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

inline bool is_fp8(te_dtype f) { return f == TE_E4M3 || f == TE_E5M2; }

// Status of the most recent launch on this thread.
inline te_status launch_status() {
  return hipGetLastError() == hipSuccess ? TE_OK : TE_ERR_HIP;
}

// Number of compute units of the current device (cached per device).
int device_cu_count();

// Whether the current device is a gfx950, the only target the kernels are
// built for (looked up once per device and cached).
bool device_is_gfx950();

// The blockwise FP8 GEMM in one scale mode (block_gemm_e8m0.hip,
// block_gemm_fp32.hip), after te_fp8_block_gemm has checked the arguments.
te_status launch_block_gemm_e8m0(const uint8_t* a, const float* sa, const uint8_t* b, const float* sb, int b2d,
                                 int64_t M, int64_t N, int64_t K, void* d, te_dtype d_dtype, te_epilogue epi,
                                 const uint16_t* bias, uint16_t* aux, float beta, te_dtype fa, te_dtype fb,
                                 hipStream_t stream);
te_status launch_block_gemm_fp32(const uint8_t* a, const float* sa, const uint8_t* b, const float* sb, int b2d,
                                 int64_t M, int64_t N, int64_t K, void* d, te_dtype d_dtype, te_epilogue epi,
                                 const uint16_t* bias, uint16_t* aux, float beta, te_dtype fa, te_dtype fb,
                                 hipStream_t stream);

}  // namespace temx

#define TE_REQUIRE(cond, status) \
  do {                           \
    if (!(cond)) return (status); \
  } while (0)
