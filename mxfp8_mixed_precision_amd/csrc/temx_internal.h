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

// Enqueues the cast of blockwise FP32 scale inverses to MXFP8 E8M0 scales
// (block_scale.hip) for up to two tensors of k_blocks 128-blocks per row:
// rows_a rows from sa into out_a [rows_a, 4 k_blocks], then rows_b rows from
// sb into out_b; a_2d / b_2d select 128 x 128 blocks (one scale row per 128
// rows).  Arguments are not checked.
te_status launch_block_scale_expand(const float* sa, int64_t rows_a, int a_2d, uint8_t* out_a, const float* sb,
                                    int64_t rows_b, int b_2d, uint8_t* out_b, int64_t k_blocks,
                                    hipStream_t stream);

}  // namespace temx

#define TE_REQUIRE(cond, status) \
  do {                           \
    if (!(cond)) return (status); \
  } while (0)
