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

}  // namespace temx

#define TE_REQUIRE(cond, status) \
  do {                           \
    if (!(cond)) return (status); \
  } while (0)
