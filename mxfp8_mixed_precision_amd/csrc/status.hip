// te_status_str: names of the C-ABI status codes; the device architecture check.
#include <string.h>

#include <atomic>

#include "temx_internal.h"

namespace temx {

bool device_is_gfx950() {
  static std::atomic<int> cached[64];  // 0 unknown, 1 gfx950, 2 another target
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return false;
  int c = cached[dev].load(std::memory_order_relaxed);
  if (c == 0) {
    hipDeviceProp_t prop;
    // gcnArchName reads "gfx950" followed by its target features (":sramecc+:xnack-")
    const bool ok = hipGetDeviceProperties(&prop, dev) == hipSuccess && strncmp(prop.gcnArchName, "gfx950", 6) == 0 &&
                    (prop.gcnArchName[6] == '\0' || prop.gcnArchName[6] == ':');
    c = ok ? 1 : 2;
    cached[dev].store(c, std::memory_order_relaxed);
  }
  return c == 1;
}

}  // namespace temx

extern "C" const char* te_status_str(te_status status) {
  switch (status) {
    case TE_OK: return "TE_OK";
    case TE_ERR_NULL: return "TE_ERR_NULL: a required pointer is NULL, or an unused one is not";
    case TE_ERR_SHAPE: return "TE_ERR_SHAPE: a size violates the shape rules";
    case TE_ERR_ALIGN: return "TE_ERR_ALIGN: a pointer is not suitably aligned";
    case TE_ERR_DTYPE: return "TE_ERR_DTYPE: unsupported format or format combination";
    case TE_ERR_WORKSPACE: return "TE_ERR_WORKSPACE: workspace too small";
    case TE_ERR_HIP: return "TE_ERR_HIP: a HIP call or kernel launch failed";
    case TE_ERR_VALUE: return "TE_ERR_VALUE: an enum argument is out of range";
    case TE_ERR_ARCH: return "TE_ERR_ARCH: the current device is not a gfx950";
  }
  return "unknown te_status";
}
