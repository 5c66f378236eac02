// te_status_str: names of the C-ABI status codes.
#include "temx_internal.h"

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
  }
  return "unknown te_status";
}
