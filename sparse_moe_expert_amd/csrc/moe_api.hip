// Library-wide host pieces of the C ABI: status strings and the cached
// device query used to size persistent grids.
#include "moe_common.h"

namespace moe {

int device_cu_count() {
  static int cached[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return 0;
  if (dev < 64 && cached[dev] > 0) return cached[dev];
  int cus = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
  if (dev < 64) cached[dev] = cus;
  return cus;
}

}  // namespace moe

extern "C" const char* moe_status_string(moe_status s) {
  switch (s) {
    case MOE_OK: return "ok";
    case MOE_ERR_NULL_POINTER: return "a required pointer is NULL";
    case MOE_ERR_INVALID_SHAPE: return "invalid shape (need T >= 0, 1 <= k <= E, H and I multiples of 32)";
    case MOE_ERR_UNSUPPORTED: return "shape outside the supported envelope";
    case MOE_ERR_MISALIGNED: return "a tensor pointer is not 16-byte aligned";
    case MOE_ERR_WORKSPACE_TOO_SMALL: return "workspace smaller than moe_expert_ffn_workspace_size()";
    case MOE_ERR_HIP: return "HIP runtime error (launch or device query)";
    case MOE_ERR_SCRATCH_TOO_SMALL:
      return "sizes need more workspace than moe_step_noalloc's static scratch (MOE_NOALLOC_SCRATCH_BYTES)";
  }
  return "unknown status";
}
