// Library-wide entry points of libmoe_fp8 that launch no kernel.
#include "moe_fp8.h"

extern "C" int moe_abi_version(void) { return 9; }

extern "C" const char* moe_status_string(moe_status_t status) {
  switch (status) {
    case MOE_OK: return "ok";
    case MOE_INVALID_ARG: return "invalid argument";
    case MOE_UNSUPPORTED_SHAPE: return "unsupported shape or alignment";
    case MOE_HIP_ERROR: return "HIP launch error";
    case MOE_SCRATCH_LIMIT:
      return "problem larger than the allocation-free call's fixed device scratch (1 MiB)";
    default: return "unknown status";
  }
}
