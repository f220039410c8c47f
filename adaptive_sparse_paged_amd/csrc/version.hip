// Library identification and status names.

#include "common.h"

extern "C" const char* sparse_version(void) { return "sparse_paged 0.1.0 (gfx950)"; }

extern "C" const char* sparse_status_string(int32_t status) {
  switch (status) {
    case SPARSE_OK: return "ok";
    case SPARSE_ERR_INVALID: return "invalid argument";
    case SPARSE_ERR_UNSUPPORTED: return "unsupported shape";
    case SPARSE_ERR_WORKSPACE: return "workspace missing or too small";
    case SPARSE_ERR_HIP: return "HIP launch failed";
    default: return "unknown status";
  }
}
