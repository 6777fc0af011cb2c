// Status strings and the ABI version of the C ABI in include/tk_engram.h.
// Host code only, kept apart from the kernels: each status code is shared by
// every call, so its message names every limit that can raise it.

#include "tk_engram.h"

extern "C" {

int32_t tk_abi_version(void) { return TK_ENGRAM_ABI_VERSION; }

const char* tk_status_string(tk_status s) {
  switch (s) {
    case TK_SUCCESS:
      return "success";
    case TK_ERR_NULL:
      return "a required pointer is NULL";
    case TK_ERR_SHAPE:
      return "invalid shape: a negative count or a non-positive width or table count";
    case TK_ERR_ALIGN:
      return "a width is not a multiple of 8, or a pointer is not aligned as the call requires";
    case TK_ERR_UNSUPPORTED:
      return "a size exceeds the call's supported maximum (H or d above 8192, more than 32 "
             "tables, a batch above the hash's limit, or T above 2^31 - 1 for the gather)";
    case TK_ERR_WORKSPACE:
      return "backward workspace is smaller than required";
    case TK_ERR_LAUNCH:
      return "kernel launch failed";
    case TK_ERR_VALUE:
      return "a scalar or table parameter is out of range";
    default:
      return "unknown status";
  }
}

}  // extern "C"
