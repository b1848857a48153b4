// Small host-only entry points of libfp8blk: status names and ABI version.
#include "host_common.h"

extern "C" const char* fp8blk_status_string(fp8blk_status_t status) {
  switch (status) {
    case FP8BLK_OK: return "FP8BLK_OK";
    case FP8BLK_ERR_INVALID_ARG: return "FP8BLK_ERR_INVALID_ARG";
    case FP8BLK_ERR_UNSUPPORTED: return "FP8BLK_ERR_UNSUPPORTED";
    case FP8BLK_ERR_LAUNCH: return "FP8BLK_ERR_LAUNCH";
  }
  return "FP8BLK_UNKNOWN_STATUS";
}

extern "C" int fp8blk_abi_version(void) { return 6; }

