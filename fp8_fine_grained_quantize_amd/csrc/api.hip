// Small host-only entry points of libfp8blk: status names, ABI version and the
// scratch-size query.
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

extern "C" int fp8blk_abi_version(void) { return 1; }

extern "C" size_t fp8blk_workspace_bytes(int64_t M, int64_t N, int64_t K, int64_t G) {
  (void)M; (void)N; (void)K; (void)G;
  return 0;
}
