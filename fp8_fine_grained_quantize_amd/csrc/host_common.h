// Host-side argument checks and launch helpers shared by the libfp8blk entry
// points.  Every check runs before anything is enqueued.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <atomic>

#include "../../include/libfp8blk.h"

namespace fp8blk {

inline bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

// A matrix argument: pointer non-null and 16-byte aligned, pitch >= row
// length, pitch * element size a multiple of 16 bytes.  An empty matrix
// (no rows or no columns) only needs non-negative sizes.
inline bool matrix_ok(const void* p, int64_t rows, int64_t cols, int64_t pitch, int64_t elem_bytes) {
  if (rows < 0 || cols < 0 || pitch < 0) return false;
  if (rows == 0 || cols == 0) return true;
  if ((pitch * elem_bytes) % 16 != 0) return false;
  if (p == nullptr || !aligned(p, 16)) return false;
  return pitch >= cols;
}

inline bool vec_ok(const void* p, int64_t n, uintptr_t align = 4) {
  if (n < 0) return false;
  if (n == 0) return true;
  return p != nullptr && aligned(p, align);
}

inline fp8blk_status_t launch_status() {
  return hipGetLastError() == hipSuccess ? FP8BLK_OK : FP8BLK_ERR_LAUNCH;
}

inline hipStream_t as_stream(void* s) { return reinterpret_cast<hipStream_t>(s); }

inline int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

// Compute units of the current device: queried once per device and kept
// (a benign race: concurrent first calls store the same value).
inline int device_cus() {
  static std::atomic<int> cus[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  int n = cus[dev].load(std::memory_order_relaxed);
  if (n == 0) {
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
    cus[dev].store(n, std::memory_order_relaxed);
  }
  return n;
}


}  // namespace fp8blk
