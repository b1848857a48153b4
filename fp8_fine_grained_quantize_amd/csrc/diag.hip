// Diagnostic entry points.
//
// fp8blk_mfma_probe: one 16x16 tile product over 128 FP8 (E4M3) k by a
// chosen matrix-core instruction, returned raw.  The GEMMs' error model rests
// on how the matrix cores add the products inside one instruction (the pages
// describe the H800's limited tensor-core accumulation and promote partial
// sums into FP32 at a fixed K interval for that reason [p2¶3, p5¶4]); this
// call lets a test pin that behaviour on the device.
//
// fp8blk_stream_probe: a plain streaming kernel with the quantizers' traffic
// (16 bytes read, 8 written per 16-byte chunk) and no arithmetic to speak of,
// which gives the HBM rate that a kernel of this shape reaches on the device
// at a given size, the practical ceiling the quantizers are compared with.
// Citations [pN¶k]: N-th page of the source collection, k-th paragraph
// (p2 = inprokorea.com wr_id 735329, p5 = inprokorea.com wr_id 890463).
#include "host_common.h"

namespace fp8blk {

typedef int v8i_d __attribute__((ext_vector_type(8)));
typedef float v4f_d __attribute__((ext_vector_type(4)));

// One wave.  D[i][j] = sum_k dec(A[i][k]) * dec(B[j][k]); lane l holds
// D[4*(l/16) + r][l % 16], r = 0..3.
//   instr 0: one v_mfma_scale_f32_16x16x128_f8f6f4 from a zero accumulator,
//            unit (E8M0 127) scales; lane l supplies row l%16, k = 32*(l/16) .. +31.
//   instr 1: four v_mfma_f32_16x16x32_fp8_fp8, K = 32 each, chained through
//            the FP32 accumulator from zero; lane l supplies row l%16,
//            k = 32*q + 8*(l/16) .. +7 for instruction q.
__global__ __launch_bounds__(64) void k_mfma_probe(int instr, const uint8_t* __restrict__ A,
                                                   const uint8_t* __restrict__ B, float* __restrict__ C) {
  const int lane = threadIdx.x;
  const int row = lane & 15, kq = lane >> 4;
  v4f_d d = v4f_d{0.0f, 0.0f, 0.0f, 0.0f};
  if (instr == 0) {
    const uint4 a0 = *reinterpret_cast<const uint4*>(A + row * 128 + 32 * kq);
    const uint4 a1 = *reinterpret_cast<const uint4*>(A + row * 128 + 32 * kq + 16);
    const uint4 b0 = *reinterpret_cast<const uint4*>(B + row * 128 + 32 * kq);
    const uint4 b1 = *reinterpret_cast<const uint4*>(B + row * 128 + 32 * kq + 16);
    const v8i_d a = v8i_d{(int)a0.x, (int)a0.y, (int)a0.z, (int)a0.w, (int)a1.x, (int)a1.y, (int)a1.z, (int)a1.w};
    const v8i_d b = v8i_d{(int)b0.x, (int)b0.y, (int)b0.z, (int)b0.w, (int)b1.x, (int)b1.y, (int)b1.z, (int)b1.w};
    d = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, d, 0, 0, 0, 127, 0, 127);
  } else {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const long a = *reinterpret_cast<const long*>(A + row * 128 + 32 * q + 8 * kq);
      const long b = *reinterpret_cast<const long*>(B + row * 128 + 32 * q + 8 * kq);
      d = __builtin_amdgcn_mfma_f32_16x16x32_fp8_fp8(a, b, d, 0, 0, 0);
    }
  }
#pragma unroll
  for (int r = 0; r < 4; ++r) C[(4 * kq + r) * 16 + row] = d[r];
}

// Grid-stride over 16-byte chunks, two chunks in flight per lane; each chunk's
// words are folded pairwise (x ^ y, z ^ w) into the 8 bytes written, so every
// byte read is used.  Two chunks per lane and four workgroups of 256 lanes
// per compute unit measured the best of 1-8 chunks and 4-32 workgroups per
// compute unit (88 MB and 25 MB moved, rotating buffers).
__global__ __launch_bounds__(256) void k_stream_probe(const uint4* __restrict__ src, uint2* __restrict__ dst,
                                                      int64_t n) {
  constexpr int U = 2;
  const int64_t stride = (int64_t)gridDim.x * 256 * U;
  for (int64_t base = (int64_t)blockIdx.x * 256 * U + threadIdx.x; base < n; base += stride) {
    uint4 v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t i = base + (int64_t)u * 256;
      v[u] = i < n ? src[i] : make_uint4(0u, 0u, 0u, 0u);
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t i = base + (int64_t)u * 256;
      if (i < n) dst[i] = make_uint2(v[u].x ^ v[u].y, v[u].z ^ v[u].w);
    }
  }
}

}  // namespace fp8blk

using namespace fp8blk;

extern "C" fp8blk_status_t fp8blk_mfma_probe(int instr, const uint8_t* A, const uint8_t* B, float* C, void* stream) {
  if (instr != 0 && instr != 1) return FP8BLK_ERR_INVALID_ARG;
  if (A == nullptr || B == nullptr || C == nullptr || !aligned(A, 16) || !aligned(B, 16) || !aligned(C, 4))
    return FP8BLK_ERR_INVALID_ARG;
  hipLaunchKernelGGL(k_mfma_probe, dim3(1), dim3(64), 0, as_stream(stream), instr, A, B, C);
  return launch_status();
}

extern "C" fp8blk_status_t fp8blk_stream_probe(const void* src, int64_t chunks, void* dst, void* stream) {
  if (chunks < 0) return FP8BLK_ERR_INVALID_ARG;
  if (chunks == 0) return FP8BLK_OK;
  if (src == nullptr || dst == nullptr || !aligned(src, 16) || !aligned(dst, 8)) return FP8BLK_ERR_INVALID_ARG;
  int64_t grid = ceil_div(chunks, (int64_t)512);
  const int64_t cap = (int64_t)device_cus() * 4;
  if (grid > cap) grid = cap;
  hipLaunchKernelGGL(k_stream_probe, dim3((unsigned)grid), dim3(256), 0, as_stream(stream),
                     reinterpret_cast<const uint4*>(src), reinterpret_cast<uint2*>(dst), chunks);
  return launch_status();
}
