// Ragged 128-token groups of MoE experts, read from device-resident offsets.
//
// The tokens routed to expert e are rows [off[e], off[e+1]) of the token
// matrix.  Quantizing them with 128x1 tiles along tokens (the Wgrad operand
// tiling [p5¶4]) inside each expert gives ceil(M_e / 128) token groups per
// expert, M_e = off[e+1] - off[e], starting at the expert's first token; the
// last one is partial when M_e is not a multiple of 128.  The groups of all
// experts are stored one after another: expert e's first group is slot
//   PG[e] = sum over e' < e of ceil(M_e' / 128),
// and its token j (0 <= j < M_e) is column 128 * PG[e] + j of the transposed
// code matrix.  The host never reads the offsets: every workgroup derives what
// it needs from them with the block-wide helpers below (all NT threads of the
// block must call them, with the same arguments).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fp8blk {

__device__ __forceinline__ int64_t token_groups_of(const int32_t* __restrict__ off, int64_t e) {
  const int64_t m = (int64_t)off[e + 1] - (int64_t)off[e];
  return (m + 127) / 128;
}

// PG[e]: the group slot where expert e's groups start.  `red` is NT int64
// of LDS.
template <int NT>
__device__ int64_t token_group_start(const int32_t* __restrict__ off, int64_t e, int64_t* red) {
  int64_t sum = 0;
  for (int64_t i = threadIdx.x; i < e; i += NT) sum += token_groups_of(off, i);
  red[threadIdx.x] = sum;
  __syncthreads();
  for (int d = NT / 2; d > 0; d >>= 1) {
    if ((int)threadIdx.x < d) red[threadIdx.x] += red[threadIdx.x + d];
    __syncthreads();
  }
  const int64_t r = red[0];
  __syncthreads();
  return r;
}

// The expert owning group slot `slot` and that slot's index within the
// expert's groups; e = -1 when slot >= PG[G] (a surplus slot).  `scan` is
// NT + 1 int64 of LDS, `found` 2 int64.  Experts are walked in chunks of NT:
// each thread counts one expert's groups and an LDS prefix sum locates the
// owner.
template <int NT>
__device__ void token_group_owner(const int32_t* __restrict__ off, int64_t G, int64_t slot, int64_t* scan,
                                  int64_t* found, int64_t& e_out, int64_t& local_out) {
  const int tid = threadIdx.x;
  int64_t base = 0;
  if (tid == 0) found[0] = -1;
  for (int64_t e0 = 0; e0 < G; e0 += NT) {
    const int64_t e = e0 + tid;
    const int64_t cnt = e < G ? token_groups_of(off, e) : 0;
    __syncthreads();
    scan[tid + 1] = cnt;
    if (tid == 0) scan[0] = 0;
    __syncthreads();
    for (int d = 1; d <= NT; d <<= 1) {  // inclusive scan of entries 1..NT
      const int64_t v = (tid + 1 - d >= 0) ? scan[tid + 1 - d] : 0;
      __syncthreads();
      if (tid + 1 - d >= 0) scan[tid + 1] += v;
      __syncthreads();
    }
    const int64_t lo = base + scan[tid], hi = base + scan[tid + 1];
    if (e < G && slot >= lo && slot < hi) {
      found[0] = e;
      found[1] = slot - lo;
    }
    const int64_t total = scan[NT];
    __syncthreads();
    if (found[0] >= 0) break;
    base += total;
  }
  e_out = found[0];
  local_out = found[1];
  __syncthreads();
}

}  // namespace fp8blk
