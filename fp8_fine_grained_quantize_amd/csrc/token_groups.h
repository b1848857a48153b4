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
// it needs from them with the helpers below.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fp8blk {

__device__ __forceinline__ int64_t token_groups_of(const int32_t* __restrict__ off, int64_t e) {
  const int64_t m = (int64_t)off[e + 1] - (int64_t)off[e];
  return (m + 127) / 128;
}

// token_group_owner runs in every wave independently (lane exchanges only,
// no LDS and no barrier), so each wave of a block gets the same result;
// against a block-wide LDS prefix scan (about 20 barriers per workgroup) the
// ragged 128x1 quantizer measured H [65536][2048] 108.8 -> 101.9 us and
// dOut [65536][7168] 358 -> 333 us (interleaved, one box, bitwise equal).

// A value every lane of the wave holds, moved to a scalar register (the
// compiler cannot tell that a lane-exchange result is uniform, and copy
// resources built from it must be scalar).
__device__ __forceinline__ int64_t wave_uniform(int64_t v) {
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)((uint64_t)v >> 32));
  return (int64_t)(((uint64_t)hi << 32) | lo);
}

// Inclusive sum over the wave's 64 lanes.
__device__ __forceinline__ int32_t wave_inclusive_sum(int32_t v) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int32_t u = __shfl_up(v, d);
    if (lane >= d) v += u;
  }
  return v;
}

// PG[e]: the group slot where expert e's groups start, block-wide: all NT
// threads of the block call it with the same e; `red` is NT int64 of LDS.
// (A wave-level version without LDS or barriers, as below, made the grouped
// Wgrad with FP32 output 10 % slower in an interleaved A/B on one box, BF16
// output unchanged: the barriers here stagger the workgroups' starts.)
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
// expert's groups; e = -1 when slot >= PG[G] (a surplus slot).  The wave
// walks the experts 64 at a time, one per lane, with an inclusive scan of
// their group counts.  (Loading all 256 experts' counts at once, as the
// grouped GEMM does, measured 1.5-5 % slower in the ragged 128x1 quantizer,
// bitwise identical: its many resident workgroups per CU hide the walk's
// load latency, and slots of the first experts stop after one chunk.)
__device__ __forceinline__ void token_group_owner(const int32_t* __restrict__ off, int64_t G, int64_t slot,
                                                  int64_t& e_out, int64_t& local_out) {
  const int lane = threadIdx.x & 63;
  int64_t base = 0;
  e_out = -1;
  local_out = 0;
  for (int64_t e0 = 0; e0 < G; e0 += 64) {
    const int64_t e = e0 + lane;
    const int32_t cnt = e < G ? (int32_t)token_groups_of(off, e) : 0;
    const int32_t incl = wave_inclusive_sum(cnt);
    const int64_t lo = base + incl - cnt, hi = base + incl;
    const bool mine = e < G && slot >= lo && slot < hi;
    const uint64_t who = __ballot(mine);
    if (who) {
      const int src = __ffsll((unsigned long long)who) - 1;
      e_out = wave_uniform(e0 + src);
      local_out = wave_uniform(slot - __shfl(lo, src));
      return;
    }
    base = wave_uniform(base + __shfl(incl, 63));
  }
}

}  // namespace fp8blk
