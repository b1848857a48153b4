// Device-side building blocks shared by the libfp8blk kernels (gfx950).
//
// Citations [pN¶k] name the N-th page of the source collection and its k-th
// paragraph (p1 = xn--9g3bo1gtkw0l8ubf92bgle.kr wr_id 85187, p2 = inprokorea.com
// wr_id 735329, p5 = inprokorea.com wr_id 890463).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fp8blk {

constexpr float kE4M3Max = 448.0f;

// ---------------------------------------------------------------------------
// BF16 unpacking: a BF16 value is the upper half of a binary32 word.
// ---------------------------------------------------------------------------
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// Largest |x| over the two BF16 halves of each word, as a BF16 bit pattern in
// the low 16 bits.  Non-negative BF16 values order like their integer bits, so
// the maximum is exact integer arithmetic (NaN inputs are outside the contract).
__device__ __forceinline__ uint32_t abs_max_bits(uint32_t acc, uint32_t w) {
  const uint32_t a = w & 0x7FFF7FFFu;
  const uint32_t lo = a & 0xFFFFu, hi = a >> 16;
  return max(acc, max(lo, hi));
}

// Maximum over the 16 lanes of each DPP row (lanes 16r..16r+15): swap
// neighbours, swap pairs, mirror halves, mirror the row.  Every lane of the row
// ends with the row maximum.
__device__ __forceinline__ uint32_t row16_max(uint32_t v) {
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0xB1, 0xF, 0xF, false));   // quad_perm 1,0,3,2
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x4E, 0xF, 0xF, false));   // quad_perm 2,3,0,1
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x141, 0xF, 0xF, false));  // row_half_mirror
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x140, 0xF, 0xF, false));  // row_mirror
  return v;
}

// ---------------------------------------------------------------------------
// Tile scale.  The pages take the maximum absolute value of each 1x128 tile or
// 128x128 block online [p2¶4] and store one FP32 scale beside the codes [p1¶3];
// the E4M3 range is 448.  Default: s = fl32(amax / 448).  Power-of-two mode
// (used by the pages for some activations [p2¶4]): the smallest 2^e with
// 448 * 2^e >= amax.  amax = 0 gives s = 1.
//
// The quotient fl32(x / s) is formed one of three ways:
//   FASTDIV (BF16 inputs, default mode): r = fl32(1/s); y0 = x*r;
//          y = fma(fma(-s, y0, x), r, y0) with the sign of x.  Markstein's
//          FMA correction of a faithful quotient.  For scales in
//          [2^-100, 2^100] an exhaustive CPU check over every BF16 (x, amax)
//          pair finds it equal to IEEE x/s except below 2^-10, where every
//          value encodes to a signed zero anyway.
//   POW2:  r = 2^-e exactly (1/s a normal float): x * r is the correctly
//          rounded x / s.
//   otherwise, and for tiles outside those ranges (`slow`): IEEE division,
//          clamped to +-448.  Saturation can only happen here (a subnormal
//          scale loses precision); the hardware conversion turns values from
//          about 464 up into NaN, hence the clamp.
// ---------------------------------------------------------------------------
struct TileScale {
  float s;
  float r;
  bool slow;
};

// amax_bits: binary32 bit pattern of the (non-negative) tile maximum.
template <bool POW2, bool FASTDIV>
__device__ __forceinline__ TileScale make_scale(uint32_t amax_bits) {
  TileScale t;
  if (amax_bits == 0) {
    t.s = 1.0f; t.r = 1.0f; t.slow = !(POW2 || FASTDIV);
    return t;
  }
  if (!POW2) {
    const float amax = __uint_as_float(amax_bits);
    t.s = amax / kE4M3Max;  // IEEE division (the library is compiled with correctly rounded fp32 division)
    t.r = 1.0f / t.s;
    t.slow = !(FASTDIV && t.s >= 0x1p-100f && t.s <= 0x1p100f);
    return t;
  }
  // amax = m * 2^(E - 150) with integer significand m in [2^23, 2^24)
  // (subnormals normalised by shifting).  amax / 448 = (m / 7) * 2^(E - 156)
  // and m / 7 lies in (2^20, 2^22): it exceeds 2^21 exactly when
  // m > 7 * 2^21, so the smallest e with 448 * 2^e >= amax is
  // E - 135 + (m > 7 * 2^21).
  int E = (int)(amax_bits >> 23);
  uint32_t m = amax_bits & 0x7FFFFFu;
  if (E == 0) {
    const int sh = __builtin_clz(m) - 8;  // m in [1, 2^23) -> shift into [2^23, 2^24)
    m <<= sh;
    E = 1 - sh;
  } else {
    m |= 0x800000u;
  }
  const int e = E - 135 + (m > 7u * (1u << 21) ? 1 : 0);
  t.s = e >= -126 ? __uint_as_float((uint32_t)(e + 127) << 23) : __uint_as_float(1u << (e + 149));
  if (e >= -126 && e <= 126) {
    t.r = __uint_as_float((uint32_t)(127 - e) << 23);
    t.slow = false;
  } else {
    t.r = 0.0f;
    t.slow = true;
  }
  return t;
}

__device__ __forceinline__ float quotient_slow(float x, float s) {
  const float y = x / s;
  return fminf(fmaxf(y, -kE4M3Max), kE4M3Max);
}

// fl32(x / s) by the tile's fast formula (callers apply quotient_slow to
// tiles marked slow).
template <bool POW2, bool FASTDIV>
__device__ __forceinline__ float quotient_fast(float x, const TileScale& t) {
  if (POW2) return x * t.r;
  if (FASTDIV) {
    const float y0 = x * t.r;
    const float e = __builtin_fmaf(-t.s, y0, x);
    const float y = __builtin_fmaf(e, t.r, y0);
    return __builtin_copysignf(y, x);
  }
  return quotient_slow(x, t.s);
}

// Four binary32 values -> four E4M3 codes in one word (byte i = value i), with
// the hardware conversion (round to nearest even; inputs are within +-448
// after rounding by construction).
__device__ __forceinline__ uint32_t pack4_e4m3(float a, float b, float c, float d) {
  int w = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
  w = __builtin_amdgcn_cvt_pk_fp8_f32(c, d, w, true);
  return (uint32_t)w;
}

// Quantize the 8 BF16 values of a 16-byte chunk to 8 codes (two words).
template <bool POW2>
__device__ __forceinline__ uint2 quantize8(const uint4& v, const TileScale& t) {
  float y[8];
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    y[2 * i] = quotient_fast<POW2, true>(bf16_lo(w[i]), t);
    y[2 * i + 1] = quotient_fast<POW2, true>(bf16_hi(w[i]), t);
  }
  if (__builtin_expect(t.slow, 0)) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      y[2 * i] = quotient_slow(bf16_lo(w[i]), t.s);
      y[2 * i + 1] = quotient_slow(bf16_hi(w[i]), t.s);
    }
  }
  uint2 out;
  out.x = pack4_e4m3(y[0], y[1], y[2], y[3]);
  out.y = pack4_e4m3(y[4], y[5], y[6], y[7]);
  return out;
}

}  // namespace fp8blk
