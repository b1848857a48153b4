// Online tile quantizers: BF16 -> E4M3 codes + FP32 scales (gfx950).
//
// 1x128 tiles for activations and 128x128 blocks for weights [p1¶3, the
// description of Figure 7(a)], the tile maximum taken online at quantization
// time [p2¶4]; 128x1 tiles along tokens with transposed output for the Wgrad
// operands [p5¶4].  Citations [pN¶k]: N-th page of the source collection, k-th
// paragraph (p1 = xn--9g3bo1gtkw0l8ubf92bgle.kr wr_id 85187, p2 =
// inprokorea.com wr_id 735329, p5 = inprokorea.com wr_id 890463).
//
// All three are single HBM passes: each BF16 element is read once, its code
// written once, one FP32 scale written per tile.  The tile maximum is an
// integer maximum over BF16 magnitude bits, reduced across lanes with DPP row
// operations (1x128: one 128-element tile = 16 lanes x 16 bytes = one DPP row).
#include "fp8_device.h"
#include "host_common.h"
#include "token_groups.h"

namespace fp8blk {

// Load up to 8 BF16 elements of a row chunk starting at p; `avail` elements
// remain in the row.  Elements past the row end read as +0 (no effect on the
// maximum) and are never stored.
__device__ __forceinline__ uint4 load_chunk8(const uint16_t* p, int64_t avail) {
  if (avail >= 8) return *reinterpret_cast<const uint4*>(p);
  uint32_t w[4] = {0u, 0u, 0u, 0u};
  for (int j = 0; j < 8 && j < avail; ++j) w[j >> 1] |= (uint32_t)p[j] << ((j & 1) * 16);
  return make_uint4(w[0], w[1], w[2], w[3]);
}

__device__ __forceinline__ void store_chunk8(uint8_t* p, int64_t avail, uint2 c) {
  if (avail >= 8) {
    *reinterpret_cast<uint2*>(p) = c;
    return;
  }
  for (int j = 0; j < 8 && j < avail; ++j) p[j] = (uint8_t)(((j < 4 ? c.x : c.y) >> ((j & 3) * 8)) & 0xFF);
}

__device__ __forceinline__ uint32_t chunk_abs_max(const uint4& v) {
  uint32_t a = 0;
  a = abs_max_bits(a, v.x);
  a = abs_max_bits(a, v.y);
  a = abs_max_bits(a, v.z);
  a = abs_max_bits(a, v.w);
  return a;
}

// ---------------------------------------------------------------------------
// 1x128: a workgroup of 256 lanes covers 16 * Q1_RPL rows x one 128-column
// group.  Lane (sub = tid/16, c16 = tid%16) holds bytes [16*c16, 16*c16+16)
// of the tile's 256 bytes for rows sub, sub+16, ...  Workgroups walk the
// column groups of a row band consecutively (g fastest) so that each band's
// rows are read front to back.  Two rows per lane measured 6 % faster than
// four (A [4096][7168]: 7168 workgroups instead of 3584, so the last of the
// workgroups resident at a time is a smaller share of the launch) and 10 %
// faster than eight; one row per lane was no faster than four.
// ---------------------------------------------------------------------------
constexpr int Q1_RPL = 2;

// One 1x128 workgroup's work: band `bid` of 16 * Q1_RPL rows x one column
// group, by 256 lanes numbered `tid`.
template <bool POW2>
__device__ __forceinline__ void quant_1x128_band(const uint16_t* __restrict__ x, int64_t M, int64_t K, int64_t ldx,
                                                 uint8_t* __restrict__ q, int64_t ldq, float* __restrict__ s,
                                                 int64_t G, int64_t bid, int tid) {
  constexpr int RB = 16 * Q1_RPL;  // rows per workgroup
  const int64_t g = bid % G;
  const int64_t mb = bid / G;
  const int sub = tid >> 4;
  const int c16 = tid & 15;
  const int64_t col = g * 128 + c16 * 8;
  const int64_t avail = K - col;

  uint4 v[Q1_RPL];
#pragma unroll
  for (int i = 0; i < Q1_RPL; ++i) {
    const int64_t row = mb * RB + sub + 16 * i;
    v[i] = make_uint4(0u, 0u, 0u, 0u);
    if (row < M && avail > 0) v[i] = load_chunk8(x + row * ldx + col, avail);
  }
#pragma unroll
  for (int i = 0; i < Q1_RPL; ++i) {
    const int64_t row = mb * RB + sub + 16 * i;
    const uint32_t amax = row16_max(chunk_abs_max(v[i]));  // all 16 lanes of the row active
    const TileScale ts = make_scale<POW2, true>(amax << 16);
    const uint2 codes = quantize8<POW2>(v[i], ts);
    if (row < M) {
      if (avail > 0) store_chunk8(q + row * ldq + col, avail, codes);
      if (c16 == 0) s[g * M + row] = ts.s;
    }
  }
}

template <bool POW2>
__global__ __launch_bounds__(256) void k_quant_1x128(const uint16_t* __restrict__ x, int64_t M, int64_t K,
                                                      int64_t ldx, uint8_t* __restrict__ q, int64_t ldq,
                                                      float* __restrict__ s, int64_t G) {
  quant_1x128_band<POW2>(x, M, K, ldx, q, ldq, s, G, blockIdx.x, threadIdx.x);
}

// ---------------------------------------------------------------------------
// 128x128 blocks, one block per workgroup of NT lanes: lane (sub = tid/16,
// c16 = tid%16) holds chunk c16 of rows sub, sub + NT/16, ... (2048/NT
// chunks of 8 values).  The cross-wave maximum goes through LDS.  Interior
// blocks load and store through one base pointer each.  At NT = 512 the
// kernel needs 52 VGPRs, so every workgroup of a 1792-block weight is
// resident from the start; measured against a persistent kernel that
// prefetched its next block (118 VGPRs, 4 workgroups per compute unit) with
// rotating sets on one box: 7168x4096 22.5 -> 20.6 us, 7168x2048 15.7 ->
// 13.1 us, within 3 % of a plain kernel that streams the same bytes (16 read,
// 8 written per lane step); 256 and 1024 lanes were slower.  It also replaced
// a kernel with one wave per block and the whole block in registers: 4 %
// faster at 8064 blocks, 1 % slower at 16384.
// ---------------------------------------------------------------------------
// One 128x128 block `blk` (row-major over the block grid) by NT lanes; red
// is an LDS array of NT/64 words.
template <bool POW2, int NT>
__device__ __forceinline__ void quant_block128_block(const uint16_t* __restrict__ w, int64_t R, int64_t C,
                                                     int64_t ldw, uint8_t* __restrict__ q, int64_t ldq,
                                                     float* __restrict__ s, int64_t GC, int64_t blk, uint32_t* red) {
  constexpr int CH = 2048 / NT, RSTEP = NT / 16, NWAVE = NT / 64;
  const int sub = threadIdx.x >> 4, c16 = threadIdx.x & 15;
  const int64_t bi = blk / GC, bj = blk % GC;
  const int64_t col = bj * 128 + c16 * 8;
  const bool interior = (bi + 1) * 128 <= R && (bj + 1) * 128 <= C;
  uint4 v[CH];
  if (interior) {
    const uint16_t* p = w + (bi * 128 + sub) * ldw + col;
#pragma unroll
    for (int c = 0; c < CH; ++c) v[c] = *reinterpret_cast<const uint4*>(p + (int64_t)(RSTEP * c) * ldw);
  } else {
#pragma unroll
    for (int c = 0; c < CH; ++c) {
      const int64_t row = bi * 128 + sub + RSTEP * c;
      v[c] = make_uint4(0u, 0u, 0u, 0u);
      if (row < R && col < C) v[c] = load_chunk8(w + row * ldw + col, C - col);
    }
  }
  uint32_t a = 0;
#pragma unroll
  for (int c = 0; c < CH; ++c) a = max(a, chunk_abs_max(v[c]));
  a = row16_max(a);
  a = max(a, (uint32_t)__shfl_xor((int)a, 16));
  a = max(a, (uint32_t)__shfl_xor((int)a, 32));
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = a;
  __syncthreads();
#pragma unroll
  for (int k = 0; k < NWAVE; ++k) a = max(a, red[k]);
  const TileScale ts = make_scale<POW2, true>(a << 16);
  if (interior) {
    uint8_t* o = q + (bi * 128 + sub) * ldq + col;
#pragma unroll
    for (int c = 0; c < CH; ++c) *reinterpret_cast<uint2*>(o + (int64_t)(RSTEP * c) * ldq) = quantize8<POW2>(v[c], ts);
  } else {
#pragma unroll
    for (int c = 0; c < CH; ++c) {
      const int64_t row = bi * 128 + sub + RSTEP * c;
      const uint2 codes = quantize8<POW2>(v[c], ts);
      if (row < R && col < C) store_chunk8(q + row * ldq + col, C - col, codes);
    }
  }
  if (threadIdx.x == 0) s[bi * GC + bj] = ts.s;
}

template <bool POW2, int NT>
__global__ __launch_bounds__(NT) void k_quant_block128(const uint16_t* __restrict__ w, int64_t R, int64_t C,
                                                        int64_t ldw, uint8_t* __restrict__ q, int64_t ldq,
                                                        float* __restrict__ s, int64_t GC) {
  __shared__ uint32_t red[NT / 64];
  quant_block128_block<POW2, NT>(w, R, C, ldw, q, ldq, s, GC, blockIdx.x, red);
}

// Both operands of an Fprop GEMM in one launch: workgroups [0, nW) quantize
// the weight's 128x128 blocks as above, the rest each take two 1x128 bands of
// the activation (one per 256-lane half; the 1x128 work has no barrier, so
// the halves are independent).  One launch instead of two lets the second
// tensor's loads overlap the first's stores and saves one ramp and tail.
template <bool P2A, bool P2W>
__global__ __launch_bounds__(512) void k_quant_pair(const uint16_t* __restrict__ x, int64_t M, int64_t K,
                                                     int64_t ldx, uint8_t* __restrict__ qx, int64_t ldqx,
                                                     float* __restrict__ sx, int64_t GA, int64_t nA,
                                                     const uint16_t* __restrict__ w, int64_t R, int64_t C,
                                                     int64_t ldw, uint8_t* __restrict__ qw, int64_t ldqw,
                                                     float* __restrict__ sw, int64_t GC, int64_t nW) {
  __shared__ uint32_t red[512 / 64];
  const int64_t b = blockIdx.x;
  if (b < nW) {
    quant_block128_block<P2W, 512>(w, R, C, ldw, qw, ldqw, sw, GC, b, red);
  } else {
    const int64_t band = (b - nW) * 2 + (threadIdx.x >> 8);
    if (band < nA) quant_1x128_band<P2A>(x, M, K, ldx, qx, ldqx, sx, GA, band, threadIdx.x & 255);
  }
}


// ---------------------------------------------------------------------------
// 128x1 with transposed output: one workgroup per 128 tokens x 128 channels.
// Lane (rb = tid/16, c16 = tid%16) loads tokens 8rb..8rb+7 of channels
// 8*c16..8*c16+7.  Column maxima: per lane over its 8 tokens (packed 16-bit
// max), across the 4 token groups of the wave by lane exchange, across the
// 4 waves through LDS.  Codes go through an LDS tile laid out [channel][token]
// so that the transposed rows of qT are written as contiguous 16-byte chunks.
// The tile's 8-byte segments are XOR-swizzled by channel/8 to spread banks.
// GROUPED: the tokens are split into MoE experts by device-resident offsets
// and each expert is tiled separately (ragged 128-token groups, see
// token_groups.h); workgroup row blockIdx.y is one group slot, a slot past
// the last expert's groups exits, and the tokens of a partial group beyond
// the expert's end are stored as code 0 so that the GEMM reads zeros there.
//
// The dense case uses k_quant_128x1_c64: 128 tokens x 64 channels per
// workgroup, lane (rb = tid/8, cl = tid%8) holding tokens 4rb..4rb+3 of
// channels 8cl..8cl+7; a lane's 4 codes of one channel are a 4-byte segment
// of the LDS tile, and the segments move in groups of four (XOR by a
// multiple of 4 taken from channel/8) so that the lanes of one LDS store hit
// distinct banks while each 16-byte read of the store phase stays
// contiguous.  Measured against 128 channels (rotating sets, one box): +3 %
// on X [4096][7168], +14 % on dY [4096][2048]; the grouped case keeps 128
// channels, where every workgroup scans the expert offsets and twice the
// workgroups cost 7 % on dOut [65536][7168].
// ---------------------------------------------------------------------------
constexpr int Q128X1_CW = 64;

__device__ __forceinline__ uint32_t pk_max_u16(uint32_t a, uint32_t b) {
  const uint32_t lo = max(a & 0xFFFFu, b & 0xFFFFu);
  const uint32_t hi = max(a >> 16, b >> 16);
  return lo | (hi << 16);
}

template <bool POW2, bool GROUPED>
__global__ __launch_bounds__(256) void k_quant_128x1(const uint16_t* __restrict__ x, int64_t T, int64_t C,
                                                      int64_t ldx, uint8_t* __restrict__ qT, int64_t ldqT,
                                                      float* __restrict__ s, const int32_t* __restrict__ off,
                                                      int64_t G) {
  __shared__ uint32_t red[4][16][4];
  __shared__ float sh_s[128], sh_r[128];
  __shared__ int sh_slow[128];
  __shared__ __align__(16) uint8_t tile[128 * 128];

  const int64_t c0 = (int64_t)blockIdx.x * 128;
  // Input tokens [t0, t_end) of this tile (at most 128), stored at columns
  // [o0, o_end) of qT.
  int64_t t0 = (int64_t)blockIdx.y * 128, t_end = T;
  int64_t o0 = t0, o_end = T;
  if (GROUPED) {
    int64_t e, local;
    token_group_owner(off, G, blockIdx.y, e, local);
    if (e < 0) return;  // uniform across the block
    t0 = (int64_t)off[e] + 128 * local;
    t_end = off[e + 1];
    o_end = o0 + 128;
  }
  const int tid = threadIdx.x;
  const int c16 = tid & 15;
  const int rb = tid >> 4;
  const int64_t col = c0 + c16 * 8;
  const int64_t avail = C - col;

  uint4 v[8];
  uint32_t m2[4] = {0u, 0u, 0u, 0u};
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int64_t t = t0 + rb * 8 + j;
    v[j] = make_uint4(0u, 0u, 0u, 0u);
    if (t < t_end && avail > 0) v[j] = load_chunk8(x + t * ldx + col, avail);
  }
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    m2[0] = pk_max_u16(m2[0], v[j].x & 0x7FFF7FFFu);
    m2[1] = pk_max_u16(m2[1], v[j].y & 0x7FFF7FFFu);
    m2[2] = pk_max_u16(m2[2], v[j].z & 0x7FFF7FFFu);
    m2[3] = pk_max_u16(m2[3], v[j].w & 0x7FFF7FFFu);
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    m2[i] = pk_max_u16(m2[i], (uint32_t)__shfl_xor((int)m2[i], 16));
    m2[i] = pk_max_u16(m2[i], (uint32_t)__shfl_xor((int)m2[i], 32));
  }
  if ((tid & 63) < 16) {
#pragma unroll
    for (int i = 0; i < 4; ++i) red[tid >> 6][c16][i] = m2[i];
  }
  __syncthreads();
  if (tid < 128) {
    const int c = tid, cc = c >> 3, pair = (c & 7) >> 1, half = c & 1;
    uint32_t a = 0;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const uint32_t d = red[w][cc][pair];
      a = max(a, half ? (d >> 16) : (d & 0xFFFFu));
    }
    const TileScale ts = make_scale<POW2, true>(a << 16);
    sh_s[c] = ts.s;
    sh_r[c] = ts.r;
    sh_slow[c] = ts.slow ? 1 : 0;
    if (c0 + c < C) s[(int64_t)blockIdx.y * C + c0 + c] = ts.s;
  }
  __syncthreads();
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int c = c16 * 8 + i;
    TileScale ts;
    ts.s = sh_s[c];
    ts.r = sh_r[c];
    ts.slow = sh_slow[c] != 0;
    float y[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const uint32_t wd = (i >> 1) == 0 ? v[j].x : (i >> 1) == 1 ? v[j].y : (i >> 1) == 2 ? v[j].z : v[j].w;
      const float xv = (i & 1) ? bf16_hi(wd) : bf16_lo(wd);
      y[j] = quotient_fast<POW2, true>(xv, ts);
    }
    if (__builtin_expect(ts.slow, 0)) {
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const uint32_t wd = (i >> 1) == 0 ? v[j].x : (i >> 1) == 1 ? v[j].y : (i >> 1) == 2 ? v[j].z : v[j].w;
        y[j] = quotient_slow((i & 1) ? bf16_hi(wd) : bf16_lo(wd), ts.s);
      }
    }
    uint2 codes;
    codes.x = pack4_e4m3(y[0], y[1], y[2], y[3]);
    codes.y = pack4_e4m3(y[4], y[5], y[6], y[7]);
    const int seg = rb ^ c16;  // token segment rb of channel c, swizzled by c/8
    *reinterpret_cast<uint2*>(tile + c * 128 + seg * 8) = codes;
  }
  __syncthreads();
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const int chunk = tid + 256 * k;
    const int c = chunk >> 3;
    const int part = chunk & 7;  // tokens 16*part .. 16*part+15
    if (c0 + c >= C) continue;
    const int sw = c >> 3;
    const uint2 lo = *reinterpret_cast<const uint2*>(tile + c * 128 + ((2 * part) ^ sw) * 8);
    const uint2 hi = *reinterpret_cast<const uint2*>(tile + c * 128 + ((2 * part + 1) ^ sw) * 8);
    const int64_t o = o0 + 16 * part;
    uint8_t* dst = qT + (c0 + c) * ldqT + o;
    if (o + 16 <= o_end) {
      *reinterpret_cast<uint4*>(dst) = make_uint4(lo.x, lo.y, hi.x, hi.y);
    } else {
      const uint32_t wds[4] = {lo.x, lo.y, hi.x, hi.y};
      for (int j = 0; j < 16 && o + j < o_end; ++j) dst[j] = (uint8_t)((wds[j >> 2] >> ((j & 3) * 8)) & 0xFF);
    }
  }
}

template <bool POW2>
__global__ __launch_bounds__(256) void k_quant_128x1_c64(const uint16_t* __restrict__ x, int64_t T, int64_t C,
                                                          int64_t ldx, uint8_t* __restrict__ qT, int64_t ldqT,
                                                          float* __restrict__ s) {
  constexpr int CW = Q128X1_CW, LPR = CW / 8, RB = 256 / LPR, TPL = 128 / RB;
  static_assert(TPL == 4, "4-byte token segments");
  __shared__ uint32_t red[4][LPR][4];
  __shared__ float sh_s[CW], sh_r[CW];
  __shared__ int sh_slow[CW];
  __shared__ __align__(16) uint8_t tile[CW * 128];
  const int64_t c0 = (int64_t)blockIdx.x * CW;
  const int64_t t0 = (int64_t)blockIdx.y * 128, t_end = T;
  const int64_t o0 = t0, o_end = T;
  const int tid = threadIdx.x;
  const int cl = tid % LPR;
  const int rb = tid / LPR;
  const int64_t col = c0 + cl * 8;
  const int64_t avail = C - col;
  uint4 v[TPL];
  uint32_t m2[4] = {0u, 0u, 0u, 0u};
#pragma unroll
  for (int j = 0; j < TPL; ++j) {
    const int64_t t = t0 + rb * TPL + j;
    v[j] = make_uint4(0u, 0u, 0u, 0u);
    if (t < t_end && avail > 0) v[j] = load_chunk8(x + t * ldx + col, avail);
  }
#pragma unroll
  for (int j = 0; j < TPL; ++j) {
    m2[0] = pk_max_u16(m2[0], v[j].x & 0x7FFF7FFFu);
    m2[1] = pk_max_u16(m2[1], v[j].y & 0x7FFF7FFFu);
    m2[2] = pk_max_u16(m2[2], v[j].z & 0x7FFF7FFFu);
    m2[3] = pk_max_u16(m2[3], v[j].w & 0x7FFF7FFFu);
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
#pragma unroll
    for (int d = LPR; d < 64; d <<= 1) m2[i] = pk_max_u16(m2[i], (uint32_t)__shfl_xor((int)m2[i], d));
  }
  if ((tid & 63) < LPR) {
#pragma unroll
    for (int i = 0; i < 4; ++i) red[tid >> 6][cl][i] = m2[i];
  }
  __syncthreads();
  if (tid < CW) {
    const int c = tid, cc = c >> 3, pair = (c & 7) >> 1, half = c & 1;
    uint32_t a = 0;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const uint32_t d = red[w][cc][pair];
      a = max(a, half ? (d >> 16) : (d & 0xFFFFu));
    }
    const TileScale ts = make_scale<POW2, true>(a << 16);
    sh_s[c] = ts.s;
    sh_r[c] = ts.r;
    sh_slow[c] = ts.slow ? 1 : 0;
    if (c0 + c < C) s[(int64_t)blockIdx.y * C + c0 + c] = ts.s;
  }
  __syncthreads();
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int c = cl * 8 + i;
    TileScale ts;
    ts.s = sh_s[c];
    ts.r = sh_r[c];
    ts.slow = sh_slow[c] != 0;
    float y[TPL];
#pragma unroll
    for (int j = 0; j < TPL; ++j) {
      const uint32_t wd = (i >> 1) == 0 ? v[j].x : (i >> 1) == 1 ? v[j].y : (i >> 1) == 2 ? v[j].z : v[j].w;
      y[j] = quotient_fast<POW2, true>((i & 1) ? bf16_hi(wd) : bf16_lo(wd), ts);
    }
    if (__builtin_expect(ts.slow, 0)) {
#pragma unroll
      for (int j = 0; j < TPL; ++j) {
        const uint32_t wd = (i >> 1) == 0 ? v[j].x : (i >> 1) == 1 ? v[j].y : (i >> 1) == 2 ? v[j].z : v[j].w;
        y[j] = quotient_slow((i & 1) ? bf16_hi(wd) : bf16_lo(wd), ts.s);
      }
    }
    const uint32_t codes = pack4_e4m3(y[0], y[1], y[2], y[3]);
    // 4-byte token segment rb of channel c; segments move in groups of four
    // (XOR by a multiple of 4) so a 16-byte read of the store phase stays
    // contiguous, and lanes of different cl land on different banks
    const int seg = rb ^ (4 * (cl & 7));
    *reinterpret_cast<uint32_t*>(tile + c * 128 + seg * 4) = codes;
  }
  __syncthreads();
#pragma unroll
  for (int k = 0; k < CW / 32; ++k) {
    const int chunk = tid + 256 * k;
    const int c = chunk >> 3;
    const int part = chunk & 7;  // tokens 16*part .. 16*part+15
    if (c0 + c >= C) continue;
    const uint4 w = *reinterpret_cast<const uint4*>(tile + c * 128 + (((4 * part) ^ (4 * ((c >> 3) & 7))) * 4));
    const int64_t o = o0 + 16 * part;
    uint8_t* dst = qT + (c0 + c) * ldqT + o;
    if (o + 16 <= o_end) {
      *reinterpret_cast<uint4*>(dst) = w;
    } else {
      const uint32_t wds[4] = {w.x, w.y, w.z, w.w};
      for (int j = 0; j < 16 && o + j < o_end; ++j) dst[j] = (uint8_t)((wds[j >> 2] >> ((j & 3) * 8)) & 0xFF);
    }
  }
}

// ---------------------------------------------------------------------------
// Re-quantization of a cached 1x128-quantized activation into transposed
// 128x1 tiles [p5¶4]: codes are decoded by the hardware (exact), multiplied by
// their 1x128 scale in FP32 (one rounding), and the resulting FP32 values are
// quantized along tokens exactly as k_quant_128x1 quantizes BF16 values.
// One workgroup per 128 tokens x 128 channels; the 128-channel block is also
// exactly one 1x128 scale group, so each token has one input scale here.
//
// The dequantized values are general FP32 numbers, outside the domain the
// BF16 division shortcut was checked on.  Default mode: the quotient is
// fl32(x * r), r = fl64(1 / s) formed once per column in FP64 and the product
// taken in FP64.  That equals IEEE fl32(x / s) for all FP32 x and s: with x
// and s of 24-bit significands, a quotient that is not itself a rounding
// midpoint of FP32 (in binary it never is) lies at least 2^-49 (relative)
// away from every midpoint, while the FP64 product is within 2^-52 of x / s,
// so both round to the same FP32 value.  This replaced an IEEE FP32 division
// per element that made the kernel ALU-bound.  Values past +-448 are
// possible only for a subnormal scale; a tile with one gets the clamp.
// Power-of-two scales multiply by the exact FP32 reciprocal.
// ---------------------------------------------------------------------------
typedef float v2f __attribute__((ext_vector_type(2)));

__device__ __forceinline__ uint2 load_codes8(const uint8_t* p, int64_t avail) {
  if (avail >= 8) return *reinterpret_cast<const uint2*>(p);
  uint32_t w[2] = {0u, 0u};
  for (int j = 0; j < 8 && j < avail; ++j) w[j >> 2] |= (uint32_t)p[j] << ((j & 3) * 8);
  return make_uint2(w[0], w[1]);
}

template <bool POW2>
__global__ __launch_bounds__(256) void k_requant_128x1(const uint8_t* __restrict__ q, const float* __restrict__ sq,
                                                        int64_t T, int64_t C, int64_t ldq, uint8_t* __restrict__ qT,
                                                        int64_t ldqT, float* __restrict__ sT) {
  __shared__ uint32_t red[4][16][8];
  __shared__ float sh_s[128], sh_r[128];
  __shared__ double sh_r64[128];
  __shared__ int sh_slow[128];
  __shared__ __align__(16) uint8_t tile[128 * 128];

  const int64_t c0 = (int64_t)blockIdx.x * 128;
  const int64_t t0 = (int64_t)blockIdx.y * 128;
  const int tid = threadIdx.x;
  const int c16 = tid & 15;
  const int rb = tid >> 4;
  const int64_t col = c0 + c16 * 8;
  const int64_t avail = C - col;

  float xv[8][8];  // [token j][channel i]
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int64_t t = t0 + rb * 8 + j;
    uint2 v = make_uint2(0u, 0u);
    float so = 0.0f;
    if (t < T) {
      if (avail > 0) v = load_codes8(q + t * ldq + col, avail);
      so = sq[(int64_t)blockIdx.x * T + t];
    }
    const v2f d01 = __builtin_amdgcn_cvt_pk_f32_fp8((int)v.x, false);
    const v2f d23 = __builtin_amdgcn_cvt_pk_f32_fp8((int)v.x, true);
    const v2f d45 = __builtin_amdgcn_cvt_pk_f32_fp8((int)v.y, false);
    const v2f d67 = __builtin_amdgcn_cvt_pk_f32_fp8((int)v.y, true);
    xv[j][0] = d01[0] * so; xv[j][1] = d01[1] * so;
    xv[j][2] = d23[0] * so; xv[j][3] = d23[1] * so;
    xv[j][4] = d45[0] * so; xv[j][5] = d45[1] * so;
    xv[j][6] = d67[0] * so; xv[j][7] = d67[1] * so;
  }
  uint32_t m[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    uint32_t a = 0;
#pragma unroll
    for (int j = 0; j < 8; ++j) a = max(a, __float_as_uint(xv[j][i]) & 0x7FFFFFFFu);
    a = max(a, (uint32_t)__shfl_xor((int)a, 16));
    a = max(a, (uint32_t)__shfl_xor((int)a, 32));
    m[i] = a;
  }
  if ((tid & 63) < 16) {
#pragma unroll
    for (int i = 0; i < 8; ++i) red[tid >> 6][c16][i] = m[i];
  }
  __syncthreads();
  bool slow_col = false;
  if (tid < 128) {
    const int c = tid;
    uint32_t a = 0;
#pragma unroll
    for (int w = 0; w < 4; ++w) a = max(a, red[w][c >> 3][c & 7]);
    const TileScale ts = make_scale<POW2, false>(a);
    sh_s[c] = ts.s;
    sh_r[c] = ts.r;
    if (!POW2) sh_r64[c] = 1.0 / (double)ts.s;
    sh_slow[c] = ts.slow ? 1 : 0;
    if (c0 + c < C) sT[(int64_t)blockIdx.y * C + c0 + c] = ts.s;
    slow_col = POW2 ? ts.slow : ts.s < 0x1p-126f;
  }
  const bool any_slow = __syncthreads_or(slow_col ? 1 : 0) != 0;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int c = c16 * 8 + i;
    float y[8];
    if (POW2) {
      TileScale ts;
      ts.s = sh_s[c];
      ts.r = sh_r[c];
      ts.slow = sh_slow[c] != 0;
#pragma unroll
      for (int j = 0; j < 8; ++j) y[j] = quotient_fast<true, false>(xv[j][i], ts);
      if (__builtin_expect(ts.slow, 0)) {
#pragma unroll
        for (int j = 0; j < 8; ++j) y[j] = quotient_slow(xv[j][i], ts.s);
      }
    } else {
      const double r64 = sh_r64[c];
#pragma unroll
      for (int j = 0; j < 8; ++j) y[j] = (float)((double)xv[j][i] * r64);
      if (__builtin_expect(any_slow, 0)) {
#pragma unroll
        for (int j = 0; j < 8; ++j) y[j] = fminf(fmaxf(y[j], -kE4M3Max), kE4M3Max);
      }
    }
    uint2 codes;
    codes.x = pack4_e4m3(y[0], y[1], y[2], y[3]);
    codes.y = pack4_e4m3(y[4], y[5], y[6], y[7]);
    *reinterpret_cast<uint2*>(tile + c * 128 + ((rb ^ c16) * 8)) = codes;
  }
  __syncthreads();
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const int chunk = tid + 256 * k;
    const int c = chunk >> 3;
    const int part = chunk & 7;
    if (c0 + c >= C) continue;
    const int sw = c >> 3;
    const uint2 lo = *reinterpret_cast<const uint2*>(tile + c * 128 + ((2 * part) ^ sw) * 8);
    const uint2 hi = *reinterpret_cast<const uint2*>(tile + c * 128 + ((2 * part + 1) ^ sw) * 8);
    const int64_t t = t0 + 16 * part;
    uint8_t* dst = qT + (c0 + c) * ldqT + t;
    if (t + 16 <= T) {
      *reinterpret_cast<uint4*>(dst) = make_uint4(lo.x, lo.y, hi.x, hi.y);
    } else {
      const uint32_t wds[4] = {lo.x, lo.y, hi.x, hi.y};
      for (int j = 0; j < 16 && t + j < T; ++j) dst[j] = (uint8_t)((wds[j >> 2] >> ((j & 3) * 8)) & 0xFF);
    }
  }
}

}  // namespace fp8blk

using namespace fp8blk;

extern "C" fp8blk_status_t fp8blk_quantize_1x128(const uint16_t* x, int64_t M, int64_t K, int64_t ldx, uint8_t* q,
                                                 int64_t ldq, float* s, uint32_t flags, void* stream) {
  if (flags & ~FP8BLK_SCALE_POW2) return FP8BLK_ERR_INVALID_ARG;
  if (!matrix_ok(x, M, K, ldx, 2) || !matrix_ok(q, M, K, ldq, 1)) return FP8BLK_ERR_INVALID_ARG;
  const int64_t G = ceil_div(K, 128);
  if (!vec_ok(s, G * M)) return FP8BLK_ERR_INVALID_ARG;
  if (M == 0 || K == 0) return FP8BLK_OK;
  const int64_t blocks = ceil_div(M, 16 * Q1_RPL) * G;
  if (blocks > 0x7FFFFFFF) return FP8BLK_ERR_UNSUPPORTED;
  if (flags & FP8BLK_SCALE_POW2)
    hipLaunchKernelGGL(k_quant_1x128<true>, dim3((unsigned)blocks), dim3(256), 0, as_stream(stream), x, M, K, ldx, q,
                       ldq, s, G);
  else
    hipLaunchKernelGGL(k_quant_1x128<false>, dim3((unsigned)blocks), dim3(256), 0, as_stream(stream), x, M, K, ldx,
                       q, ldq, s, G);
  return launch_status();
}

extern "C" fp8blk_status_t fp8blk_quantize_block128(const uint16_t* w, int64_t R, int64_t C, int64_t ldw,
                                                    uint8_t* q, int64_t ldq, float* s, uint32_t flags,
                                                    void* stream) {
  if (flags & ~FP8BLK_SCALE_POW2) return FP8BLK_ERR_INVALID_ARG;
  if (!matrix_ok(w, R, C, ldw, 2) || !matrix_ok(q, R, C, ldq, 1)) return FP8BLK_ERR_INVALID_ARG;
  const int64_t GR = ceil_div(R, 128), GC = ceil_div(C, 128);
  if (!vec_ok(s, GR * GC)) return FP8BLK_ERR_INVALID_ARG;
  if (R == 0 || C == 0) return FP8BLK_OK;
  constexpr int NT = 512;
  const int64_t blocks = GR * GC;
  if (blocks > 0x7FFFFFFF) return FP8BLK_ERR_UNSUPPORTED;
  if (flags & FP8BLK_SCALE_POW2)
    hipLaunchKernelGGL((k_quant_block128<true, NT>), dim3((unsigned)blocks), dim3(NT), 0, as_stream(stream), w, R, C,
                       ldw, q, ldq, s, GC);
  else
    hipLaunchKernelGGL((k_quant_block128<false, NT>), dim3((unsigned)blocks), dim3(NT), 0, as_stream(stream), w, R, C,
                       ldw, q, ldq, s, GC);
  return launch_status();
}

extern "C" fp8blk_status_t fp8blk_quantize_1x128_block128(const uint16_t* x, int64_t M, int64_t K, int64_t ldx,
                                                          uint8_t* qx, int64_t ldqx, float* sx, uint32_t xflags,
                                                          const uint16_t* w, int64_t R, int64_t C, int64_t ldw,
                                                          uint8_t* qw, int64_t ldqw, float* sw, uint32_t wflags,
                                                          void* stream) {
  if ((xflags | wflags) & ~FP8BLK_SCALE_POW2) return FP8BLK_ERR_INVALID_ARG;
  if (!matrix_ok(x, M, K, ldx, 2) || !matrix_ok(qx, M, K, ldqx, 1)) return FP8BLK_ERR_INVALID_ARG;
  if (!matrix_ok(w, R, C, ldw, 2) || !matrix_ok(qw, R, C, ldqw, 1)) return FP8BLK_ERR_INVALID_ARG;
  const int64_t GA = ceil_div(K, 128), GR = ceil_div(R, 128), GC = ceil_div(C, 128);
  if (!vec_ok(sx, GA * M) || !vec_ok(sw, GR * GC)) return FP8BLK_ERR_INVALID_ARG;
  const bool xa = M > 0 && K > 0, wa = R > 0 && C > 0;
  if (!xa && !wa) return FP8BLK_OK;
  if (!xa) return fp8blk_quantize_block128(w, R, C, ldw, qw, ldqw, sw, wflags, stream);
  if (!wa) return fp8blk_quantize_1x128(x, M, K, ldx, qx, ldqx, sx, xflags, stream);
  const int64_t nA = ceil_div(M, 16 * Q1_RPL) * GA, nW = GR * GC;
  const int64_t blocks = nW + ceil_div(nA, (int64_t)2);
  if (blocks > 0x7FFFFFFF) return FP8BLK_ERR_UNSUPPORTED;
  const bool pa = (xflags & FP8BLK_SCALE_POW2) != 0, pw = (wflags & FP8BLK_SCALE_POW2) != 0;
#define FP8BLK_PAIR_LAUNCH(PA, PW)                                                                                \
  hipLaunchKernelGGL((k_quant_pair<PA, PW>), dim3((unsigned)blocks), dim3(512), 0, as_stream(stream), x, M, K, ldx, \
                     qx, ldqx, sx, GA, nA, w, R, C, ldw, qw, ldqw, sw, GC, nW)
  if (pa) {
    if (pw) FP8BLK_PAIR_LAUNCH(true, true); else FP8BLK_PAIR_LAUNCH(true, false);
  } else {
    if (pw) FP8BLK_PAIR_LAUNCH(false, true); else FP8BLK_PAIR_LAUNCH(false, false);
  }
#undef FP8BLK_PAIR_LAUNCH
  return launch_status();
}

extern "C" fp8blk_status_t fp8blk_quantize_128x1(const uint16_t* x, int64_t T, int64_t C, int64_t ldx, uint8_t* qT,
                                                 int64_t ldqT, float* s, uint32_t flags, void* stream) {
  if (flags & ~FP8BLK_SCALE_POW2) return FP8BLK_ERR_INVALID_ARG;
  if (!matrix_ok(x, T, C, ldx, 2) || !matrix_ok(qT, C, T, ldqT, 1)) return FP8BLK_ERR_INVALID_ARG;
  const int64_t GT = ceil_div(T, 128), GC = ceil_div(C, Q128X1_CW);
  if (!vec_ok(s, GT * C)) return FP8BLK_ERR_INVALID_ARG;
  if (T == 0 || C == 0) return FP8BLK_OK;
  if (GC > 0x7FFFFFFF || GT > 65535) return FP8BLK_ERR_UNSUPPORTED;
  const dim3 grid((unsigned)GC, (unsigned)GT);
  if (flags & FP8BLK_SCALE_POW2)
    hipLaunchKernelGGL(k_quant_128x1_c64<true>, grid, dim3(256), 0, as_stream(stream), x, T, C, ldx, qT, ldqT, s);
  else
    hipLaunchKernelGGL(k_quant_128x1_c64<false>, grid, dim3(256), 0, as_stream(stream), x, T, C, ldx, qT, ldqT, s);
  return launch_status();
}

extern "C" int64_t fp8blk_token_group_slots(int64_t T, int64_t G) {
  if (T < 0 || G < 0) return 0;
  return T / 128 + G;
}

extern "C" fp8blk_status_t fp8blk_quantize_128x1_grouped(const uint16_t* x, int64_t T, int64_t C, int64_t ldx,
                                                         int64_t G, const int32_t* group_offsets, uint8_t* qT,
                                                         int64_t ldqT, float* s, uint32_t flags, void* stream) {
  if (flags & ~FP8BLK_SCALE_POW2) return FP8BLK_ERR_INVALID_ARG;
  if (T < 0 || C < 0 || G < 0 || !matrix_ok(x, T, C, ldx, 2)) return FP8BLK_ERR_INVALID_ARG;
  if (T == 0 || C == 0 || G == 0) return FP8BLK_OK;  // no groups: nothing is written
  const int64_t slots = fp8blk_token_group_slots(T, G);
  if (!matrix_ok(qT, C, 128 * slots, ldqT, 1) || !vec_ok(s, slots * C)) return FP8BLK_ERR_INVALID_ARG;
  if (group_offsets == nullptr || !aligned(group_offsets, 4)) return FP8BLK_ERR_INVALID_ARG;
  const int64_t GC = ceil_div(C, 128);
  if (GC > 0x7FFFFFFF || slots > 65535) return FP8BLK_ERR_UNSUPPORTED;
  const dim3 grid((unsigned)GC, (unsigned)slots);
  if (flags & FP8BLK_SCALE_POW2)
    hipLaunchKernelGGL((k_quant_128x1<true, true>), grid, dim3(256), 0, as_stream(stream), x, T, C, ldx, qT, ldqT, s,
                       group_offsets, G);
  else
    hipLaunchKernelGGL((k_quant_128x1<false, true>), grid, dim3(256), 0, as_stream(stream), x, T, C, ldx, qT, ldqT,
                       s, group_offsets, G);
  return launch_status();
}

extern "C" fp8blk_status_t fp8blk_requantize_128x1_from_1x128(const uint8_t* q, const float* sq, int64_t T, int64_t C,
                                                              int64_t ldq, uint8_t* qT, int64_t ldqT, float* sT,
                                                              uint32_t flags, void* stream) {
  if (flags & ~FP8BLK_SCALE_POW2) return FP8BLK_ERR_INVALID_ARG;
  if (!matrix_ok(q, T, C, ldq, 1) || !matrix_ok(qT, C, T, ldqT, 1)) return FP8BLK_ERR_INVALID_ARG;
  const int64_t GT = ceil_div(T, 128), GC = ceil_div(C, 128);
  if (!vec_ok(sq, GC * T) || !vec_ok(sT, GT * C)) return FP8BLK_ERR_INVALID_ARG;
  if (T == 0 || C == 0) return FP8BLK_OK;
  if (GC > 0x7FFFFFFF || GT > 65535) return FP8BLK_ERR_UNSUPPORTED;
  const dim3 grid((unsigned)GC, (unsigned)GT);
  if (flags & FP8BLK_SCALE_POW2)
    hipLaunchKernelGGL(k_requant_128x1<true>, grid, dim3(256), 0, as_stream(stream), q, sq, T, C, ldq, qT, ldqT, sT);
  else
    hipLaunchKernelGGL(k_requant_128x1<false>, grid, dim3(256), 0, as_stream(stream), q, sq, T, C, ldq, qT, ldqT, sT);
  return launch_status();
}
