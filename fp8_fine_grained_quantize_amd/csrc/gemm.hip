// Block-scaled FP8 GEMM for gfx950: dense and grouped (per-expert).
//
//   C[m][n] = sum_g sA[g][m] * sB(g, n) * P_g[m][n],
//   P_g     = the 128-deep K group g's FP8 product.
//
// The pages apply one scale per 128-element group along K, multiply the
// scales in during dequantization [p2¶4] and promote the matrix-core partial
// sums into full-precision FP32 accumulators at a fixed K interval [p2¶3].
// Here the interval is the scale group itself: each 16x16 output tile gets one
// v_mfma_scale_f32_16x16x128_f8f6f4 per group (K = 128 in one instruction,
// starting from zero), and the FP32 result is folded into a separate FP32
// accumulator with one FMA by fl32(sA * sB).  Fprop, Dgrad and Wgrad all use
// this kernel family [p1¶3, Figure 6; p5¶4].
// Citations [pN¶k]: N-th page of the source collection, k-th paragraph
// (p1 = xn--9g3bo1gtkw0l8ubf92bgle.kr wr_id 85187, p2 = inprokorea.com wr_id
// 735329, p5 = inprokorea.com wr_id 890463).
//
// Data flow per workgroup tile (BM x BN), per K group:
//   global -> LDS directly (global_load_lds_dwordx4, 16 bytes per lane),
//     double buffered: group g+1 is copied while group g is computed; one
//     barrier per group.
//   LDS -> MFMA operands:
//     K-major tiles (A, and B stored [N][K]): two ds_read_b128 per lane;
//       16-byte chunks XOR-swizzled by row to spread LDS banks.
//     N-major tiles (B stored [K][N]): four ds_read_b64_tr_b8 per lane; each
//       16-lane group reads an 8(k) x 16(n) byte block and receives it
//       transposed, so the MFMA's B operand (32 consecutive k of one column
//       per lane) comes straight from the [K][N] layout.
//   MFMA operand layout (16x16x128, FP8): lane l holds row/column l%16 and
//   k = 32*(l/16) .. 32*(l/16)+31; result lane l holds rows 4*(l/16)+i,
//   column l%16.
#include "fp8_device.h"
#include "host_common.h"

namespace fp8blk {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef int v2i __attribute__((ext_vector_type(2)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v2i lds_v2i;
typedef __attribute__((address_space(3))) void lds_void;

template <int WAVES_M_, int WAVES_N_, int TM_, int TN_>
struct TileCfg {
  static constexpr int WAVES_M = WAVES_M_, WAVES_N = WAVES_N_, TM = TM_, TN = TN_;
  static constexpr int NW = WAVES_M * WAVES_N;
  static constexpr int NT = NW * 64;
  static constexpr int WTM = 16 * TM, WTN = 16 * TN;
  static constexpr int BM = WAVES_M * WTM, BN = WAVES_N * WTN;
  static constexpr int A_BYTES = BM * 128, B_BYTES = BN * 128;
  static constexpr int A_CHUNKS = A_BYTES / 16, B_CHUNKS = B_BYTES / 16;
  static constexpr int BUF_BYTES = A_BYTES + B_BYTES;
  static constexpr int LDS_BYTES = 2 * BUF_BYTES + 2 * BM * 4 + 2 * BN * 4;
  static_assert(WTN <= 128 && 128 % WTN == 0, "a wave's columns must lie in one 128-column scale block");
  static_assert(BN >= 128, "the N-major swizzle needs BN >= 128");
  static_assert(A_CHUNKS % (64 * NW) == 0 && B_CHUNKS % (64 * NW) == 0, "whole 1 KB copy blocks per wave");
  static_assert(BM % 64 == 0 && BN % 64 == 0, "scale copies in 64-float blocks");
};

using SmallCfg = TileCfg<2, 2, 4, 4>;  // 128 x 128 tile, 4 waves of 64 x 64
using BigCfg = TileCfg<2, 4, 8, 4>;    // 256 x 256 tile, 8 waves of 128 x 64

// --- LDS addressing -------------------------------------------------------
// K-major tile [rows][128 bytes]: 16-byte chunk c of row r lives at chunk
// c ^ ((r >> 1) & 7).
__device__ __forceinline__ int kmaj_off(int r, int c16) { return r * 128 + ((c16 ^ ((r >> 1) & 7)) << 4); }

// N-major tile [128 k][BN bytes]: 16-byte chunk m of row k lives at chunk
// m ^ (k & 7) (BN >= 128), keeping the two 8-byte halves of a chunk adjacent.
template <int BN>
__device__ __forceinline__ int nmaj_off(int k, int m16) {
  return k * BN + ((m16 ^ (k & 7)) << 4);
}

// Direct global->LDS copies.  The LDS destination of lane i is base + size*i
// (base uniform across the wave), so tile swizzles are applied by choosing,
// for each lane, the global chunk that belongs at that LDS position.
__device__ __forceinline__ void dma16(const void* src, uint8_t* lds_base) {
  __builtin_amdgcn_global_load_lds(src, (lds_void*)lds_base, 16, 0, 0);
}
__device__ __forceinline__ void dma4(const void* src, uint8_t* lds_base) {
  __builtin_amdgcn_global_load_lds(src, (lds_void*)lds_base, 4, 0, 0);
}

// Arguments of one output tile: where its operands start and how far they
// extend.  The dense kernel and the grouped kernel both build one of these.
struct TileArgs {
  const uint8_t* A;   // row 0 of this tile's row range (A + m0 * lda)
  int64_t lda;
  int64_t rows;       // valid rows from A (1..BM)
  const float* sA;    // sA + m0 (column index into the [G][M_total] table)
  int64_t sA_ld;      // M_total
  const uint8_t* B;   // B of this expert/matrix
  int64_t ldb;
  int64_t n0, N;
  const float* sB;    // scale table of this B
  int64_t sB_ld;      // row length of the scale table
  float* C;           // C + m0 * ldc
  int64_t ldc;
  int64_t K;
};

// Copy K group g of the tile's operands and scales into one LDS buffer.
// Operand rows or columns past the matrix edge are fetched from a clamped,
// valid address: they only feed output rows/columns that are never stored
// (column n of C depends only on column n of B, row m only on row m of A).
template <class CFG, bool OPB_T, bool ROW128>
__device__ __forceinline__ void issue_tile_loads(const TileArgs& t, int g, uint8_t* buf, float* sAs_buf,
                                                 float* sBs_buf) {
  constexpr int BM = CFG::BM, BN = CFG::BN, NW = CFG::NW;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t k0 = (int64_t)g * 128;
  uint8_t* As = buf;
  uint8_t* Bs = buf + CFG::A_BYTES;
#pragma unroll
  for (int it = 0; it < CFG::A_CHUNKS / (64 * NW); ++it) {
    const int blk = it * NW + wave;  // 1 KB block of the A tile
    const int ci = blk * 64 + lane;  // physical 16-byte chunk
    const int r = ci >> 3, pc = ci & 7;
    const int c = pc ^ ((r >> 1) & 7);
    const int64_t rr = r < t.rows ? r : t.rows - 1;
    dma16(t.A + rr * t.lda + k0 + c * 16, As + blk * 1024);
  }
#pragma unroll
  for (int it = 0; it < CFG::B_CHUNKS / (64 * NW); ++it) {
    const int blk = it * NW + wave;
    const int ci = blk * 64 + lane;
    if (OPB_T) {
      const int r = ci >> 3, pc = ci & 7;
      const int c = pc ^ ((r >> 1) & 7);
      const int64_t n = t.n0 + r < t.N ? t.n0 + r : t.N - 1;
      dma16(t.B + n * t.ldb + k0 + c * 16, Bs + blk * 1024);
    } else {
      constexpr int CPR = BN / 16;  // chunks per k row
      const int k = ci / CPR, pm = ci % CPR;
      const int m = pm ^ (k & 7);
      const int64_t col = t.n0 + m * 16;
      dma16(t.B + (k0 + k) * t.ldb + (col < t.N ? col : 0), Bs + blk * 1024);
    }
  }
  // scales: BM floats of sA (and BN of sB for ROW128), 64 per instruction
  if (wave == 0) {
#pragma unroll
    for (int it = 0; it < BM / 64; ++it) {
      const int64_t r = it * 64 + lane;
      dma4(t.sA + (int64_t)g * t.sA_ld + (r < t.rows ? r : t.rows - 1), (uint8_t*)(sAs_buf + it * 64));
    }
  }
  if (ROW128 && wave == NW - 1) {
#pragma unroll
    for (int it = 0; it < BN / 64; ++it) {
      const int64_t n = t.n0 + it * 64 + lane;
      dma4(t.sB + (int64_t)g * t.sB_ld + (n < t.N ? n : t.N - 1), (uint8_t*)(sBs_buf + it * 64));
    }
  }
}

template <class CFG, bool OPB_T, bool ROW128>
__device__ __forceinline__ void gemm_tile(const TileArgs& t, uint8_t* lds) {
  constexpr int BM = CFG::BM, BN = CFG::BN;
  constexpr int TM = CFG::TM, TN = CFG::TN;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave / CFG::WAVES_N, wn = wave % CFG::WAVES_N;
  const int l16 = lane & 15, lq = lane >> 4;

  float* sAs = reinterpret_cast<float*>(lds + 2 * CFG::BUF_BYTES);  // [2][BM]
  float* sBs = sAs + 2 * BM;                                          // [2][BN] (ROW128)

  const int G = (int)(t.K / 128);
  // Block-scale index of this wave's columns (uniform per wave).
  const int64_t nblk = (t.n0 + wn * CFG::WTN) / 128;
  const bool nblk_ok = nblk * 128 < t.N;

  v4f acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j) acc[i][j] = v4f{0.0f, 0.0f, 0.0f, 0.0f};

  issue_tile_loads<CFG, OPB_T, ROW128>(t, 0, lds, sAs, sBs);

  for (int g = 0; g < G; ++g) {
    const int cur = g & 1;
    // Group g has landed in buffer `cur` once every lane's copies are done,
    // and after the barrier every wave has finished reading the other buffer
    // (group g-1): start group g+1's copies into it, then compute group g.
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (g + 1 < G)
      issue_tile_loads<CFG, OPB_T, ROW128>(t, g + 1, lds + (cur ^ 1) * CFG::BUF_BYTES, sAs + (cur ^ 1) * BM,
                                           sBs + (cur ^ 1) * BN);
    __builtin_amdgcn_sched_barrier(0);

    const uint8_t* As = lds + cur * CFG::BUF_BYTES;
    const uint8_t* Bs = As + CFG::A_BYTES;

    // B scale for this group: block value (uniform) or per column.
    float sbv[TN];
    if (ROW128) {
#pragma unroll
      for (int j = 0; j < TN; ++j) sbv[j] = sBs[cur * BN + wn * CFG::WTN + 16 * j + l16];
    } else {
      const float sbb = nblk_ok ? (OPB_T ? t.sB[nblk * t.sB_ld + g] : t.sB[(int64_t)g * t.sB_ld + nblk]) : 0.0f;
#pragma unroll
      for (int j = 0; j < TN; ++j) sbv[j] = sbb;
    }

    // B fragments of this wave's TN column tiles.
    v8i bfr[TN];
#pragma unroll
    for (int j = 0; j < TN; ++j) {
      const int ncol = wn * CFG::WTN + 16 * j;  // within the tile
      if (OPB_T) {
        const int r = ncol + l16;
        const uint4 lo = *reinterpret_cast<const uint4*>(Bs + kmaj_off(r, 2 * lq));
        const uint4 hi = *reinterpret_cast<const uint4*>(Bs + kmaj_off(r, 2 * lq + 1));
        bfr[j] = v8i{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
      } else {
        const int jj = l16 >> 1, h = l16 & 1;
        v2i part[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int k = 32 * lq + 8 * r + jj;
          // 8-byte half h of 16-byte chunk (ncol/16) in row k
          const int off = nmaj_off<BN>(k, ncol >> 4) + 8 * h;
          part[r] = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_v2i*)(Bs + off));
        }
        bfr[j] = v8i{part[0][0], part[0][1], part[1][0], part[1][1], part[2][0], part[2][1], part[3][0], part[3][1]};
      }
    }

#pragma unroll
    for (int i = 0; i < TM; ++i) {
      const int r = wm * CFG::WTM + 16 * i + l16;
      const uint4 lo = *reinterpret_cast<const uint4*>(As + kmaj_off(r, 2 * lq));
      const uint4 hi = *reinterpret_cast<const uint4*>(As + kmaj_off(r, 2 * lq + 1));
      const v8i afr = v8i{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
      const float4 sa = *reinterpret_cast<const float4*>(sAs + cur * BM + wm * CFG::WTM + 16 * i + 4 * lq);
      v4f p[TN];
#pragma unroll
      for (int j = 0; j < TN; ++j)
        p[j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(afr, bfr[j], v4f{0.0f, 0.0f, 0.0f, 0.0f}, 0, 0, 0,
                                                                127, 0, 127);
#pragma unroll
      for (int j = 0; j < TN; ++j) {
        acc[i][j][0] = __builtin_fmaf(p[j][0], sa.x * sbv[j], acc[i][j][0]);
        acc[i][j][1] = __builtin_fmaf(p[j][1], sa.y * sbv[j], acc[i][j][1]);
        acc[i][j][2] = __builtin_fmaf(p[j][2], sa.z * sbv[j], acc[i][j][2]);
        acc[i][j][3] = __builtin_fmaf(p[j][3], sa.w * sbv[j], acc[i][j][3]);
      }
    }
    __builtin_amdgcn_sched_barrier(0);
  }

  // ---- epilogue: FP32 C ----
#pragma unroll
  for (int i = 0; i < TM; ++i) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int64_t row = wm * CFG::WTM + 16 * i + 4 * lq + r;
      if (row >= t.rows) continue;
#pragma unroll
      for (int j = 0; j < TN; ++j) {
        const int64_t col = t.n0 + wn * CFG::WTN + 16 * j + l16;
        if (col < t.N) t.C[row * t.ldc + col] = acc[i][j][r];
      }
    }
  }
}

// Map a linear workgroup id to a tile so that the workgroups placed on one
// XCD (ids are dealt round-robin over the 8 XCDs) cover a contiguous run of
// tiles, and consecutive tiles in a run walk down GROUP_M tile rows before
// moving right, so that A and B tiles are shared through that XCD's L2.
__device__ __forceinline__ void tile_of(int64_t bid, int64_t nblocks, int64_t tiles_m, int64_t tiles_n,
                                        int64_t& tm, int64_t& tn) {
  constexpr int XCD = 8;
  int64_t lin = bid;
  if (nblocks % XCD == 0) lin = (bid % XCD) * (nblocks / XCD) + bid / XCD;
  constexpr int64_t GROUP_M = 4;
  const int64_t per_group = GROUP_M * tiles_n;
  const int64_t grp = lin / per_group;
  const int64_t first_m = grp * GROUP_M;
  const int64_t gm = (tiles_m - first_m) < GROUP_M ? (tiles_m - first_m) : GROUP_M;
  const int64_t in = lin % per_group;
  tm = first_m + in % gm;
  tn = in / gm;
}

template <class CFG, bool OPB_T, bool ROW128>
__global__ __launch_bounds__(CFG::NT) void k_gemm(int64_t M, int64_t N, int64_t K, const uint8_t* __restrict__ A,
                                                   int64_t lda, const float* __restrict__ sA,
                                                   const uint8_t* __restrict__ B, int64_t ldb,
                                                   const float* __restrict__ sB, int64_t sB_ld,
                                                   float* __restrict__ C, int64_t ldc, int64_t tiles_m,
                                                   int64_t tiles_n) {
  extern __shared__ __align__(16) uint8_t lds[];
  int64_t tm, tn;
  tile_of(blockIdx.x, gridDim.x, tiles_m, tiles_n, tm, tn);
  const int64_t m0 = tm * CFG::BM;
  TileArgs t;
  t.A = A + m0 * lda;
  t.lda = lda;
  t.rows = (M - m0) < CFG::BM ? (M - m0) : CFG::BM;
  t.sA = sA + m0;
  t.sA_ld = M;
  t.B = B;
  t.ldb = ldb;
  t.n0 = tn * CFG::BN;
  t.N = N;
  t.sB = sB;
  t.sB_ld = sB_ld;
  t.C = C + m0 * ldc;
  t.ldc = ldc;
  t.K = K;
  gemm_tile<CFG, OPB_T, ROW128>(t, lds);
}

// Grouped: tiles are enumerated expert by expert, within an expert column
// tile by column tile, row tiles innermost, so that concurrently running
// workgroups share each expert's weight tile.  The per-expert row counts are
// read from the device-resident offsets (prefix scan in LDS), so the host
// never synchronizes; surplus workgroups of the upper-bound grid exit.
template <class CFG, bool OPB_T>
__global__ __launch_bounds__(CFG::NT) void k_grouped_gemm(int64_t G, const int32_t* __restrict__ offsets,
                                                           int64_t M_total, int64_t N, int64_t K,
                                                           const uint8_t* __restrict__ A, int64_t lda,
                                                           const float* __restrict__ sA,
                                                           const uint8_t* __restrict__ B, int64_t ldb,
                                                           int64_t strideB, const float* __restrict__ sB,
                                                           int64_t stride_sB, int64_t sB_ld,
                                                           float* __restrict__ C, int64_t ldc, int64_t tiles_n) {
  extern __shared__ __align__(16) uint8_t lds[];
  // Scan scratch lives in the (not yet used) operand buffers.
  int64_t* s_tile_base = reinterpret_cast<int64_t*>(lds);            // [NT + 1]
  int64_t* s_found = s_tile_base + CFG::NT + 1;                      // [2]
  const int tid = threadIdx.x;
  // Linear tile id with the XCD remap.
  const int64_t nblocks = gridDim.x;
  int64_t lin = blockIdx.x;
  if (nblocks % 8 == 0) lin = (lin % 8) * (nblocks / 8) + lin / 8;

  // Walk the experts in chunks of NT: each thread counts one expert's tiles,
  // an LDS prefix sum locates the expert that owns tile `lin`.
  int64_t base = 0;
  if (tid == 0) s_found[0] = -1;
  for (int64_t e0 = 0; e0 < G; e0 += CFG::NT) {
    const int64_t e = e0 + tid;
    int64_t cnt = 0;
    if (e < G) {
      const int64_t rows = (int64_t)offsets[e + 1] - (int64_t)offsets[e];
      cnt = ((rows + CFG::BM - 1) / CFG::BM) * tiles_n;
    }
    __syncthreads();
    s_tile_base[tid + 1] = cnt;
    if (tid == 0) s_tile_base[0] = 0;
    __syncthreads();
    // inclusive scan (Hillis-Steele) of entries 1..NT; entry 0 stays 0
    for (int d = 1; d <= CFG::NT; d <<= 1) {
      const int64_t v = (tid + 1 - d >= 0) ? s_tile_base[tid + 1 - d] : 0;
      __syncthreads();
      if (tid + 1 - d >= 0) s_tile_base[tid + 1] += v;
      __syncthreads();
    }
    const int64_t lo = base + s_tile_base[tid];
    const int64_t hi = base + s_tile_base[tid + 1];
    if (e < G && lin >= lo && lin < hi) {
      s_found[0] = e;
      s_found[1] = lin - lo;
    }
    const int64_t chunk_total = s_tile_base[CFG::NT];
    __syncthreads();
    if (s_found[0] >= 0) break;
    base += chunk_total;
  }
  const int64_t e = s_found[0];
  const int64_t local = s_found[1];
  __syncthreads();  // the scan scratch is about to be overwritten by tile data
  if (e < 0) return;  // surplus workgroup (uniform across the block)
  const int64_t r0 = offsets[e];
  const int64_t rows_e = (int64_t)offsets[e + 1] - r0;
  const int64_t tiles_m_e = (rows_e + CFG::BM - 1) / CFG::BM;
  const int64_t tn = local / tiles_m_e;
  const int64_t tm = local % tiles_m_e;
  const int64_t m0 = r0 + tm * CFG::BM;
  TileArgs t;
  t.A = A + m0 * lda;
  t.lda = lda;
  t.rows = (rows_e - tm * CFG::BM) < CFG::BM ? (rows_e - tm * CFG::BM) : CFG::BM;
  t.sA = sA + m0;
  t.sA_ld = M_total;
  t.B = B + e * strideB;
  t.ldb = ldb;
  t.n0 = tn * CFG::BN;
  t.N = N;
  t.sB = sB + e * stride_sB;
  t.sB_ld = sB_ld;
  t.C = C + m0 * ldc;
  t.ldc = ldc;
  t.K = K;
  gemm_tile<CFG, OPB_T, false>(t, lds);
}

// Dynamic LDS above the default limit must be allowed once per kernel; the
// call configures the function, it does not allocate.
template <class KERNEL>
static void allow_lds(KERNEL k, int bytes) {
  static const hipError_t once = hipFuncSetAttribute(reinterpret_cast<const void*>(k),
                                                     hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
  static_cast<void>(once);
}

template <class CFG, bool OPB_T, bool ROW128>
static fp8blk_status_t launch_dense(int64_t M, int64_t N, int64_t K, const uint8_t* A, int64_t lda, const float* sA,
                                    const uint8_t* B, int64_t ldb, const float* sB, int64_t sB_ld, float* C,
                                    int64_t ldc, hipStream_t stream) {
  const int64_t tiles_m = ceil_div(M, CFG::BM), tiles_n = ceil_div(N, CFG::BN);
  const int64_t blocks = tiles_m * tiles_n;
  if (blocks > 0x7FFFFFFF) return FP8BLK_ERR_UNSUPPORTED;
  auto kern = k_gemm<CFG, OPB_T, ROW128>;
  allow_lds(kern, CFG::LDS_BYTES);
  hipLaunchKernelGGL(kern, dim3((unsigned)blocks), dim3(CFG::NT), CFG::LDS_BYTES, stream, M, N, K, A, lda, sA, B,
                     ldb, sB, sB_ld, C, ldc, tiles_m, tiles_n);
  return launch_status();
}

template <class CFG>
static fp8blk_status_t dispatch_dense(bool t, bool row, int64_t M, int64_t N, int64_t K, const uint8_t* A,
                                      int64_t lda, const float* sA, const uint8_t* B, int64_t ldb, const float* sB,
                                      int64_t sB_ld, float* C, int64_t ldc, hipStream_t st) {
  if (t && row) return launch_dense<CFG, true, true>(M, N, K, A, lda, sA, B, ldb, sB, sB_ld, C, ldc, st);
  if (t) return launch_dense<CFG, true, false>(M, N, K, A, lda, sA, B, ldb, sB, sB_ld, C, ldc, st);
  if (row) return launch_dense<CFG, false, true>(M, N, K, A, lda, sA, B, ldb, sB, sB_ld, C, ldc, st);
  return launch_dense<CFG, false, false>(M, N, K, A, lda, sA, B, ldb, sB, sB_ld, C, ldc, st);
}

}  // namespace fp8blk

using namespace fp8blk;

extern "C" fp8blk_status_t fp8blk_gemm_fp8_blockscaled(int64_t M, int64_t N, int64_t K, const uint8_t* A, int64_t lda,
                                                       const float* sA, const uint8_t* B, int64_t ldb, int opB,
                                                       const float* sB, int bscale_mode, float* C, int64_t ldc,
                                                       void* workspace, size_t workspace_bytes, void* stream) {
  (void)workspace;
  (void)workspace_bytes;
  if (M < 0 || N < 0 || K < 0) return FP8BLK_ERR_INVALID_ARG;
  if (opB != FP8BLK_OP_N && opB != FP8BLK_OP_T) return FP8BLK_ERR_INVALID_ARG;
  if (bscale_mode != FP8BLK_BSCALE_BLOCK128 && bscale_mode != FP8BLK_BSCALE_ROW128) return FP8BLK_ERR_INVALID_ARG;
  if (K % 128 != 0) return FP8BLK_ERR_INVALID_ARG;
  if (M == 0 || N == 0) return FP8BLK_OK;
  if (K == 0) return FP8BLK_ERR_INVALID_ARG;
  if (!matrix_ok(A, M, K, lda, 1) || !matrix_ok(C, M, N, ldc, 4)) return FP8BLK_ERR_INVALID_ARG;
  if (opB == FP8BLK_OP_N ? !matrix_ok(B, K, N, ldb, 1) : !matrix_ok(B, N, K, ldb, 1)) return FP8BLK_ERR_INVALID_ARG;
  const int64_t G = K / 128;
  const int64_t NB = ceil_div(N, 128);
  if (!vec_ok(sA, G * M)) return FP8BLK_ERR_INVALID_ARG;
  int64_t sB_ld;
  if (bscale_mode == FP8BLK_BSCALE_ROW128) {
    if (!vec_ok(sB, G * N)) return FP8BLK_ERR_INVALID_ARG;
    sB_ld = N;
  } else {
    if (!vec_ok(sB, G * NB)) return FP8BLK_ERR_INVALID_ARG;
    sB_ld = opB == FP8BLK_OP_N ? NB : G;
  }
  hipStream_t st = as_stream(stream);
  const bool t = opB == FP8BLK_OP_T, row = bscale_mode == FP8BLK_BSCALE_ROW128;
  // 256x256 tiles when they give at least half a wave of workgroups over
  // the 256 CUs, 128x128 tiles otherwise.
  const int64_t big_tiles = ceil_div(M, BigCfg::BM) * ceil_div(N, BigCfg::BN);
  if (big_tiles >= 128)
    return dispatch_dense<BigCfg>(t, row, M, N, K, A, lda, sA, B, ldb, sB, sB_ld, C, ldc, st);
  return dispatch_dense<SmallCfg>(t, row, M, N, K, A, lda, sA, B, ldb, sB, sB_ld, C, ldc, st);
}

extern "C" fp8blk_status_t fp8blk_grouped_gemm_fp8_blockscaled(
    int64_t G, const int32_t* group_offsets, int64_t M_total, int64_t max_group_rows, int64_t N, int64_t K,
    const uint8_t* A, int64_t lda, const float* sA, const uint8_t* B, int64_t ldb, int64_t strideB, int opB,
    const float* sB, int64_t stride_sB, float* C, int64_t ldc, void* workspace, size_t workspace_bytes,
    void* stream) {
  (void)workspace;
  (void)workspace_bytes;
  using CFG = BigCfg;
  if (G < 0 || M_total < 0 || N < 0 || K < 0 || max_group_rows < 0) return FP8BLK_ERR_INVALID_ARG;
  if (opB != FP8BLK_OP_N && opB != FP8BLK_OP_T) return FP8BLK_ERR_INVALID_ARG;
  if (K % 128 != 0) return FP8BLK_ERR_INVALID_ARG;
  if (G == 0 || M_total == 0 || N == 0) return FP8BLK_OK;
  if (K == 0 || group_offsets == nullptr || !aligned(group_offsets, 4)) return FP8BLK_ERR_INVALID_ARG;
  if (!matrix_ok(A, M_total, K, lda, 1) || !matrix_ok(C, M_total, N, ldc, 4)) return FP8BLK_ERR_INVALID_ARG;
  const int64_t Gk = K / 128, NB = ceil_div(N, 128);
  const int64_t brows = opB == FP8BLK_OP_N ? K : N, bcols = opB == FP8BLK_OP_N ? N : K;
  if (!matrix_ok(B, brows, bcols, ldb, 1)) return FP8BLK_ERR_INVALID_ARG;
  if (strideB < brows * ldb || strideB % 16 != 0) return FP8BLK_ERR_INVALID_ARG;
  if (!vec_ok(sA, Gk * M_total) || !vec_ok(sB, Gk * NB)) return FP8BLK_ERR_INVALID_ARG;
  if (stride_sB < Gk * NB) return FP8BLK_ERR_INVALID_ARG;
  const int64_t sB_ld = opB == FP8BLK_OP_N ? NB : Gk;
  const int64_t tiles_n = ceil_div(N, CFG::BN);
  // Each expert adds at most one partial row tile.
  int64_t tiles_m = ceil_div(M_total, CFG::BM) + G;
  if (max_group_rows > 0) {
    const int64_t alt = G * ceil_div(max_group_rows, CFG::BM);
    if (alt < tiles_m) tiles_m = alt;
  }
  int64_t blocks = tiles_m * tiles_n;
  if (blocks == 0) return FP8BLK_OK;
  if (blocks % 8) blocks += 8 - blocks % 8;  // keep the XCD remap a bijection on the grid
  if (blocks > 0x7FFFFFFF) return FP8BLK_ERR_UNSUPPORTED;
  hipStream_t st = as_stream(stream);
  static_assert((CFG::NT + 3) * 8 <= CFG::BUF_BYTES, "scan scratch fits in the operand buffers");
  if (opB == FP8BLK_OP_T) {
    auto kern = k_grouped_gemm<CFG, true>;
    allow_lds(kern, CFG::LDS_BYTES);
    hipLaunchKernelGGL(kern, dim3((unsigned)blocks), dim3(CFG::NT), CFG::LDS_BYTES, st, G, group_offsets, M_total, N,
                       K, A, lda, sA, B, ldb, strideB, sB, stride_sB, sB_ld, C, ldc, tiles_n);
  } else {
    auto kern = k_grouped_gemm<CFG, false>;
    allow_lds(kern, CFG::LDS_BYTES);
    hipLaunchKernelGGL(kern, dim3((unsigned)blocks), dim3(CFG::NT), CFG::LDS_BYTES, st, G, group_offsets, M_total, N,
                       K, A, lda, sA, B, ldb, strideB, sB, stride_sB, sB_ld, C, ldc, tiles_n);
  }
  return launch_status();
}
