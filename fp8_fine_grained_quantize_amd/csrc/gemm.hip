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

// Workgroup tile: WAVES_M x WAVES_N waves, each owning TM x TN MFMA tiles of
// 16x16; STAGES LDS buffers in the copy pipeline (group g+STAGES-1 is in
// flight while group g is computed).
template <int WAVES_M_, int WAVES_N_, int TM_, int TN_, int STAGES_>
struct TileCfg {
  static constexpr int WAVES_M = WAVES_M_, WAVES_N = WAVES_N_, TM = TM_, TN = TN_, STAGES = STAGES_;
  static constexpr int NW = WAVES_M * WAVES_N;
  static constexpr int NT = NW * 64;
  static constexpr int WTM = 16 * TM, WTN = 16 * TN;
  static constexpr int BM = WAVES_M * WTM, BN = WAVES_N * WTN;
  static constexpr int A_BYTES = BM * 128, B_BYTES = BN * 128;
  static constexpr int A_CHUNKS = A_BYTES / 16, B_CHUNKS = B_BYTES / 16;
  static constexpr int A_ITERS = A_CHUNKS / (64 * NW), B_ITERS = B_CHUNKS / (64 * NW);
  // Scale copies: BM floats of sA then BN floats of sB, 64 floats per wave
  // instruction, spread so that every wave issues the same number of copies.
  static constexpr int S_BLOCKS = (BM + BN) / 64;
  static constexpr int S_ITERS = (S_BLOCKS + NW - 1) / NW;
  static constexpr int LOADS_PER_STAGE = A_ITERS + B_ITERS + S_ITERS;  // per wave
  static constexpr int BUF_BYTES = A_BYTES + B_BYTES;
  static constexpr int LDS_BYTES = STAGES * (BUF_BYTES + BM * 4 + BN * 4);
  static_assert(WTN <= 128 && 128 % WTN == 0, "a wave's columns must lie in one 128-column scale block");
  static_assert(BN >= 128, "the N-major swizzle needs BN >= 128");
  static_assert(A_CHUNKS % (64 * NW) == 0 && B_CHUNKS % (64 * NW) == 0, "whole 1 KB copy blocks per wave");
  static_assert(BM % 64 == 0 && BN % 64 == 0, "scale copies in 64-float blocks");
  static_assert(STAGES >= 2, "at least double buffering");
  static_assert((STAGES - 2) * LOADS_PER_STAGE <= 63, "vmcnt range");
  static_assert(LDS_BYTES <= 160 * 1024, "LDS capacity");
};

#ifndef FP8BLK_BIG_CFG
#define FP8BLK_BIG_CFG 2, 4, 8, 4, 2  // 256 x 256 tile, 8 waves of 128 x 64, double buffered
#endif
#ifndef FP8BLK_SMALL_CFG
#define FP8BLK_SMALL_CFG 2, 2, 4, 4, 2  // 128 x 128 tile, 4 waves of 64 x 64
#endif
using BigCfg = TileCfg<FP8BLK_BIG_CFG>;
using SmallCfg = TileCfg<FP8BLK_SMALL_CFG>;

// s_waitcnt with vmcnt = N and no wait on the other counters (gfx9 encoding:
// vmcnt in bits 3:0 and 15:14, expcnt 6:4, lgkmcnt 11:8).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N <= 63, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

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

// Direct global->LDS copies through buffer resources: buffer_load_dwordx4
// (or _dword) with the lds modifier writes lane i's data at M0 + size*i, M0
// uniform across the wave.  Tile swizzles are applied by choosing, for each
// lane, the global chunk that belongs at its LDS position.  One per-lane
// offset per operand is computed once per tile; successive copies of a group
// differ by a scalar offset, and each K group only moves the scalar resource
// base, so copies cost no vector arithmetic inside the K loop.
//
// Each resource's record count ends at the last valid byte of the operand
// slab it covers: chunks of rows (or, for [K][N] B, of the final row) beyond
// the matrix edge are out of range and read as zero.  Such rows and columns
// only feed output rows/columns that are never stored (column n of C depends
// only on column n of B, row m only on row m of A), as do the padding
// columns of a [K][N] B tile that runs past N.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc_of(const void* base, int64_t bytes) {
  const int32_t n = bytes > 0x7FFFFFFF ? 0x7FFFFFFF : (bytes < 0 ? 0 : (int32_t)bytes);
  // raw buffer (stride 0); 0x00020000 = gfx9 raw-buffer descriptor word 3
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, n, 0x00020000);
}
__device__ __forceinline__ void dma16(__amdgpu_buffer_rsrc_t r, uint32_t voff, int32_t soff, uint8_t* lds_base) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void*)lds_base, 16, voff, soff, 0, 0);
}
__device__ __forceinline__ void dma4(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint8_t* lds_base) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void*)lds_base, 4, voff, 0, 0, 0);
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

// Copies of one K group.  Group bases: A tile A + k0; B tile B + n0*ldb + k0
// ([N][K]) or B + k0*ldb + n0 ([K][N]); scales sA + g*ld and sB + g*ld + n0.
// The sA copy is permuted so that each lane later reads the TM row scales it
// needs (rows 16*i + lane%16 of its wave's rows) as one contiguous run.
template <class CFG, bool OPB_T, bool ROW128>
struct CopyPlan {
  static constexpr int NW = CFG::NW, BM = CFG::BM, BN = CFG::BN;
  static_assert(CFG::S_ITERS == 1, "one scale copy per wave");
  // [K][N] B tile: BN/16 chunks per k row, so one copy iteration advances k
  // by KSTEP rows; the row swizzle (k & 7) must repeat across iterations.
  static constexpr int KSTEP = NW * 64 / (BN / 16);
  static_assert(KSTEP % 8 == 0, "[K][N] copies keep the row swizzle across iterations");
  uint32_t a, b, sc;
  bool sc_is_b;  // uniform per wave

  __device__ __forceinline__ void init(const TileArgs& t) {
    constexpr int TM = CFG::TM, WTM = CFG::WTM;
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    {  // A and [N][K] B: chunk ci = (it*NW + wave)*64 + lane; row ci/8 advances by 8*NW per it
      const int ci = wave * 64 + lane;
      const int r = ci >> 3, c = (ci & 7) ^ ((r >> 1) & 7);
      a = (uint32_t)(r * t.lda + c * 16);
      if (OPB_T) b = (uint32_t)(r * t.ldb + c * 16);
    }
    if (!OPB_T) {  // [K][N] B: BN/16 chunks per k row; k advances by KSTEP per it
      constexpr int CPR = BN / 16;
      const int ci = wave * 64 + lane;
      const int k = ci / CPR, m = (ci % CPR) ^ (k & 7);
      b = (uint32_t)(k * t.ldb + m * 16);
    }
    int blk = wave;
    if (blk >= CFG::S_BLOCKS) blk = 0;  // surplus copy: rewrites block 0 with the same data
    const int p = blk * 64 + lane;      // float position in the [BM + BN] scale buffer
    if (p < BM) {
      const int w = p / WTM, q = p % WTM;
      sc = (uint32_t)((w * WTM + 16 * (q % TM) + q / TM) * 4);
      sc_is_b = false;
    } else {
      sc = ROW128 ? (uint32_t)((p - BM) * 4) : 0u;  // block-scale mode: the half is unused
      sc_is_b = ROW128;
    }
  }

  __device__ __forceinline__ void issue(const TileArgs& t, int g, uint8_t* buf, float* sbuf) const {
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int64_t k0 = (int64_t)g * 128;
    const __amdgpu_buffer_rsrc_t ra = rsrc_of(t.A + k0, (t.rows - 1) * t.lda + 128);
    __amdgpu_buffer_rsrc_t rb;
    if (OPB_T) {
      const int64_t nvalid = t.N - t.n0 < BN ? t.N - t.n0 : BN;
      rb = rsrc_of(t.B + t.n0 * t.ldb + k0, (nvalid - 1) * t.ldb + 128);
    } else {
      rb = rsrc_of(t.B + k0 * t.ldb + t.n0, (t.K - k0) * t.ldb - t.n0);
    }
    const __amdgpu_buffer_rsrc_t rsa = rsrc_of(t.sA + (int64_t)g * t.sA_ld, t.rows * 4);
    const __amdgpu_buffer_rsrc_t rsb =
        rsrc_of(t.sB + (int64_t)g * t.sB_ld + (ROW128 ? t.n0 : 0), ROW128 ? (t.N - t.n0) * 4 : 4);
#pragma unroll
    for (int it = 0; it < CFG::A_ITERS; ++it)
      dma16(ra, a, (int32_t)(it * 8 * NW * t.lda), buf + (it * NW + wave) * 1024);
#pragma unroll
    for (int it = 0; it < CFG::B_ITERS; ++it) {
      const int32_t so = OPB_T ? (int32_t)(it * 8 * NW * t.ldb) : (int32_t)(it * KSTEP * t.ldb);
      dma16(rb, b, so, buf + CFG::A_BYTES + (it * NW + wave) * 1024);
    }
    const int blk = wave < CFG::S_BLOCKS ? wave : 0;
    dma4(sc_is_b ? rsb : rsa, sc, (uint8_t*)(sbuf + blk * 64));
  }
};

template <class CFG, bool OPB_T, bool ROW128>
__device__ __forceinline__ void gemm_tile(const TileArgs& t, uint8_t* lds) {
  constexpr int BM = CFG::BM, BN = CFG::BN;
  constexpr int TM = CFG::TM, TN = CFG::TN;
  constexpr int S = CFG::STAGES;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave / CFG::WAVES_N, wn = wave % CFG::WAVES_N;
  const int l16 = lane & 15, lq = lane >> 4;

  // LDS: S operand buffers, then S scale buffers of BM + BN floats.
  float* sbase = reinterpret_cast<float*>(lds + S * CFG::BUF_BYTES);

  const int G = (int)(t.K / 128);
  // Block-scale index of this wave's columns (uniform per wave).
  const int64_t nblk = (t.n0 + wn * CFG::WTN) / 128;
  const bool nblk_ok = nblk * 128 < t.N;

  CopyPlan<CFG, OPB_T, ROW128> plan;
  plan.init(t);

  // acc[i][j] holds C[16*i + lane%16][16*j + 4*(lane/16) + r] of the wave's
  // block: the MFMA computes C^T tiles (B fragment as the row operand), so a
  // lane's four results share one row and one row scale.
  v4f acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j) acc[i][j] = v4f{0.0f, 0.0f, 0.0f, 0.0f};

#pragma unroll
  for (int s0 = 0; s0 < S - 1; ++s0)
    if (s0 < G) plan.issue(t, s0, lds + s0 * CFG::BUF_BYTES, sbase + s0 * (BM + BN));

  int cur = 0;
  for (int g = 0; g < G; ++g) {
    // Group g has landed in buffer `cur` once this wave's copies of it are
    // complete (later groups may stay in flight); after the barrier every
    // wave's copies are visible and every wave has finished reading the
    // buffer of group g-1, which then receives group g+S-1.
    if (g + S - 2 < G)
      wait_vmcnt<(S - 2) * CFG::LOADS_PER_STAGE>();
    else
      wait_vmcnt<0>();
    __syncthreads();
    if (g + S - 1 < G) {
      const int nb = cur == 0 ? S - 1 : cur - 1;
      plan.issue(t, g + S - 1, lds + nb * CFG::BUF_BYTES, sbase + nb * (BM + BN));
    }
    __builtin_amdgcn_sched_barrier(0);

    const uint8_t* As = lds + cur * CFG::BUF_BYTES;
    const uint8_t* Bs = As + CFG::A_BYTES;
    const float* sAc = sbase + cur * (BM + BN);
    const float* sBc = sAc + BM;

    // Row scales of this lane's TM row tiles (contiguous by the copy plan).
    float sa[TM];
#pragma unroll
    for (int i = 0; i < TM; i += 4) {
      const float4 v = *reinterpret_cast<const float4*>(sAc + wm * CFG::WTM + l16 * TM + i);
      sa[i] = v.x; sa[i + 1] = v.y; sa[i + 2] = v.z; sa[i + 3] = v.w;
    }
    // Column scales: one block value per wave, or four per column tile.
    float4 sbv[TN];
    float sbb = 0.0f;
    if (ROW128) {
#pragma unroll
      for (int j = 0; j < TN; ++j) sbv[j] = *reinterpret_cast<const float4*>(sBc + wn * CFG::WTN + 16 * j + 4 * lq);
    } else {
      sbb = nblk_ok ? (OPB_T ? t.sB[nblk * t.sB_ld + g] : t.sB[(int64_t)g * t.sB_ld + nblk]) : 0.0f;
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

    // MFMAs of row tile i interleaved with the folds of row tile i-1, whose
    // results are ready by then: one MFMA, then four FMAs (plus the scale
    // multiply), so the matrix core and the vector ALU work side by side.
    v4f pprev[TN];
#pragma unroll
    for (int i = 0; i <= TM; ++i) {
      v4f pcur[TN];
      if (i < TM) {
        const int r = wm * CFG::WTM + 16 * i + l16;
        const uint4 lo = *reinterpret_cast<const uint4*>(As + kmaj_off(r, 2 * lq));
        const uint4 hi = *reinterpret_cast<const uint4*>(As + kmaj_off(r, 2 * lq + 1));
        const v8i afr = v8i{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
#pragma unroll
        for (int j = 0; j < TN; ++j)
          pcur[j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(bfr[j], afr, v4f{0.0f, 0.0f, 0.0f, 0.0f}, 0,
                                                                     0, 0, 127, 0, 127);
      }
      if (i > 0) {
        const int ip = i - 1;
        if (ROW128) {
#pragma unroll
          for (int j = 0; j < TN; ++j) {
            acc[ip][j][0] = __builtin_fmaf(pprev[j][0] * sbv[j].x, sa[ip], acc[ip][j][0]);
            acc[ip][j][1] = __builtin_fmaf(pprev[j][1] * sbv[j].y, sa[ip], acc[ip][j][1]);
            acc[ip][j][2] = __builtin_fmaf(pprev[j][2] * sbv[j].z, sa[ip], acc[ip][j][2]);
            acc[ip][j][3] = __builtin_fmaf(pprev[j][3] * sbv[j].w, sa[ip], acc[ip][j][3]);
          }
        } else {
          const float sc = sa[ip] * sbb;
#pragma unroll
          for (int j = 0; j < TN; ++j) {
            acc[ip][j][0] = __builtin_fmaf(pprev[j][0], sc, acc[ip][j][0]);
            acc[ip][j][1] = __builtin_fmaf(pprev[j][1], sc, acc[ip][j][1]);
            acc[ip][j][2] = __builtin_fmaf(pprev[j][2], sc, acc[ip][j][2]);
            acc[ip][j][3] = __builtin_fmaf(pprev[j][3], sc, acc[ip][j][3]);
          }
        }
      }
      if (i < TM) {
#pragma unroll
        for (int j = 0; j < TN; ++j) pprev[j] = pcur[j];
      }
    }
    // Scheduling: alternate each MFMA with a group of vector instructions.
#pragma unroll
    for (int k = 0; k < TM * TN; ++k) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);               // 1 MFMA
      __builtin_amdgcn_sched_group_barrier(0x002, ROW128 ? 8 : 5, 0);  // VALU (fold)
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);               // 1 LDS read
    }
    __builtin_amdgcn_sched_barrier(0);
    cur = cur + 1 == S ? 0 : cur + 1;
  }

  // ---- epilogue: FP32 C, four consecutive columns per lane ----
#pragma unroll
  for (int i = 0; i < TM; ++i) {
    const int64_t row = wm * CFG::WTM + 16 * i + l16;
    if (row >= t.rows) continue;
#pragma unroll
    for (int j = 0; j < TN; ++j) {
      const int64_t col = t.n0 + wn * CFG::WTN + 16 * j + 4 * lq;
      float* dst = t.C + row * t.ldc + col;
      if (col + 3 < t.N) {
        *reinterpret_cast<float4*>(dst) = make_float4(acc[i][j][0], acc[i][j][1], acc[i][j][2], acc[i][j][3]);
      } else {
#pragma unroll
        for (int r = 0; r < 4; ++r)
          if (col + r < t.N) dst[r] = acc[i][j][r];
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

// Per-lane copy offsets are 32-bit: operand pitches stay below 2^23 bytes.
static constexpr int64_t kMaxPitch = int64_t(1) << 23;

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
  if (lda >= kMaxPitch || ldb >= kMaxPitch) return FP8BLK_ERR_UNSUPPORTED;
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
  if (lda >= kMaxPitch || ldb >= kMaxPitch) return FP8BLK_ERR_UNSUPPORTED;
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
