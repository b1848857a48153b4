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
//
// When every scale is a power of two (the pages' choice for some activations
// [p2¶4]; FP8BLK_GEMM_POW2_SCALES), the scales are exact E8M0 block scales:
// the MFMA applies them to its operands and adds the group's product to the
// FP32 accumulator itself (srcC, round to nearest even), so the promotion
// needs no vector-ALU work.
// Citations [pN¶k]: N-th page of the source collection, k-th paragraph
// (p1 = xn--9g3bo1gtkw0l8ubf92bgle.kr wr_id 85187, p2 = inprokorea.com wr_id
// 735329, p5 = inprokorea.com wr_id 890463).
//
// Data flow per workgroup tile (BM x BN), per K group:
//   global -> LDS directly (buffer_load_dwordx4 ... lds, 16 bytes per lane),
//     double buffered in two distinct LDS arrays: group g+1 is copied while
//     group g is computed; one barrier per group.
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
#include <atomic>
#include <mutex>

#include "fp8_device.h"
#include "host_common.h"
#include "token_groups.h"

namespace fp8blk {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef int v2i __attribute__((ext_vector_type(2)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v2i lds_v2i;
typedef __attribute__((address_space(3))) void lds_void;

// Workgroup tile: WAVES_M x WAVES_N waves, each owning TM x TN MFMA tiles of
// 16x16.  Operands are double buffered in LDS: group g+1 is copied while
// group g is computed.
template <int WAVES_M_, int WAVES_N_, int TM_, int TN_>
struct TileCfg {
  static constexpr int WAVES_M = WAVES_M_, WAVES_N = WAVES_N_, TM = TM_, TN = TN_;
  static constexpr int NW = WAVES_M * WAVES_N;
  static constexpr int NT = NW * 64;
  static constexpr int WTM = 16 * TM, WTN = 16 * TN;
  static constexpr int BM = WAVES_M * WTM, BN = WAVES_N * WTN;
  static constexpr int A_BYTES = BM * 128, B_BYTES = BN * 128;
  static constexpr int A_CHUNKS = A_BYTES / 16, B_CHUNKS = B_BYTES / 16;
  // Copy iterations of 1 KB per wave; the last A iteration is partial when
  // BM is not a multiple of 8 * NW rows (only its first waves copy).
  static constexpr int A_ITERS = (A_CHUNKS + 64 * NW - 1) / (64 * NW), B_ITERS = B_CHUNKS / (64 * NW);
  static constexpr bool A_PARTIAL = A_CHUNKS % (64 * NW) != 0;
  // Scale copies: row scales of sA then BN floats of sB-side scales, 64
  // floats per wave instruction, one instruction per wave.  A lane's row
  // scales are a run of TMP = TM rounded up to 4 floats (read as float4), so
  // the row part holds BMP = WAVES_M * 16 * TMP floats (BM when TM % 4 == 0).
  static constexpr int TMP = (TM + 3) / 4 * 4, WTMP = 16 * TMP, BMP = WAVES_M * WTMP;
  static constexpr int S_BLOCKS = (BMP + BN) / 64;
  static constexpr int BUF_BYTES = A_BYTES + B_BYTES;
  static constexpr int SC_FLOATS = BMP + BN;
  static constexpr int LDS_BYTES = 2 * (BUF_BYTES + SC_FLOATS * 4);
  static_assert(WTN <= 128 && 128 % WTN == 0, "a wave's columns must lie in one 128-column scale block");
  static_assert(BN >= 128, "the N-major swizzle needs BN >= 128");
  static_assert(A_CHUNKS % 64 == 0 && B_CHUNKS % (64 * NW) == 0, "whole 1 KB copy blocks per wave");
  static_assert(BMP % 64 == 0 && BN % 64 == 0, "scale copies in 64-float blocks");
  static_assert(S_BLOCKS <= NW, "one scale copy per wave");
  static_assert(LDS_BYTES <= 160 * 1024, "LDS capacity");
};

#ifndef FP8BLK_BIG_CFG
#define FP8BLK_BIG_CFG 2, 4, 8, 4  // 256 x 256 tile, 8 waves of 128 x 64
#endif
#ifndef FP8BLK_BIG224_CFG
#define FP8BLK_BIG224_CFG 2, 4, 7, 4  // 224 x 256 tile, 8 waves of 112 x 64
#endif
#ifndef FP8BLK_SMALL_CFG
#define FP8BLK_SMALL_CFG 2, 2, 4, 4  // 128 x 128 tile, 4 waves of 64 x 64
#endif
#ifndef FP8BLK_ROW_CFG
#define FP8BLK_ROW_CFG 2, 2, 4, 4  // 128 x 128 tile, 4 waves of 64 x 64 (per-column scales need more registers)
#endif
using BigCfg = TileCfg<FP8BLK_BIG_CFG>;
using Big224Cfg = TileCfg<FP8BLK_BIG224_CFG>;
using SmallCfg = TileCfg<FP8BLK_SMALL_CFG>;
using RowCfg = TileCfg<FP8BLK_ROW_CFG>;

// s_waitcnt with vmcnt = N and no wait on the other counters (gfx9 encoding:
// vmcnt in bits 3:0 and 15:14, expcnt 6:4, lgkmcnt 11:8).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N <= 63, "vmcnt range");
  asm volatile("s_waitcnt vmcnt(%0)" : : "i"(N) : "memory");
}

// --- LDS addressing -------------------------------------------------------
// Both swizzles were picked by measuring the LDS read rate of the exact
// fragment read patterns on gfx950 (one CU, eight waves, reads back to back):
// a swizzle that looks conflict-free for 16-lane phases can still run at
// half rate there.
//
// K-major tile [rows][128 bytes]: 16-byte chunk c of row r lives at chunk
// c ^ kmaj_swz(r).  A fragment read has lane l take row 16*i + l%16, chunk
// 2*(l/16) (+1).  Measured: 4.0 cycles per 1 KB ds_read_b128 (the rate of a
// linear read) with this swizzle, 8.1 with c ^ ((r >> 1) & 7) or c ^ (r & 7).
__device__ __forceinline__ int kmaj_swz(int r) { return ((r >> 1) & 1) | (r & 4); }
__device__ __forceinline__ int kmaj_off(int r, int c16) { return r * 128 + ((c16 ^ kmaj_swz(r)) << 4); }

// N-major tile [128 k][BN bytes]: 16-byte chunk m of row k lives at chunk
// m ^ nmaj_swz(k) (BN >= 128), keeping the two 8-byte halves of a chunk
// adjacent.  A transposing fragment read has the 16-lane group g = l/16 read
// rows 32*g + 8*r + (0..7); bit 5 of k (g odd) moves those rows to the other
// half of a 256-byte row (BN = 256) or to the odd chunks (BN = 128).
// Measured: 2.6 cycles per ds_read_b64_tr_b8 (2.35 for a linear read) against
// 4.0 with m ^ (k & 7) alone.
template <int BN>
__device__ __forceinline__ int nmaj_swz(int k) {
  return (k & 7) ^ (((k >> 5) & 1) * (BN >= 256 ? 8 : 1));
}
template <int BN>
__device__ __forceinline__ int nmaj_off(int k, int m16) {
  return k * BN + ((m16 ^ nmaj_swz<BN>(k)) << 4);
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
typedef int v4i __attribute__((ext_vector_type(4)));
// Raw buffer resource (stride 0): base address, record count, and the gfx9
// raw-buffer flags word.
__device__ __forceinline__ v4i rsrc_of(const void* base, int64_t bytes) {
  const int32_t n = bytes > 0x7FFFFFFF ? 0x7FFFFFFF : (bytes < 0 ? 0 : (int32_t)bytes);
  const uint64_t a = reinterpret_cast<uint64_t>(base);
  return v4i{(int)(uint32_t)a, (int)((uint32_t)(a >> 32) & 0xFFFFu), n, 0x00020000};
}
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) uint8_t*)p;
}
// The copies are issued from inline assembly: the compiler then does not
// track them as pending LDS writes (its alias tracking of LDS DMA loses the
// stage arrays apart and stalls LDS reads of the other stage on them); the K
// loop synchronizes them itself (vmcnt wait, then barrier, before a stage is
// read).  The instructions have no register results.
__device__ __forceinline__ void dma16(v4i r, uint32_t voff, int32_t soff, uint8_t* lds_base) {
  asm volatile("s_mov_b32 m0, %3\n\tbuffer_load_dwordx4 %0, %1, %2 offen lds"
               :
               : "v"(voff), "s"(r), "s"(soff), "s"(lds_addr(lds_base))
               : "memory", "m0");
}
// dma16 issued only when `left` > 0 (a scalar test inside the same asm
// block, so the compiler's schedule around it is that of a plain copy).
__device__ __forceinline__ void dma16_if(v4i r, uint32_t voff, int32_t soff, uint8_t* lds_base, int32_t left) {
  asm volatile("s_cmp_gt_i32 %4, 0\n\ts_cbranch_scc0 1f\n\ts_mov_b32 m0, %3\n\tbuffer_load_dwordx4 %0, %1, %2 offen lds\n1:"
               :
               : "v"(voff), "s"(r), "s"(soff), "s"(lds_addr(lds_base)), "s"(left)
               : "memory", "m0", "scc");
}
__device__ __forceinline__ void dma4(v4i r, uint32_t voff, uint8_t* lds_base) {
  asm volatile("s_mov_b32 m0, %2\n\tbuffer_load_dword %0, %1, 0 offen lds"
               :
               : "v"(voff), "s"(r), "s"(lds_addr(lds_base))
               : "memory", "m0");
}

// Two FP32 values rounded to BF16 (nearest even; subnormals kept; values
// beyond the largest finite BF16 become infinities; a NaN stays a NaN),
// packed: `lo` in bits 15:0, `hi` in bits 31:16.  One v_cvt_pk_bf16_f32.
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t bf16_pack(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2_t{lo, hi}, bf16x2_t));
}

// 4 x 4 transpose between the four 16-lane rows of a wave and four
// registers: afterwards register k of lane l16 + 16 r holds what register r
// of lane l16 + 16 k held.  Two swaps of wave halves (v_permlane32_swap),
// then two swaps of neighbouring rows (v_permlane16_swap).  Every lane of the
// wave must be active.
__device__ __forceinline__ void transpose_rows4(uint32_t (&c)[4]) {
  const auto s02 = __builtin_amdgcn_permlane32_swap(c[0], c[2], false, false);
  const auto s13 = __builtin_amdgcn_permlane32_swap(c[1], c[3], false, false);
  const auto s01 = __builtin_amdgcn_permlane16_swap(s02[0], s13[0], false, false);
  const auto s23 = __builtin_amdgcn_permlane16_swap(s02[1], s13[1], false, false);
  c[0] = s01[0];
  c[1] = s01[1];
  c[2] = s23[0];
  c[3] = s23[1];
}

// Output modes of a GEMM kernel: FP32 C, BF16 C, or C quantized on store to
// E4M3 with 1x128 scales (default or power-of-two scales).
enum { OUT_F32 = 0, OUT_BF16 = 1, OUT_Q = 2, OUT_Q_POW2 = 3 };
constexpr int out_elem_bytes(int om) { return om == OUT_F32 ? 4 : om == OUT_BF16 ? 2 : 1; }

// Row `row` of an output matrix whose elements have `esize` bytes.
__device__ __forceinline__ void* out_row(void* C, int64_t ldc, int64_t row, int esize) {
  return static_cast<char*>(C) + row * ldc * esize;
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
  void* C;            // row m0 of C (FP32, BF16 or E4M3 codes by the kernel's output mode)
  int64_t ldc;        // row pitch of C in elements
  float* sQ;          // quantized output: its 1x128 scales [ceil(N/128)][sQ_ld]
  int64_t sQ_ld;      //   (row count of the whole output)
  int64_t m0;         //   first output row of this tile
  int64_t K;
  int g0, g1;         // K groups [g0, g1) of this tile's (partial) product
};

// Copies of one K group.  Group bases: A tile A + k0; B tile B + n0*ldb + k0
// ([N][K]) or B + k0*ldb + n0 ([K][N]); scales sA + g*ld and sB + g*ld + n0.
// The sA copy is permuted so that each lane later reads the TM row scales it
// needs (rows 16*i + lane%16 of its wave's rows) as one contiguous run.
template <class CFG, bool OPB_T, bool ROW128>
struct CopyPlan {
  static constexpr int NW = CFG::NW, BM = CFG::BM, BN = CFG::BN;
  // [K][N] B tile: BN/16 chunks per k row, so one copy iteration advances k
  // by KSTEP rows: k = it * KSTEP + (the lane's row).  Then k & 7 is the same
  // in every iteration, and bit 5 of k is the lane's own (KSTEP a multiple of
  // 64) or flips on odd iterations (KSTEP = 32 mod 64): two per-lane offsets
  // cover both.
  static constexpr int KSTEP = NW * 64 / (BN / 16);
  static_assert(KSTEP % 32 == 0, "[K][N] copies: bit 5 of k per lane or alternating per iteration");
  uint32_t a, b, b2;

  __device__ __forceinline__ void init(const TileArgs& t) {
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    {  // A and [N][K] B: chunk ci = (it*NW + wave)*64 + lane; row ci/8 advances by 8*NW per it
      const int ci = wave * 64 + lane;
      const int r = ci >> 3, c = (ci & 7) ^ kmaj_swz(r);
      a = (uint32_t)(r * t.lda + c * 16);
      if (OPB_T) b = b2 = (uint32_t)(r * t.ldb + c * 16);
    }
    if (!OPB_T) {  // [K][N] B: BN/16 chunks per k row; k advances by KSTEP per it
      constexpr int CPR = BN / 16;
      const int ci = wave * 64 + lane;
      const int k = ci / CPR, p16 = ci % CPR;
      // global chunk for LDS position p16 when bit 5 of k is that of this
      // lane's row (b) or its complement (b2, the odd iterations)
      b = (uint32_t)(k * t.ldb + (p16 ^ nmaj_swz<BN>(k)) * 16);
      b2 = KSTEP % 64 == 0 ? b : (uint32_t)(k * t.ldb + (p16 ^ nmaj_swz<BN>(k ^ 32)) * 16);
    }
  }

  // Per-lane byte offset of this lane's scale copy.  The 128x128 kernels
  // form it at each issue from an opaque copy of the thread id (a few
  // integer operations per group instead of a VGPR held across the K loop);
  // the row-pipelined loop forms it once per tile.
  __device__ __forceinline__ uint32_t sc_offset(const TileArgs& t) const {
    constexpr int TMP = CFG::TMP, WTM = CFG::WTM, WTMP = CFG::WTMP, BMP = CFG::BMP;
    int tid = threadIdx.x;
    asm volatile("" : "+v"(tid));
    const int lane = tid & 63;
    int blk = __builtin_amdgcn_readfirstlane(tid >> 6);
    if (blk >= CFG::S_BLOCKS) blk = 0;  // surplus copy: rewrites block 0 with the same data
    const int p = blk * 64 + lane;      // float position in the [BMP + BN] scale buffer
    // BMP is a multiple of 64, so the row/column choice is uniform per wave
    // (derived from blk alone), which keeps the resource in scalar registers.
    // Position q of wave row w is lane q / TMP's row tile q % TMP; padding
    // positions (row tile >= TM) load a row that is never read back (past
    // the tile's rows it reads as zero).
    const int w = p / WTMP, q = p % WTMP;
    const uint32_t row_off = (uint32_t)((w * WTM + 16 * (q % TMP) + q / TMP) * 4);
    // column scale of column n0 + (p - BMP), or block scale of column block
    // n0/128 + (p - BMP) (only the first BN/128 positions are used)
    const uint32_t col_off =
        ROW128 ? (uint32_t)((p - BMP) * 4) : (uint32_t)((p - BMP) * (OPB_T ? (int)(t.K >> 7) : 1) * 4);
    if (blk * 64 < BMP) return row_off;
    return col_off;
  }

  __device__ __forceinline__ void issue(const TileArgs& t, int g, uint8_t* buf, float* sbuf) const {
    const Rsrc r = rsrc(t, g);
#pragma unroll
    for (int n = 0; n < LOADS; ++n) issue_one(r.a, r.b, r.sa, r.sb, n, t, buf, sbuf);
  }

  // Resources of group g's copies.
  struct Rsrc {
    v4i a, b, sa, sb;
  };
  __device__ __forceinline__ Rsrc rsrc(const TileArgs& t, int g) const {
    const int64_t k0 = (int64_t)g * 128;
    Rsrc r;
    r.a = rsrc_of(t.A + k0, (t.rows - 1) * t.lda + 128);
    if (OPB_T) {
      const int64_t nvalid = t.N - t.n0 < BN ? t.N - t.n0 : BN;
      r.b = rsrc_of(t.B + t.n0 * t.ldb + k0, (nvalid - 1) * t.ldb + 128);
    } else {
      r.b = rsrc_of(t.B + k0 * t.ldb + t.n0, (t.K - k0) * t.ldb - t.n0);
    }
    r.sa = rsrc_of(t.sA + (int64_t)g * t.sA_ld, t.rows * 4);
    if (ROW128) {
      r.sb = rsrc_of(t.sB + (int64_t)g * t.sB_ld + t.n0, (t.N - t.n0) * 4);
    } else {
      const int64_t nb0 = t.n0 / 128, NB = (t.N + 127) / 128, Gk = t.K / 128;
      r.sb = OPB_T ? rsrc_of(t.sB + nb0 * Gk + g, ((NB - nb0 - 1) * Gk + 1) * 4)
                   : rsrc_of(t.sB + (int64_t)g * t.sB_ld + nb0, (NB - nb0) * 4);
    }
    return r;
  }

  // Copy number n (0 .. LOADS-1) of a group: A blocks, then B blocks, then
  // the scale block.
  static constexpr int LOADS = CFG::A_ITERS + CFG::B_ITERS + 1;
  __device__ __forceinline__ void issue_one(v4i ra, v4i rb,
                                            v4i rsa, v4i rsb, int n,
                                            const TileArgs& t, uint8_t* buf, float* sbuf) const {
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    static_assert(!CFG::A_PARTIAL, "the 128x128 tiles copy whole A iterations");
    if (n < CFG::A_ITERS) {
      const int it = n;
      dma16(ra, a, (int32_t)(it * 8 * NW * t.lda), buf + (it * NW + wave) * 1024);
    } else if (n < CFG::A_ITERS + CFG::B_ITERS) {
      const int it = n - CFG::A_ITERS;
      const int32_t so = OPB_T ? (int32_t)(it * 8 * NW * t.ldb) : (int32_t)(it * KSTEP * t.ldb);
      dma16(rb, (!OPB_T && (it & 1)) ? b2 : b, so, buf + CFG::A_BYTES + (it * NW + wave) * 1024);
    } else {
      const int blk = wave < CFG::S_BLOCKS ? wave : 0;
      const bool rows = blk * 64 < CFG::BMP;  // wave-uniform; a select keeps the copy branch-free
      const v4i rs = v4i{rows ? rsa[0] : rsb[0], rows ? rsa[1] : rsb[1], rows ? rsa[2] : rsb[2], rows ? rsa[3] : rsb[3]};
      dma4(rs, sc_offset(t), (uint8_t*)(sbuf + blk * 64));
    }
  }
};

// Whether a tile runs the row-pipelined K loop (gemm_loop_rows below): tiles
// with ROWPIPE_MIN_TM or more row tiles per wave (the 256x256 and 224x256
// tiles).  The
// 128x128 tiles (two workgroups per CU) keep the loop that issues a group's
// copies at its start (compute_group below).
#ifndef FP8BLK_ROWPIPE_MIN_TM
#define FP8BLK_ROWPIPE_MIN_TM 7
#endif
template <class CFG, bool ROW128>
constexpr bool row_pipelined() { return CFG::TM >= FP8BLK_ROWPIPE_MIN_TM; }

// One K group of MFMAs and scale folds on operands already in LDS (`ops`:
// A tile then B tile; `sc`: row scales in lane order, then column/block
// scales).  acc[i][j] holds C[16*i + lane%16][16*j + 4*(lane/16) + r] of the
// wave's block: the MFMA computes C^T tiles (B fragment as the row operand),
// so a lane's four results share one row and one row scale.
// MFMA with E8M0 block scales: byte OA of `sa` scales the rows of the first
// operand, byte OB of `sb` those of the second (lane l supplies the scale of
// row l%16 for its 32-deep k block l/16); srcC is accumulated in FP32.
template <int OA, int OB>
__device__ __forceinline__ v4f mfma_e8m0(const v8i& a, const v8i& b, const v4f& c, uint32_t sa, uint32_t sb) {
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 0, OA, sa, OB, sb);
}
template <int OA>
__device__ __forceinline__ v4f mfma_e8m0_b(int ob, const v8i& a, const v8i& b, const v4f& c, uint32_t sa,
                                           uint32_t sb) {
  switch (ob & 3) {
    case 0: return mfma_e8m0<OA, 0>(a, b, c, sa, sb);
    case 1: return mfma_e8m0<OA, 1>(a, b, c, sa, sb);
    case 2: return mfma_e8m0<OA, 2>(a, b, c, sa, sb);
    default: return mfma_e8m0<OA, 3>(a, b, c, sa, sb);
  }
}
__device__ __forceinline__ v4f mfma_e8m0_sel(int oa, int ob, const v8i& a, const v8i& b, const v4f& c, uint32_t sa,
                                             uint32_t sb) {
  switch (oa & 3) {
    case 0: return mfma_e8m0_b<0>(ob, a, b, c, sa, sb);
    case 1: return mfma_e8m0_b<1>(ob, a, b, c, sa, sb);
    case 2: return mfma_e8m0_b<2>(ob, a, b, c, sa, sb);
    default: return mfma_e8m0_b<3>(ob, a, b, c, sa, sb);
  }
}
// E8M0 code of a power-of-two FP32 scale: its biased exponent.
__device__ __forceinline__ uint32_t e8m0_of(float s) { return (__float_as_uint(s) >> 23) & 0xFFu; }

// One K group on the 128x128 tiles: the group's copies were issued at its
// start by the caller.
template <class CFG, bool OPB_T, bool ROW128, bool P2>
__device__ __forceinline__ void compute_group(const uint8_t* ops, const float* sc,
                                              v4f (&acc)[CFG::TM][CFG::TN]) {
  constexpr int BN = CFG::BN, TM = CFG::TM, TN = CFG::TN;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / CFG::WAVES_N, wn = wave % CFG::WAVES_N;
  const int l16 = lane & 15, lq = lane >> 4;
  const uint8_t* As = ops;
  const uint8_t* Bs = ops + CFG::A_BYTES;

  // Row scales of this lane's TM row tiles (contiguous by the copy plan).
  float sa[CFG::TMP];
#pragma unroll
  for (int i = 0; i < TM; i += 4) {
    const float4 v = *reinterpret_cast<const float4*>(sc + wm * CFG::WTMP + l16 * CFG::TMP + i);
    sa[i] = v.x; sa[i + 1] = v.y; sa[i + 2] = v.z; sa[i + 3] = v.w;
  }
  // Column scales: one block value per wave, or four per column tile.
  float4 sbv[TN];
  float sbb = 0.0f;
  if (ROW128) {
#pragma unroll
    for (int j = 0; j < TN; ++j) sbv[j] = *reinterpret_cast<const float4*>(sc + CFG::BMP + wn * CFG::WTN + 16 * j + 4 * lq);
  } else {
    sbb = sc[CFG::BMP + (wn * CFG::WTN) / 128];
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

  auto load_a = [&](int i) {
    const int r = wm * CFG::WTM + 16 * i + l16;
    const uint4 lo = *reinterpret_cast<const uint4*>(As + kmaj_off(r, 2 * lq));
    const uint4 hi = *reinterpret_cast<const uint4*>(As + kmaj_off(r, 2 * lq + 1));
    return v8i{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
  };
  static_assert(!(P2 && ROW128) || TN <= 4, "four column tiles per packed scale register");
  if (P2) {
    // Power-of-two scales applied by the matrix core: E8M0 exponents of the
    // TM row scales, four per register (byte i%4 for row tile i), and of the
    // column scales (four column tiles per register, byte j) or the block
    // scale; each group's product is added to the FP32 accumulator by the
    // MFMA itself.
    uint32_t sae[(TM + 3) / 4];
#pragma unroll
    for (int q = 0; q < (TM + 3) / 4; ++q) sae[q] = 0;
#pragma unroll
    for (int i = 0; i < TM; ++i) sae[i / 4] |= e8m0_of(sa[i]) << (8 * (i % 4));
    uint32_t sbe = 0;
    if (ROW128) {
#pragma unroll
      for (int j = 0; j < TN && j < 4; ++j)
        sbe |= e8m0_of(sc[CFG::BMP + wn * CFG::WTN + 16 * j + l16]) << (8 * j);
    } else {
      sbe = e8m0_of(sbb);
    }
    v8i af[TM];
    af[0] = load_a(0);
    if (TM > 1) af[1] = load_a(1);
#pragma unroll
    for (int i = 0; i < TM; ++i) {
      if (i + 2 < TM) af[i + 2] = load_a(i + 2);
#pragma unroll
      for (int j = 0; j < TN; ++j)
        acc[i][j] = mfma_e8m0_sel(ROW128 ? j : 0, i % 4, bfr[j], af[i], acc[i][j], sbe, sae[i / 4]);
      __builtin_amdgcn_sched_barrier(0);
    }
    return;
  }

  // Each MFMA's partial is folded right after the next MFMA has been issued
  // (a two-entry ring), so the matrix core and the vector ALU can work side
  // by side with only two partials live.  The next row tile's A fragment is
  // read from LDS while the current row's MFMAs run.
  auto fold = [&](const v4f& p, int i, int j) {
    if (ROW128) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float sb = r == 0 ? sbv[j].x : r == 1 ? sbv[j].y : r == 2 ? sbv[j].z : sbv[j].w;
        acc[i][j][r] = __builtin_fmaf(p[r] * sb, sa[i], acc[i][j][r]);
      }
    } else {
      const float sc = sa[i] * sbb;
#pragma unroll
      for (int r = 0; r < 4; ++r) acc[i][j][r] = __builtin_fmaf(p[r], sc, acc[i][j][r]);
    }
  };
  v4f ring[2];
  v8i afr = load_a(0);
#pragma unroll
  for (int i = 0; i < TM; ++i) {
    const v8i anext = i + 1 < TM ? load_a(i + 1) : afr;
#pragma unroll
    for (int j = 0; j < TN; ++j) {
      const int k = i * TN + j;
      // C^T tile: the B fragment is the row operand.
      ring[k & 1] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(bfr[j], afr, v4f{0.0f, 0.0f, 0.0f, 0.0f}, 0, 0,
                                                                     0, 127, 0, 127);
      if (k > 0) fold(ring[(k - 1) & 1], (k - 1) / TN, (k - 1) % TN);
    }
    afr = anext;
  }
  fold(ring[(TM * TN - 1) & 1], TM - 1, TN - 1);
}

// ---- Row-pipelined K loop (256x256 tiles) ---------------------------------
// After each group's barrier a wave reads its B fragments and first A
// fragment, then walks its TM row tiles: row tile i reads the A fragment of
// row i+1, issues (in the first FP8BLK_COPY_ROWS rows) its share of the next
// group's copies, and runs its TN MFMAs; the fold path folds each partial
// FP8BLK_FOLD_RING-1 MFMAs after it was issued.  The copy resources advance
// from per-tile cursors held in scalar registers and the scale copy's lane
// offset is computed once per tile, so a group issues little beyond its
// MFMAs, folds, LDS reads and copies.
// Measured on the 4096x4096x7168 Fprop (interleaved on one box, results
// bitwise identical): cursors and once-per-tile offsets against per-group
// recomputation -9 %; copies spread over the first 4 of 8 rows against all
// rows -5 %, against the first 1 / 2 / 3 rows -4 / -3 / -5 %; fold ring 4
// against 2 and 3 -3 %.  Ablations (timing only): without the copies -17 %,
// without the A and B fragment reads -18 %, without the barrier -11 %,
// without any MFMA -12 %: the loop is bound by moving the operands (a
// copy-only loop of the same traffic takes half the GEMM's time, and copies
// overlap the MFMAs only in part), not by the matrix cores.
#ifndef FP8BLK_FOLD_RING
#define FP8BLK_FOLD_RING 4
#endif
#ifndef FP8BLK_COPY_ROWS
#define FP8BLK_COPY_ROWS 4
#endif

// Copy resources of the next K group: A tile, B tile and this wave's scale
// run, each a 64-bit address advanced by a fixed stride per group.
template <class CFG, bool OPB_T, bool ROW128>
struct GroupCursor {
  uint64_t a, b, s;
  int64_t b_step, s_step;
  int64_t b_left;  // valid bytes from b on ([K][N] B: shrinks per group)
  int32_t a_cnt, s_cnt;

  __device__ __forceinline__ void init(const TileArgs& t, int g, bool rows_wave) {
    constexpr int BN = CFG::BN;
    const int64_t Gk = t.K / 128, NB = (t.N + 127) / 128, nb0 = t.n0 / 128;
    a = reinterpret_cast<uint64_t>(t.A) + (uint64_t)g * 128;
    a_cnt = (int32_t)((t.rows - 1) * t.lda + 128);
    if (OPB_T) {
      b = reinterpret_cast<uint64_t>(t.B + t.n0 * t.ldb) + (uint64_t)g * 128;
      const int64_t nvalid = t.N - t.n0 < BN ? t.N - t.n0 : BN;
      b_left = (nvalid - 1) * t.ldb + 128;
      b_step = 128;
    } else {
      b = reinterpret_cast<uint64_t>(t.B + t.n0) + (uint64_t)g * 128 * t.ldb;
      b_left = (t.K - (int64_t)g * 128) * t.ldb - t.n0;
      b_step = 128 * t.ldb;
    }
    if (rows_wave) {
      s = reinterpret_cast<uint64_t>(t.sA + (int64_t)g * t.sA_ld);
      s_step = t.sA_ld * 4;
      s_cnt = (int32_t)(t.rows * 4);
    } else if (ROW128) {  // column scales [K/128][N]: the tile's BN columns of group g
      s = reinterpret_cast<uint64_t>(t.sB + (int64_t)g * t.sB_ld + t.n0);
      s_step = t.sB_ld * 4;
      s_cnt = (int32_t)((t.N - t.n0) * 4);
    } else if (OPB_T) {
      s = reinterpret_cast<uint64_t>(t.sB + nb0 * Gk + g);
      s_step = 4;
      s_cnt = (int32_t)(((NB - nb0 - 1) * Gk + 1) * 4);
    } else {
      s = reinterpret_cast<uint64_t>(t.sB + (int64_t)g * t.sB_ld + nb0);
      s_step = t.sB_ld * 4;
      s_cnt = (int32_t)((NB - nb0) * 4);
    }
  }
  __device__ __forceinline__ void advance() {
    a += 128;
    b += b_step;
    if (!OPB_T) b_left -= b_step;
    s += s_step;
  }
  // Resources; `on` false gives a zero record count (every copy reads nothing).
  static __device__ __forceinline__ v4i rsrc(uint64_t addr, int64_t n) {
    const int32_t c = n > 0x7FFFFFFF ? 0x7FFFFFFF : (n < 0 ? 0 : (int32_t)n);
    return v4i{(int)(uint32_t)addr, (int)((uint32_t)(addr >> 32) & 0xFFFFu), c, 0x00020000};
  }
  __device__ __forceinline__ v4i ra(bool on) const { return rsrc(a, on ? a_cnt : 0); }
  __device__ __forceinline__ v4i rb(bool on) const { return rsrc(b, on ? b_left : 0); }
  __device__ __forceinline__ v4i rs(bool on) const { return rsrc(s, on ? s_cnt : 0); }
};

// Copies n0 .. n1-1 of a group (A blocks, then B blocks, then the scale run).
// SKIP: an A block whose 8 rows all lie past the tile's valid rows is not
// issued (its LDS rows keep stale data, which only feeds output rows that
// are never stored).
template <class CFG, bool OPB_T, bool ROW128, bool SKIP>
__device__ __forceinline__ void issue_copies(const TileArgs& t, const CopyPlan<CFG, OPB_T, ROW128>& plan,
                                             uint32_t scoff, const v4i& ra, const v4i& rb, const v4i& rs, int n0,
                                             int n1, uint8_t* buf, float* sbuf, int wave, int blk) {
  constexpr int NW = CFG::NW, KSTEP = CopyPlan<CFG, OPB_T, ROW128>::KSTEP;
#pragma unroll
  for (int n = n0; n < n1; ++n) {
    if (n < CFG::A_ITERS) {
      // The partial last iteration of a BM that is not a multiple of 8 * NW
      // rows: a wave whose 8 rows start at or past the tile's valid rows
      // (t.rows <= BM) issues nothing, so no copy lands beyond the A tile.
      if (SKIP || (CFG::A_PARTIAL && n == CFG::A_ITERS - 1))
        dma16_if(ra, plan.a, (int32_t)(n * 8 * NW * t.lda), buf + (n * NW + wave) * 1024,
                 (int32_t)t.rows - (n * NW + wave) * 8);
      else
        dma16(ra, plan.a, (int32_t)(n * 8 * NW * t.lda), buf + (n * NW + wave) * 1024);
    } else if (n < CFG::A_ITERS + CFG::B_ITERS) {
      const int it = n - CFG::A_ITERS;
      const int32_t so = OPB_T ? (int32_t)(it * 8 * NW * t.ldb) : (int32_t)(it * KSTEP * t.ldb);
      dma16(rb, (!OPB_T && (it & 1)) ? plan.b2 : plan.b, so, buf + CFG::A_BYTES + (it * NW + wave) * 1024);
    } else {
      dma4(rs, scoff, (uint8_t*)(sbuf + blk * 64));
    }
  }
}

// One K group of a row-pipelined tile: operands of this group in `ops`/`sc`,
// the next group's copies (resources ra/rb/rs) into `nops`/`nsc`.
template <class CFG, bool OPB_T, bool ROW128, bool P2, bool SKIP>
__device__ __forceinline__ void compute_group_rows(const uint8_t* ops, const float* sc, v4f (&acc)[CFG::TM][CFG::TN],
                                                   const TileArgs& t, const CopyPlan<CFG, OPB_T, ROW128>& plan,
                                                   uint32_t scoff, const v4i& ra, const v4i& rb, const v4i& rs,
                                                   uint8_t* nops, float* nsc, int wave, int blk) {
  constexpr int BN = CFG::BN, TM = CFG::TM, TN = CFG::TN, R = FP8BLK_FOLD_RING;
  constexpr int LOADS = CopyPlan<CFG, OPB_T, ROW128>::LOADS, CR = FP8BLK_COPY_ROWS;
  static_assert(CR >= 1 && CR <= TM, "copy rows");
  const int lane = threadIdx.x & 63;
  const int wm = wave / CFG::WAVES_N, wn = wave % CFG::WAVES_N;
  const int l16 = lane & 15, lq = lane >> 4;
  const uint8_t* As = ops;
  const uint8_t* Bs = ops + CFG::A_BYTES;
  auto load_a = [&](int i) {
    const int r = wm * CFG::WTM + 16 * i + l16;
    const uint4 lo = *reinterpret_cast<const uint4*>(As + kmaj_off(r, 2 * lq));
    const uint4 hi = *reinterpret_cast<const uint4*>(As + kmaj_off(r, 2 * lq + 1));
    return v8i{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
  };
  v8i afr = load_a(0);
  v8i bfr[TN];
#pragma unroll
  for (int j = 0; j < TN; ++j) {
    const int ncol = wn * CFG::WTN + 16 * j;
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
        part[r] = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_v2i*)(Bs + nmaj_off<BN>(k, ncol >> 4) + 8 * h));
      }
      bfr[j] = v8i{part[0][0], part[0][1], part[1][0], part[1][1], part[2][0], part[2][1], part[3][0], part[3][1]};
    }
  }
  // Row scales of this lane's row tiles, and the wave's block scale or (ROW128)
  // the column scales of its column tiles.
  float sa[CFG::TMP];
#pragma unroll
  for (int i = 0; i < TM; i += 4) {
    const float4 v = *reinterpret_cast<const float4*>(sc + wm * CFG::WTMP + l16 * CFG::TMP + i);
    sa[i] = v.x; sa[i + 1] = v.y; sa[i + 2] = v.z; sa[i + 3] = v.w;
  }
  float sbb = 0.0f;
  float4 sbv[ROW128 ? TN : 1];
  if constexpr (ROW128) {
#pragma unroll
    for (int j = 0; j < TN; ++j) sbv[j] = *reinterpret_cast<const float4*>(sc + CFG::BMP + wn * CFG::WTN + 16 * j + 4 * lq);
  } else {
    sbb = sc[CFG::BMP + (wn * CFG::WTN) / 128];
  }

  if constexpr (P2) {
    // E8M0 exponents: row tile i in byte i%4 of sae[i/4]; the block scale,
    // or (ROW128) column tile j's column l16 in byte j of sbe.
    static_assert(!ROW128 || TN <= 4, "four column tiles per packed scale register");
    uint32_t sae[(TM + 3) / 4];
#pragma unroll
    for (int q = 0; q < (TM + 3) / 4; ++q) sae[q] = 0;
#pragma unroll
    for (int i = 0; i < TM; ++i) sae[i / 4] |= e8m0_of(sa[i]) << (8 * (i % 4));
    uint32_t sbe = 0;
    if constexpr (ROW128) {
#pragma unroll
      for (int j = 0; j < TN; ++j) sbe |= e8m0_of(sc[CFG::BMP + wn * CFG::WTN + 16 * j + l16]) << (8 * j);
    } else {
      sbe = e8m0_of(sbb);
    }
#pragma unroll
    for (int i = 0; i < TM; ++i) {
      const v8i anext = i + 1 < TM ? load_a(i + 1) : afr;
      if (i < CR)
        issue_copies<CFG, OPB_T, ROW128, SKIP>(t, plan, scoff, ra, rb, rs, (i * LOADS) / CR, ((i + 1) * LOADS) / CR,
                                               nops, nsc, wave, blk);
#pragma unroll
      for (int j = 0; j < TN; ++j)
        acc[i][j] = mfma_e8m0_sel(ROW128 ? j : 0, i % 4, bfr[j], afr, acc[i][j], sbe, sae[i / 4]);
      afr = anext;
      __builtin_amdgcn_sched_barrier(0);
    }
    return;
  }

  float scl[TM];  // fl32(sA * sB) per row tile (block scales)
#pragma unroll
  for (int i = 0; i < TM; ++i) scl[i] = ROW128 ? sa[i] : sa[i] * sbb;
  v4f ring[R];
  auto fold = [&](int kk) {
    const int i = kk / TN, j = kk % TN;
    if constexpr (ROW128) {
      // per-column scales: fl32(P * sB) then one FMA by sA, as the
      // 128 x 128 tiles fold
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float sb = r == 0 ? sbv[j].x : r == 1 ? sbv[j].y : r == 2 ? sbv[j].z : sbv[j].w;
        acc[i][j][r] = __builtin_fmaf(ring[kk % R][r] * sb, scl[i], acc[i][j][r]);
      }
    } else {
#pragma unroll
      for (int r = 0; r < 4; ++r) acc[i][j][r] = __builtin_fmaf(ring[kk % R][r], scl[i], acc[i][j][r]);
    }
  };
#pragma unroll
  for (int i = 0; i < TM; ++i) {
    const v8i anext = i + 1 < TM ? load_a(i + 1) : afr;
    if (i < CR)
      issue_copies<CFG, OPB_T, ROW128, SKIP>(t, plan, scoff, ra, rb, rs, (i * LOADS) / CR, ((i + 1) * LOADS) / CR, nops,
                                             nsc, wave, blk);
#pragma unroll
    for (int j = 0; j < TN; ++j) {
      const int k = i * TN + j;
      // C^T tile: the B fragment is the row operand.
      ring[k % R] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(bfr[j], afr, v4f{0.0f, 0.0f, 0.0f, 0.0f}, 0, 0,
                                                                     0, 127, 0, 127);
      if (k >= R - 1) fold(k - (R - 1));
    }
    afr = anext;
    __builtin_amdgcn_sched_barrier(0);
  }
#pragma unroll
  for (int kk = TM * TN - (R - 1); kk < TM * TN; ++kk) fold(kk);
}

// The K loop of a row-pipelined tile (groups t.g0 .. t.g1-1).  Two groups per
// iteration, one per LDS stage, with no branch inside the iteration (a
// branch there lets the compiler sink the MFMAs of the first group below it,
// past the row fences); an odd last group runs after the loop.
template <class CFG, bool OPB_T, bool ROW128, bool P2, bool SKIP>
__device__ __forceinline__ void gemm_loop_rows(const TileArgs& t, uint8_t* ops0, uint8_t* ops1, float* sc0, float* sc1,
                                               v4f (&acc)[CFG::TM][CFG::TN]) {
  const int g0 = t.g0, G = t.g1;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  // SKIP: a wave whose rows all lie past the tile's valid rows (the partial
  // last row tile of an expert) issues its copies but no MFMAs or folds.
  const bool computes = !SKIP || (wave / CFG::WAVES_N) * CFG::WTM < t.rows;
  const int blk = wave < CFG::S_BLOCKS ? wave : 0;  // this wave's 64-float block of the scale buffer
  CopyPlan<CFG, OPB_T, ROW128> plan;
  plan.init(t);
  const uint32_t scoff = plan.sc_offset(t);
  GroupCursor<CFG, OPB_T, ROW128> cur;
  cur.init(t, g0, blk * 64 < CFG::BMP);
  if (g0 < G)  // no groups (an expert without tokens): C = 0
    issue_copies<CFG, OPB_T, ROW128, SKIP>(t, plan, scoff, cur.ra(true), cur.rb(true), cur.rs(true), 0,
                             CopyPlan<CFG, OPB_T, ROW128>::LOADS, ops0, sc0, wave, blk);
  cur.advance();
  auto step = [&](int gnext, uint8_t* ops, float* sc, uint8_t* nops, float* nsc) {
    // This group has landed in `ops` once this lane's copies are complete;
    // after the barrier every wave's copies are visible and every wave is
    // done reading the other stage, which then receives group gnext.
    wait_vmcnt<0>();
    __syncthreads();
    const bool on = gnext < G;
    const v4i ra = cur.ra(on), rb = cur.rb(on), rs = cur.rs(on);
    __builtin_amdgcn_sched_barrier(0);
    if (computes)
      compute_group_rows<CFG, OPB_T, ROW128, P2, SKIP>(ops, sc, acc, t, plan, scoff, ra, rb, rs, nops, nsc, wave, blk);
    else
      issue_copies<CFG, OPB_T, ROW128, SKIP>(t, plan, scoff, ra, rb, rs, 0, CopyPlan<CFG, OPB_T, ROW128>::LOADS, nops,
                                             nsc, wave, blk);
    __builtin_amdgcn_sched_barrier(0);
    cur.advance();
  };
  int g = g0;
  for (; g + 1 < G; g += 2) {
    step(g + 1, ops0, sc0, ops1, sc1);
    step(g + 2, ops1, sc1, ops0, sc0);
  }
  if (g < G) step(g + 1, ops0, sc0, ops1, sc1);
  wait_vmcnt<0>();  // the last group's (empty) copies
}

// The whole K loop of one output tile.  ops0/ops1 and sc0/sc1 are distinct
// LDS arrays (the two pipeline stages); the loop is unrolled by two so that
// every access names its array at compile time, which lets the compiler see
// that reading one stage does not have to wait for copies into the other.
template <class CFG, bool OPB_T, bool ROW128, bool P2, int OM, bool SKIP = false, bool ONE_STAGE = false>
__device__ __forceinline__ void gemm_tile(const TileArgs& t, uint8_t* ops0, uint8_t* ops1, float* sc0, float* sc1) {
  constexpr int TM = CFG::TM, TN = CFG::TN;
  const int g0 = t.g0, G = t.g1;

  v4f acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j) acc[i][j] = v4f{0.0f, 0.0f, 0.0f, 0.0f};

  if constexpr (row_pipelined<CFG, ROW128>()) {
    gemm_loop_rows<CFG, OPB_T, ROW128, P2, SKIP>(t, ops0, ops1, sc0, sc1, acc);
  } else {
    CopyPlan<CFG, OPB_T, ROW128> plan;
    plan.init(t);
    if (g0 < G) plan.issue(t, g0, ops0, sc0);  // no groups (an expert without tokens): C = 0
    // A wave whose rows all lie past the tile's valid rows (the partial last
    // row tile of an expert or of the matrix) skips its MFMAs and fold; it
    // still issues its copies and meets every barrier.
    const int wrow0 = (__builtin_amdgcn_readfirstlane(threadIdx.x >> 6) / CFG::WAVES_N) * CFG::WTM;
    const bool computes = wrow0 < t.rows;
    if constexpr (ONE_STAGE) {
      // One LDS stage (ops1/sc1 unused): each group's copies are issued once
      // every wave has finished reading the previous group.
      for (int g = g0; g < G; ++g) {
        wait_vmcnt<0>();
        __syncthreads();
        __builtin_amdgcn_sched_barrier(0);
        if (computes) compute_group<CFG, OPB_T, ROW128, P2>(ops0, sc0, acc);
        __builtin_amdgcn_sched_barrier(0);
        if (g + 1 < G) {
          __syncthreads();
          plan.issue(t, g + 1, ops0, sc0);
        }
      }
    } else
    for (int g = g0; g < G; g += 2) {
      // Group g has landed in stage 0 once this lane's copies are complete;
      // after the barrier every wave's copies are visible and every wave is
      // done reading stage 1 (group g-1), which then receives group g+1.
      wait_vmcnt<0>();
      __syncthreads();
      if (g + 1 < G) plan.issue(t, g + 1, ops1, sc1);
      __builtin_amdgcn_sched_barrier(0);
      if (computes) compute_group<CFG, OPB_T, ROW128, P2>(ops0, sc0, acc);
      __builtin_amdgcn_sched_barrier(0);
      if (g + 1 < G) {
        wait_vmcnt<0>();
        __syncthreads();
        if (g + 2 < G) plan.issue(t, g + 2, ops0, sc0);
        __builtin_amdgcn_sched_barrier(0);
        if (computes) compute_group<CFG, OPB_T, ROW128, P2>(ops1, sc1, acc);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  }

  // ---- epilogue: four consecutive columns per lane, FP32 or (OB) BF16 ----
  const int tid_e = threadIdx.x;
  const int wm_e = (tid_e >> 6) / CFG::WAVES_N, wn_e = (tid_e >> 6) % CFG::WAVES_N;
  const int l16_e = tid_e & 15, lq_e = (tid_e >> 4) & 3;
  if constexpr (OM == OUT_Q || OM == OUT_Q_POW2) {
    // Quantize on store: the BF16-rounded results in 1x128 tiles along each
    // row (a 128-column group is the columns of waves wn and wn^1), exactly
    // as quantize_1x128 quantizes a BF16 matrix.
    static_assert(CFG::WTN == 64 && CFG::WAVES_N % 2 == 0, "a 128-column scale group spans two waves");
    constexpr bool QP2 = OM == OUT_Q_POW2;
    const int wave_e = tid_e >> 6;
    // Per row: max |BF16 bits| over this wave's columns < N, combined with
    // the partner wave's through LDS (the stage buffer is free once every
    // wave has left the K loop).
    uint32_t* red = reinterpret_cast<uint32_t*>(ops0);
    // The results rounded to BF16 in place (a BF16 value is the upper half
    // of its FP32 word).
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j) {
        const uint32_t p01 = bf16_pack(acc[i][j][0], acc[i][j][1]);
        const uint32_t p23 = bf16_pack(acc[i][j][2], acc[i][j][3]);
        acc[i][j][0] = __uint_as_float(p01 << 16);
        acc[i][j][1] = __uint_as_float(p01 & 0xFFFF0000u);
        acc[i][j][2] = __uint_as_float(p23 << 16);
        acc[i][j][3] = __uint_as_float(p23 & 0xFFFF0000u);
      }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < TM; ++i) {
      uint32_t m = 0;
#pragma unroll
      for (int j = 0; j < TN; ++j) {
        const int64_t col = t.n0 + wn_e * CFG::WTN + 16 * j + 4 * lq_e;
#pragma unroll
        for (int r = 0; r < 4; ++r)
          if (col + r < t.N) m = max(m, (__float_as_uint(acc[i][j][r]) >> 16) & 0x7FFFu);
      }
      m = max(m, (uint32_t)__shfl_xor((int)m, 16));
      m = max(m, (uint32_t)__shfl_xor((int)m, 32));
      if (lq_e == 0) red[wave_e * CFG::WTM + 16 * i + l16_e] = m;
    }
    __syncthreads();
    // The codes of a row tile are transposed across the wave's four 16-lane
    // rows, so that lane (l16, lq) stores columns 16 lq .. 16 lq + 15 of the
    // wave's 64 as one 16-byte word (4x fewer, 4x wider stores).
    static_assert(TN == 4, "the store transpose covers four column tiles");
    uint8_t* Q = static_cast<uint8_t*>(t.C);
    const int64_t gcol = t.n0 + wn_e * CFG::WTN;  // first column of this wave
    const int64_t qcol = gcol + 16 * lq_e;        // first column this lane stores
#pragma unroll
    for (int i = 0; i < TM; ++i) {
      const int64_t row = wm_e * CFG::WTM + 16 * i + l16_e;
      const uint32_t amax = max(red[wave_e * CFG::WTM + 16 * i + l16_e], red[(wave_e ^ 1) * CFG::WTM + 16 * i + l16_e]);
      const TileScale ts = make_scale<QP2, true>(amax << 16);
      uint32_t codes[TN];
#pragma unroll
      for (int j = 0; j < TN; ++j) {
        float y[4], xv[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          xv[r] = acc[i][j][r];
          y[r] = quotient_fast<QP2, true>(xv[r], ts);
        }
        if (__builtin_expect(ts.slow, 0)) {
#pragma unroll
          for (int r = 0; r < 4; ++r) y[r] = quotient_slow(xv[r], ts.s);
        }
        codes[j] = pack4_e4m3(y[0], y[1], y[2], y[3]);
      }
      transpose_rows4(codes);
      if (row >= t.rows) continue;
      uint8_t* dst = Q + row * t.ldc + qcol;
      if (qcol + 15 < t.N) {
        *reinterpret_cast<uint4*>(dst) = make_uint4(codes[0], codes[1], codes[2], codes[3]);
      } else {
#pragma unroll
        for (int b = 0; b < 16; ++b)
          if (qcol + b < t.N) dst[b] = (uint8_t)(codes[b >> 2] >> (8 * (b & 3)));
      }
      if ((wn_e & 1) == 0 && lq_e == 0 && gcol < t.N) t.sQ[(gcol / 128) * t.sQ_ld + t.m0 + row] = ts.s;
    }
    return;
  }
  if constexpr (OM == OUT_BF16) {
    // BF16 pairs transposed across the wave's 16-lane rows as for the
    // quantized output: lane (l16, lq) stores columns 16 lq .. 16 lq + 15 of
    // the wave's 64 as two 16-byte words.
    static_assert(TN == 4, "the store transpose covers four column tiles");
    const int64_t qcol = t.n0 + wn_e * CFG::WTN + 16 * lq_e;
#pragma unroll
    for (int i = 0; i < TM; ++i) {
      const int64_t row = wm_e * CFG::WTM + 16 * i + l16_e;
      uint32_t lo[TN], hi[TN];
#pragma unroll
      for (int j = 0; j < TN; ++j) {
        lo[j] = bf16_pack(acc[i][j][0], acc[i][j][1]);
        hi[j] = bf16_pack(acc[i][j][2], acc[i][j][3]);
      }
      transpose_rows4(lo);
      transpose_rows4(hi);
      if (row >= t.rows) continue;
      uint16_t* dst = static_cast<uint16_t*>(t.C) + row * t.ldc + qcol;
      if (qcol + 15 < t.N) {
        reinterpret_cast<uint4*>(dst)[0] = make_uint4(lo[0], hi[0], lo[1], hi[1]);
        reinterpret_cast<uint4*>(dst)[1] = make_uint4(lo[2], hi[2], lo[3], hi[3]);
      } else {
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const uint32_t w = (e & 2) ? hi[e >> 2] : lo[e >> 2];
          if (qcol + e < t.N) dst[e] = (uint16_t)(w >> (16 * (e & 1)));
        }
      }
    }
    return;
  }
  // FP32: four consecutive columns per lane as one 16-byte store.  Tiles
  // whose columns all lie inside the matrix take a path with no per-lane
  // column test (rows past the edge, as in a MoE expert's last row tile, are
  // skipped per lane): with the column test and its element-wise tail in the
  // same code, the compiler merged the two into four predicated 4-byte
  // stores per tile column.
  if (t.n0 + CFG::BN <= t.N) {
#pragma unroll
    for (int i = 0; i < TM; ++i) {
      const int64_t row = wm_e * CFG::WTM + 16 * i + l16_e;
      if (row >= t.rows) continue;
#pragma unroll
      for (int j = 0; j < TN; ++j) {
        const int64_t col = t.n0 + wn_e * CFG::WTN + 16 * j + 4 * lq_e;
        *reinterpret_cast<float4*>(static_cast<float*>(t.C) + row * t.ldc + col) =
            make_float4(acc[i][j][0], acc[i][j][1], acc[i][j][2], acc[i][j][3]);
      }
    }
    return;
  }
#pragma unroll
  for (int i = 0; i < TM; ++i) {
    const int64_t row = wm_e * CFG::WTM + 16 * i + l16_e;
    if (row >= t.rows) continue;
#pragma unroll
    for (int j = 0; j < TN; ++j) {
      const int64_t col = t.n0 + wn_e * CFG::WTN + 16 * j + 4 * lq_e;
      float* dst = static_cast<float*>(t.C) + row * t.ldc + col;
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

// The two pipeline stages of a kernel, as distinct LDS arrays.
#define FP8BLK_DECLARE_STAGES(CFG)                                   \
  __shared__ __align__(16) uint8_t s_ops0[CFG::BUF_BYTES];           \
  __shared__ __align__(16) uint8_t s_ops1[CFG::BUF_BYTES];           \
  __shared__ __align__(16) float s_sc0[CFG::SC_FLOATS];              \
  __shared__ __align__(16) float s_sc1[CFG::SC_FLOATS]

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

template <class CFG, bool OPB_T, bool ROW128, bool P2, int OM>
__global__ __launch_bounds__(CFG::NT) void k_gemm(int64_t M, int64_t N, int64_t K, const uint8_t* __restrict__ A,
                                                   int64_t lda, const float* __restrict__ sA,
                                                   const uint8_t* __restrict__ B, int64_t ldb,
                                                   const float* __restrict__ sB, int64_t sB_ld,
                                                   void* __restrict__ C, int64_t ldc, int64_t tiles_m,
                                                   int64_t tiles_n, float* __restrict__ partials, int groups_per_split,
                                                   float* __restrict__ sQ) {
  FP8BLK_DECLARE_STAGES(CFG);
  int64_t tm, tn;
  tile_of(blockIdx.x, gridDim.x, tiles_m, tiles_n, tm, tn);
  // Split K: workgroup row blockIdx.y computes the partial product of K
  // groups [y*groups_per_split, ...) into its own [M][N] slice of `partials`.
  const int G = (int)(K / 128);
  // (Only FP32-output kernels are split: a split GEMM writes FP32 partials
  // and the reduction writes BF16 when asked to.)
  const int split = blockIdx.y;
  if (gridDim.y > 1) {  // partial slices of pitch N rounded up to 4 floats (16-byte rows)
    const int64_t Np = (N + 3) & ~int64_t(3);
    C = partials + (int64_t)split * M * Np;
    ldc = Np;
  }
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
  t.C = out_row(C, ldc, m0, out_elem_bytes(OM));
  t.ldc = ldc;
  t.sQ = sQ;
  t.sQ_ld = M;
  t.m0 = m0;
  t.K = K;
  t.g0 = split * groups_per_split;
  t.g1 = t.g0 + groups_per_split < G ? t.g0 + groups_per_split : G;
  gemm_tile<CFG, OPB_T, ROW128, P2, OM>(t, s_ops0, s_ops1, s_sc0, s_sc1);
}

// Partial row tiles of the grouped GEMM: waves whose rows all lie past the
// expert's last row skip their MFMAs and folds, and A copies of such rows
// are not issued.  Measured (interleaved, one box, bitwise identical): MoE
// up 3.26 -> 3.23 ms, down 2.055 -> 2.025 ms, down Dgrad 1.69 -> 1.68 ms.
// An L2 prefetch of each tile's weight slab 2-4 groups ahead (4-byte copies
// into a dummy LDS area) made all three 10-13 % slower and was dropped.
// Balancing the real tiles over the 8 XCDs (k_grouped_gemm, in place of a
// remap over the whole upper-bound grid, which left the MoE shapes' tiles to
// six XCDs, 1.27x the balanced share on the busiest): MoE up 3.35 ->
// 2.94 ms, down 2.15 -> 1.81 ms, down Dgrad 1.72 -> 1.45 ms (interleaved, one
// box, bitwise identical), so a grouped tile now takes within a few percent of
// a dense tile's time (2.94 ms over 25.2 tiles per CU).
#ifndef FP8BLK_GROUPED_SKIP
#define FP8BLK_GROUPED_SKIP 1
#endif
#ifndef FP8BLK_GROUPED_REG_CHUNKS
#define FP8BLK_GROUPED_REG_CHUNKS 4
#endif
// Grouped: tiles are enumerated expert by expert, within an expert column
// tile by column tile, row tiles innermost, so that concurrently running
// workgroups share each expert's weight tile.  The per-expert row counts are
// read from the device-resident offsets (a wave-level scan of the experts' tile
// counts), so the host never synchronizes; surplus workgroups of the
// upper-bound grid exit.
template <class CFG, bool OPB_T, bool P2, int OM>
__global__ __launch_bounds__(CFG::NT) void k_grouped_gemm(int64_t G, const int32_t* __restrict__ offsets,
                                                           int64_t M_total, int64_t N, int64_t K,
                                                           const uint8_t* __restrict__ A, int64_t lda,
                                                           const float* __restrict__ sA,
                                                           const uint8_t* __restrict__ B, int64_t ldb,
                                                           int64_t strideB, const float* __restrict__ sB,
                                                           int64_t stride_sB, int64_t sB_ld,
                                                           void* __restrict__ C, int64_t ldc, int64_t tiles_n) {
  FP8BLK_DECLARE_STAGES(CFG);
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  // Tiles of an expert: its row tiles times the column tiles.  The grid is
  // below 2^31 workgroups and covers every tile, so the counts fit 32 bits.
  auto expert_tiles = [&](int64_t ee) -> int32_t {
    if (ee >= G) return 0;
    const int64_t rows = (int64_t)offsets[ee + 1] - (int64_t)offsets[ee];
    return (int32_t)(((rows + CFG::BM - 1) / CFG::BM) * tiles_n);
  };
  // Each wave walks the experts 64 at a time, one per lane, with an
  // inclusive scan of their tile counts (lane exchanges only; every wave
  // reaches the same answers): first the total, then the expert that owns
  // tile `lin` and that tile's index within the expert.  Up to
  // 64 * FP8BLK_GROUPED_REG_CHUNKS experts, the counts are loaded once, all
  // chunks at the same time, and both passes run on registers: the
  // workgroup's start then waits for one load latency instead of one per
  // chunk and pass.  Measured (interleaved, one box, bitwise identical) on
  // the 256-expert MoE shapes: down 1.876 -> 1.754 ms (44 tiles per CU),
  // up 2.99 -> 2.98 ms, down Dgrad 1.46 -> 1.47 ms (25 and 13 tiles per CU).
  constexpr int RC = FP8BLK_GROUPED_REG_CHUNKS > 0 ? FP8BLK_GROUPED_REG_CHUNKS : 1;
  const bool in_regs = FP8BLK_GROUPED_REG_CHUNKS > 0 && G <= 64 * RC;
  int32_t cnt[RC], incl[RC];
  int64_t base[RC];
  int64_t total = 0;
  if (in_regs) {
#pragma unroll
    for (int c = 0; c < RC; ++c) cnt[c] = expert_tiles(64 * c + lane);
#pragma unroll
    for (int c = 0; c < RC; ++c) {
      incl[c] = wave_inclusive_sum(cnt[c]);
      base[c] = total;
      total = wave_uniform(total + __shfl(incl[c], 63));
    }
  } else {
    for (int64_t e0 = 0; e0 < G; e0 += 64)
      total = wave_uniform(total + __shfl(wave_inclusive_sum(expert_tiles(e0 + lane)), 63));
  }
  // Workgroups are dealt to the 8 XCDs round-robin: workgroup b runs on XCD
  // b % 8, as that XCD's (b / 8)-th.  XCD x takes the contiguous run
  // [x * per, (x + 1) * per) of the `total` real tiles, so that the XCDs get
  // equal shares and one XCD's workgroups share each expert's weight and
  // activation panels through its L2.  (The grid is an upper bound padded to
  // a multiple of 8; remapping over the whole grid left the real tiles to
  // the first six XCDs of the MoE shapes.)
  const int64_t per = (total + 7) / 8, slot = blockIdx.x / 8;
  if (slot >= per) return;  // surplus workgroup (uniform across the block)
  const int64_t lin = (int64_t)(blockIdx.x % 8) * per + slot;
  if (lin >= total) return;

  int64_t e = -1, local = 0;
  if (in_regs) {
#pragma unroll
    for (int c = 0; c < RC; ++c) {
      const int64_t lo = base[c] + incl[c] - cnt[c];
      const uint64_t who = __ballot(64 * c + lane < G && lin >= lo && lin < base[c] + incl[c]);
      if (who != 0 && e < 0) {
        const int src = __ffsll((unsigned long long)who) - 1;
        e = wave_uniform(64 * c + src);
        local = wave_uniform(lin - __shfl(lo, src));
      }
    }
  } else {
    int64_t b = 0;
    for (int64_t e0 = 0; e0 < G; e0 += 64) {
      const int64_t ee = e0 + lane;
      const int32_t n = expert_tiles(ee);
      const int32_t in = wave_inclusive_sum(n);
      const int64_t lo = b + in - n;
      const uint64_t who = __ballot(ee < G && lin >= lo && lin < b + in);
      if (who) {
        const int src = __ffsll((unsigned long long)who) - 1;
        e = wave_uniform(e0 + src);
        local = wave_uniform(lin - __shfl(lo, src));
        break;
      }
      b = wave_uniform(b + __shfl(in, 63));
    }
  }
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
  t.C = out_row(C, ldc, m0, out_elem_bytes(OM));
  t.ldc = ldc;
  t.K = K;
  t.g0 = 0;
  t.g1 = (int)(K / 128);
  gemm_tile<CFG, OPB_T, false, P2, OM, FP8BLK_GROUPED_SKIP != 0>(t, s_ops0, s_ops1, s_sc0, s_sc1);
}

// Grouped Wgrad of MoE experts: dW_e = X_e^T dY_e for every expert e, both
// operands 128x1-quantized along tokens inside each expert (ragged token
// groups, token_groups.h) and stored transposed, so that expert e's K range
// is its own group slots [PG[e], PG[e] + n_e) of the shared code matrices.
// Every expert's output has the same M x N tiles; tiles are enumerated expert
// by expert, column tile by column tile, row tiles innermost.  An expert
// without tokens gets dW_e = 0.
// One LDS stage: an expert's tiles have only 2-3 K groups on average, so the
// second stage bought little overlap and held the kernel to two workgroups
// per compute unit by LDS; with one stage (35 KB) three are resident (by
// registers) and one workgroup's stores overlap another's loads.  Measured
// (interleaved, one box, bitwise identical) on the MoE down projection's
// Wgrad: FP32 output 4.95 -> 4.63 ms, BF16 3.74 -> 3.41 ms.  Holding the
// kernel to 128 VGPRs for four workgroups per compute unit spills.
#ifndef FP8BLK_WGRAD_STAGES
#define FP8BLK_WGRAD_STAGES 1
#endif
template <class CFG, bool P2, int OM>
__global__ __launch_bounds__(CFG::NT) void k_grouped_wgrad(const int32_t* __restrict__ offsets, int64_t M, int64_t N,
                                                            const uint8_t* __restrict__ A, int64_t lda,
                                                            const float* __restrict__ sA,
                                                            const uint8_t* __restrict__ B, int64_t ldb,
                                                            const float* __restrict__ sB, void* __restrict__ C,
                                                            int64_t ldc, int64_t strideC, int64_t tiles_m,
                                                            int64_t tiles_n) {
#if FP8BLK_WGRAD_STAGES == 1
  __shared__ __align__(16) uint8_t s_ops0[CFG::BUF_BYTES];
  __shared__ __align__(16) float s_sc0[CFG::SC_FLOATS];
  uint8_t* s_ops1 = s_ops0;
  float* s_sc1 = s_sc0;
#else
  FP8BLK_DECLARE_STAGES(CFG);
#endif
  __shared__ int64_t s_red[CFG::NT];
  const int64_t per = tiles_m * tiles_n;
  const int64_t lin = blockIdx.x;
  // Column tiles fastest: consecutive workgroups write one 128-row band of
  // dW_e side by side (rows of 7168 FP32 are 28 KB apart), and with ids dealt
  // round-robin over the 8 XCDs each XCD keeps reading the same eighth of the
  // expert's B tiles.  Measured 14 % faster than row tiles fastest, whose
  // in-flight tiles write 512-byte pieces spread over the whole dW_e.
  const int64_t e = lin / per, rem = lin % per;
  const int64_t tm = rem / tiles_n, tn = rem % tiles_n;
  const int64_t pg = token_group_start<CFG::NT>(offsets, e, s_red);
  const int64_t ng = token_groups_of(offsets, e);
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
  t.sB_ld = N;
  t.C = out_row(out_row(C, strideC, e, out_elem_bytes(OM)), ldc, m0, out_elem_bytes(OM));
  t.ldc = ldc;
  t.K = 128 * (pg + ng);
  t.g0 = (int)pg;
  t.g1 = (int)(pg + ng);
  gemm_tile<CFG, true, true, P2, OM, false, FP8BLK_WGRAD_STAGES == 1>(t, s_ops0, s_ops1, s_sc0, s_sc1);
}

// Split-K reduction: C[m][n] = sum over s = 0 .. S-1, in that order, of the
// partial products partials[s][m][n] (FP32 additions).  The partial slices
// have row pitch Np = N rounded up to 4 floats, so every thread reads four
// consecutive columns as 16-byte words (columns from N to Np are padding,
// read but never stored).
__global__ __launch_bounds__(256) void k_splitk_reduce(const float* __restrict__ partials, int S, int64_t M,
                                                       int64_t N, void* __restrict__ Cv, int64_t ldc, int out_bf16) {
  const int64_t q = (int64_t)blockIdx.x * 256 + threadIdx.x;  // index of a 4-column chunk
  const int64_t Np = (N + 3) & ~int64_t(3);
  const int64_t cpr = Np / 4;
  const int64_t m = q / cpr, n = (q % cpr) * 4;
  if (m >= M) return;
  const int64_t MN = M * Np;
  const float* src = partials + m * Np + n;
  float4 a = *reinterpret_cast<const float4*>(src);
  for (int s = 1; s < S; ++s) {
    const float4 v = *reinterpret_cast<const float4*>(src + s * MN);
    a.x += v.x; a.y += v.y; a.z += v.z; a.w += v.w;
  }
  const float acc[4] = {a.x, a.y, a.z, a.w};
  if (out_bf16) {
    uint16_t* dst = static_cast<uint16_t*>(Cv) + m * ldc + n;
    if (n + 4 <= N)
      *reinterpret_cast<uint2*>(dst) = make_uint2(bf16_pack(acc[0], acc[1]), bf16_pack(acc[2], acc[3]));
    else
      for (int r = 0; r < 4 && n + r < N; ++r) dst[r] = (uint16_t)(bf16_pack(acc[r], 0.0f) & 0xFFFFu);
  } else {
    float* dst = static_cast<float*>(Cv) + m * ldc + n;
    if (n + 4 <= N)
      *reinterpret_cast<float4*>(dst) = make_float4(acc[0], acc[1], acc[2], acc[3]);
    else
      for (int r = 0; r < 4 && n + r < N; ++r) dst[r] = acc[r];
  }
}

// K splits for a dense GEMM: only when its 128 x 128 tiles cannot fill the
// compute units and K is long enough (at least FP8BLK_SPLITK_MIN_GROUPS
// groups) for the split to save more than the reduction's launch costs; each
// split keeps at least eight K groups, at most FP8BLK_SPLITK_MAX splits.
// Measured on 1024 x 1024 x K (one box): K = 4096 with 2 / 4 / 8 splits
// 27.6 / 22.0 / 24.4 us, K = 8192 40.7 / 28.8 / 28.9 us, K = 16384
// 70.7 / 44.7 / 38.9 us.
#ifndef FP8BLK_SPLITK_MIN_GROUPS
#define FP8BLK_SPLITK_MIN_GROUPS 16
#endif
#ifndef FP8BLK_SPLITK_MAX
#define FP8BLK_SPLITK_MAX 16
#endif
static int64_t splitk_count(int64_t M, int64_t N, int64_t K) {
  const int64_t big_tiles = ceil_div(M, BigCfg::BM) * ceil_div(N, BigCfg::BN);
  if (big_tiles >= 128) return 1;
  const int64_t G = K / 128;
  if (G < FP8BLK_SPLITK_MIN_GROUPS) return 1;
  const int64_t tiles = ceil_div(M, SmallCfg::BM) * ceil_div(N, SmallCfg::BN);
  const int64_t slots = 2 * (int64_t)device_cus();  // two 128 x 128 workgroups fit per CU
  int64_t S = ceil_div(slots, tiles);
  if (S > G / 8) S = G / 8;
  if (S > FP8BLK_SPLITK_MAX) S = FP8BLK_SPLITK_MAX;
  return S < 1 ? 1 : S;
}

// 224x256 tiles in place of 256x256 when they take fewer tile rows per CU:
// ceil(tiles / CUs) launch waves times the tile height.  On 256 CUs the
// 7168 x 2048 output (the Wgrad of a 7168-wide layer over a 2048-wide one)
// is 224 tiles of 256 rows, one launch wave with 32 CUs idle, or exactly 256
// tiles of 224 rows, each 7/8 of the MFMA work and 15/16 of the copies;
// square outputs such as 4096 x 4096 keep the 256-row tiles.  Measured
// (interleaved against 256-row tiles, one box, results bitwise identical):
// 7168 x 2048 x 4096 Wgrad 77.0 -> 73.8 us, power-of-two scales 70.8 -> 67.8;
// 4100 x 2050 x 7168 (153 -> 171 tiles) 104.5 -> 97.4 us, power-of-two
// 98.7 -> 101.6 (the one loss).
static bool use_tile224(int64_t M, int64_t N) {
  const int64_t cus = device_cus();
  const int64_t t256 = ceil_div(M, BigCfg::BM) * ceil_div(N, BigCfg::BN);
  const int64_t t224 = ceil_div(M, Big224Cfg::BM) * ceil_div(N, Big224Cfg::BN);
  return ceil_div(t224, cus) * Big224Cfg::BM < ceil_div(t256, cus) * BigCfg::BM;
}

static size_t splitk_bytes(int64_t M, int64_t N, int64_t K) {
  const int64_t S = splitk_count(M, N, K);
  const int64_t Np = (N + 3) & ~int64_t(3);
  return S > 1 ? (size_t)S * (size_t)M * (size_t)Np * sizeof(float) : 0;
}

template <class CFG, bool OPB_T, bool ROW128, bool P2>
static fp8blk_status_t launch_dense(int64_t M, int64_t N, int64_t K, const uint8_t* A, int64_t lda, const float* sA,
                                    const uint8_t* B, int64_t ldb, const float* sB, int64_t sB_ld, void* C,
                                    int64_t ldc, int out_bf16, float* partials, int64_t S, hipStream_t stream) {
  const int64_t tiles_m = ceil_div(M, CFG::BM), tiles_n = ceil_div(N, CFG::BN);
  const int64_t blocks = tiles_m * tiles_n;
  if (blocks > 0x7FFFFFFF) return FP8BLK_ERR_UNSUPPORTED;
  const int64_t G = K / 128;
  const int64_t per = ceil_div(G, S);
  S = ceil_div(G, per);  // no empty split
  if (out_bf16 && S == 1)
    hipLaunchKernelGGL((k_gemm<CFG, OPB_T, ROW128, P2, OUT_BF16>), dim3((unsigned)blocks), dim3(CFG::NT), 0, stream, M,
                       N, K, A, lda, sA, B, ldb, sB, sB_ld, C, ldc, tiles_m, tiles_n, partials, (int)per, nullptr);
  else
    hipLaunchKernelGGL((k_gemm<CFG, OPB_T, ROW128, P2, OUT_F32>), dim3((unsigned)blocks, (unsigned)S), dim3(CFG::NT), 0,
                       stream, M, N, K, A, lda, sA, B, ldb, sB, sB_ld, C, ldc, tiles_m, tiles_n, partials, (int)per,
                       nullptr);
  if (S > 1) {
    if (hipGetLastError() != hipSuccess) return FP8BLK_ERR_LAUNCH;
    const int64_t chunks = M * ceil_div(N, 4);  // N rounded up to 4 floats, in chunks of 4
    hipLaunchKernelGGL(k_splitk_reduce, dim3((unsigned)ceil_div(chunks, 256)), dim3(256), 0, stream, partials, (int)S,
                       M, N, C, ldc, out_bf16);
  }
  return launch_status();
}

template <class CFG, bool ROW128>
static fp8blk_status_t dispatch_dense(bool t, bool p2, int64_t M, int64_t N, int64_t K, const uint8_t* A,
                                      int64_t lda, const float* sA, const uint8_t* B, int64_t ldb, const float* sB,
                                      int64_t sB_ld, void* C, int64_t ldc, int ob, float* partials, int64_t S,
                                      hipStream_t st) {
  if (p2) {
    if (t) return launch_dense<CFG, true, ROW128, true>(M, N, K, A, lda, sA, B, ldb, sB, sB_ld, C, ldc, ob, partials, S, st);
    return launch_dense<CFG, false, ROW128, true>(M, N, K, A, lda, sA, B, ldb, sB, sB_ld, C, ldc, ob, partials, S, st);
  }
  if (t) return launch_dense<CFG, true, ROW128, false>(M, N, K, A, lda, sA, B, ldb, sB, sB_ld, C, ldc, ob, partials, S, st);
  return launch_dense<CFG, false, ROW128, false>(M, N, K, A, lda, sA, B, ldb, sB, sB_ld, C, ldc, ob, partials, S, st);
}

}  // namespace fp8blk

using namespace fp8blk;

// Per-lane copy offsets are 32-bit: operand pitches stay below 2^23 bytes.
static constexpr int64_t kMaxPitch = int64_t(1) << 23;

// Workspace that lets the dense GEMM split K (0: it never splits this
// shape); the grouped GEMM needs none.
extern "C" size_t fp8blk_workspace_bytes(int64_t M, int64_t N, int64_t K, int64_t G) {
  if (G > 1 || M <= 0 || N <= 0 || K <= 0 || K % 128 != 0) return 0;
  return splitk_bytes(M, N, K);
}

// Argument checks and tile/split choice shared by the dense entry points.
// `workspace` is the split-K partials buffer (S slices of M x N rounded up
// to 4 floats); with too small a workspace the GEMM runs in one pass, or,
// with `strict`, the call fails with FP8BLK_ERR_UNSUPPORTED.
static fp8blk_status_t gemm_dense(int64_t M, int64_t N, int64_t K, const uint8_t* A, int64_t lda, const float* sA,
                                  const uint8_t* B, int64_t ldb, int opB, const float* sB, int bscale_mode, void* C,
                                  int64_t ldc, void* workspace, size_t workspace_bytes, bool strict, void* stream) {
  if (M < 0 || N < 0 || K < 0) return FP8BLK_ERR_INVALID_ARG;
  const bool p2 = (opB & FP8BLK_GEMM_POW2_SCALES) != 0;
  const int ob = (opB & FP8BLK_GEMM_OUT_BF16) != 0;
  opB &= ~(FP8BLK_GEMM_POW2_SCALES | FP8BLK_GEMM_OUT_BF16);
  if (opB != FP8BLK_OP_N && opB != FP8BLK_OP_T) return FP8BLK_ERR_INVALID_ARG;
  if (bscale_mode != FP8BLK_BSCALE_BLOCK128 && bscale_mode != FP8BLK_BSCALE_ROW128) return FP8BLK_ERR_INVALID_ARG;
  if (K % 128 != 0) return FP8BLK_ERR_INVALID_ARG;
  if (M == 0 || N == 0) return FP8BLK_OK;
  if (K == 0) return FP8BLK_ERR_INVALID_ARG;
  if (!matrix_ok(A, M, K, lda, 1) || !matrix_ok(C, M, N, ldc, ob ? 2 : 4)) return FP8BLK_ERR_INVALID_ARG;
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
  const bool t = opB == FP8BLK_OP_T;
  // Split K when a large enough workspace is given and the tiles alone
  // cannot fill the GPU; otherwise one pass writes C directly.
  int64_t S = splitk_count(M, N, K);
  float* partials = nullptr;
  if (S > 1) {
    if (workspace != nullptr && workspace_bytes >= splitk_bytes(M, N, K) && aligned(workspace, 16))
      partials = static_cast<float*>(workspace);
    else if (strict)
      return FP8BLK_ERR_UNSUPPORTED;
    else
      S = 1;
  }
  // 256x256 tiles (or 224x256, see use_tile224) when they give at least
  // half a wave of workgroups over the 256 CUs, 128x128 tiles otherwise.
  const int64_t big_tiles = ceil_div(M, BigCfg::BM) * ceil_div(N, BigCfg::BN);
  const bool t224 = big_tiles >= 128 && use_tile224(M, N);
  if (bscale_mode == FP8BLK_BSCALE_ROW128) {
    if (t224)
      return dispatch_dense<Big224Cfg, true>(t, p2, M, N, K, A, lda, sA, B, ldb, sB, sB_ld, C, ldc, ob, partials, S, st);
    if (big_tiles >= 128)
      return dispatch_dense<BigCfg, true>(t, p2, M, N, K, A, lda, sA, B, ldb, sB, sB_ld, C, ldc, ob, partials, S, st);
    return dispatch_dense<SmallCfg, true>(t, p2, M, N, K, A, lda, sA, B, ldb, sB, sB_ld, C, ldc, ob, partials, S, st);
  }
  if (t224)
    return dispatch_dense<Big224Cfg, false>(t, p2, M, N, K, A, lda, sA, B, ldb, sB, sB_ld, C, ldc, ob, partials, S, st);
  if (big_tiles >= 128)
    return dispatch_dense<BigCfg, false>(t, p2, M, N, K, A, lda, sA, B, ldb, sB, sB_ld, C, ldc, ob, partials, S, st);
  return dispatch_dense<SmallCfg, false>(t, p2, M, N, K, A, lda, sA, B, ldb, sB, sB_ld, C, ldc, ob, partials, S, st);
}

extern "C" fp8blk_status_t fp8blk_gemm_fp8_blockscaled(int64_t M, int64_t N, int64_t K, const uint8_t* A, int64_t lda,
                                                       const float* sA, const uint8_t* B, int64_t ldb, int opB,
                                                       const float* sB, int bscale_mode, void* C, int64_t ldc,
                                                       void* workspace, size_t workspace_bytes, void* stream) {
  return gemm_dense(M, N, K, A, lda, sA, B, ldb, opB, sB, bscale_mode, C, ldc, workspace, workspace_bytes, false,
                    stream);
}

// ---- The same GEMM without any allocation --------------------------------
// For callers that cannot allocate (code under graph capture, serving loops,
// harnesses that forbid it): the split-K partials live in `scratch`, a
// file-scope device array of FP8BLK_NOALLOC_SCRATCH_BYTES that each GPU holds
// for the life of the process.  Its device address is looked up once per
// device (hipGetSymbolAddress with that device current) and kept; host code
// passes only that address to the kernels, never the array's name.
static __device__ __align__(256) float scratch[FP8BLK_NOALLOC_SCRATCH_BYTES / sizeof(float)];

static float* scratch_on_current_device() {
  static std::mutex mu;
  static std::atomic<float*> ptrs[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return nullptr;
  float* p = ptrs[dev].load(std::memory_order_acquire);
  if (p != nullptr) return p;
  std::lock_guard<std::mutex> lock(mu);
  p = ptrs[dev].load(std::memory_order_relaxed);
  if (p == nullptr) {
    void* q = nullptr;
    if (hipGetSymbolAddress(&q, HIP_SYMBOL(scratch)) != hipSuccess || q == nullptr) return nullptr;
    p = static_cast<float*>(q);
    ptrs[dev].store(p, std::memory_order_release);
  }
  return p;
}

extern "C" fp8blk_status_t fp8blk_gemm_fp8_blockscaled_noalloc(int64_t M, int64_t N, int64_t K, const uint8_t* A,
                                                               int64_t lda, const float* sA, const uint8_t* B,
                                                               int64_t ldb, int opB, const float* sB, int bscale_mode,
                                                               void* C, int64_t ldc, void* stream) {
  // Shapes whose partials would not fit are rejected before anything is
  // looked up or enqueued (the split count is the workspace entry point's).
  if (M > 0 && N > 0 && K > 0 && K % 128 == 0 && splitk_bytes(M, N, K) > FP8BLK_NOALLOC_SCRATCH_BYTES)
    return FP8BLK_ERR_UNSUPPORTED;
  float* ws = nullptr;
  if (M > 0 && N > 0 && K > 0 && K % 128 == 0 && splitk_bytes(M, N, K) > 0) {
    ws = scratch_on_current_device();
    if (ws == nullptr) return FP8BLK_ERR_LAUNCH;
  }
  return gemm_dense(M, N, K, A, lda, sA, B, ldb, opB, sB, bscale_mode, C, ldc, ws,
                    ws != nullptr ? (size_t)FP8BLK_NOALLOC_SCRATCH_BYTES : 0, true, stream);
}

// Dense GEMM with the output quantized on store (1x128 tiles along each row
// of the BF16-rounded result); block-scaled B only, never split.
template <class CFG, bool OPB_T, bool P2>
static fp8blk_status_t launch_q(int64_t M, int64_t N, int64_t K, const uint8_t* A, int64_t lda, const float* sA,
                                const uint8_t* B, int64_t ldb, const float* sB, int64_t sB_ld, uint8_t* Q, int64_t ldq,
                                float* sQ, bool qpow2, hipStream_t st) {
  const int64_t tiles_m = ceil_div(M, CFG::BM), tiles_n = ceil_div(N, CFG::BN);
  const int64_t blocks = tiles_m * tiles_n;
  if (blocks > 0x7FFFFFFF) return FP8BLK_ERR_UNSUPPORTED;
  const int per = (int)(K / 128);
  if (qpow2)
    hipLaunchKernelGGL((k_gemm<CFG, OPB_T, false, P2, OUT_Q_POW2>), dim3((unsigned)blocks), dim3(CFG::NT), 0, st, M, N,
                       K, A, lda, sA, B, ldb, sB, sB_ld, Q, ldq, tiles_m, tiles_n, nullptr, per, sQ);
  else
    hipLaunchKernelGGL((k_gemm<CFG, OPB_T, false, P2, OUT_Q>), dim3((unsigned)blocks), dim3(CFG::NT), 0, st, M, N, K,
                       A, lda, sA, B, ldb, sB, sB_ld, Q, ldq, tiles_m, tiles_n, nullptr, per, sQ);
  return launch_status();
}

template <class CFG>
static fp8blk_status_t dispatch_q(bool t, bool p2, int64_t M, int64_t N, int64_t K, const uint8_t* A, int64_t lda,
                                  const float* sA, const uint8_t* B, int64_t ldb, const float* sB, int64_t sB_ld,
                                  uint8_t* Q, int64_t ldq, float* sQ, bool qpow2, hipStream_t st) {
  if (p2) {
    if (t) return launch_q<CFG, true, true>(M, N, K, A, lda, sA, B, ldb, sB, sB_ld, Q, ldq, sQ, qpow2, st);
    return launch_q<CFG, false, true>(M, N, K, A, lda, sA, B, ldb, sB, sB_ld, Q, ldq, sQ, qpow2, st);
  }
  if (t) return launch_q<CFG, true, false>(M, N, K, A, lda, sA, B, ldb, sB, sB_ld, Q, ldq, sQ, qpow2, st);
  return launch_q<CFG, false, false>(M, N, K, A, lda, sA, B, ldb, sB, sB_ld, Q, ldq, sQ, qpow2, st);
}

extern "C" fp8blk_status_t fp8blk_gemm_fp8_blockscaled_q1x128(int64_t M, int64_t N, int64_t K, const uint8_t* A,
                                                              int64_t lda, const float* sA, const uint8_t* B,
                                                              int64_t ldb, int opB, const float* sB, uint8_t* Q,
                                                              int64_t ldq, float* sQ, uint32_t qflags, void* stream) {
  if (M < 0 || N < 0 || K < 0) return FP8BLK_ERR_INVALID_ARG;
  if (qflags & ~FP8BLK_SCALE_POW2) return FP8BLK_ERR_INVALID_ARG;
  const bool p2 = (opB & FP8BLK_GEMM_POW2_SCALES) != 0;
  opB &= ~FP8BLK_GEMM_POW2_SCALES;
  if (opB != FP8BLK_OP_N && opB != FP8BLK_OP_T) return FP8BLK_ERR_INVALID_ARG;
  if (K % 128 != 0) return FP8BLK_ERR_INVALID_ARG;
  if (M == 0 || N == 0) return FP8BLK_OK;
  if (K == 0) return FP8BLK_ERR_INVALID_ARG;
  if (!matrix_ok(A, M, K, lda, 1) || !matrix_ok(Q, M, N, ldq, 1)) return FP8BLK_ERR_INVALID_ARG;
  if (opB == FP8BLK_OP_N ? !matrix_ok(B, K, N, ldb, 1) : !matrix_ok(B, N, K, ldb, 1)) return FP8BLK_ERR_INVALID_ARG;
  if (lda >= kMaxPitch || ldb >= kMaxPitch) return FP8BLK_ERR_UNSUPPORTED;
  const int64_t G = K / 128, NB = ceil_div(N, 128);
  if (!vec_ok(sA, G * M) || !vec_ok(sB, G * NB) || !vec_ok(sQ, NB * M)) return FP8BLK_ERR_INVALID_ARG;
  const int64_t sB_ld = opB == FP8BLK_OP_N ? NB : G;
  const bool t = opB == FP8BLK_OP_T, qpow2 = (qflags & FP8BLK_SCALE_POW2) != 0;
  hipStream_t st = as_stream(stream);
  const int64_t big_tiles = ceil_div(M, BigCfg::BM) * ceil_div(N, BigCfg::BN);
  if (big_tiles >= 128) return dispatch_q<BigCfg>(t, p2, M, N, K, A, lda, sA, B, ldb, sB, sB_ld, Q, ldq, sQ, qpow2, st);
  return dispatch_q<SmallCfg>(t, p2, M, N, K, A, lda, sA, B, ldb, sB, sB_ld, Q, ldq, sQ, qpow2, st);
}

extern "C" fp8blk_status_t fp8blk_grouped_gemm_fp8_blockscaled(
    int64_t G, const int32_t* group_offsets, int64_t M_total, int64_t max_group_rows, int64_t N, int64_t K,
    const uint8_t* A, int64_t lda, const float* sA, const uint8_t* B, int64_t ldb, int64_t strideB, int opB,
    const float* sB, int64_t stride_sB, void* C, int64_t ldc, void* workspace, size_t workspace_bytes,
    void* stream) {
  (void)workspace;
  (void)workspace_bytes;
  // 256 x 256 tiles on the row-pipelined loop.  With 256 experts of mean
  // 256 rows (skewed), 256-row tiles pad the experts' row ranges more than
  // 128-row tiles (64 % against 79 % useful rows), but each group's copies
  // feed four times the MFMA work, and the copies, not the matrix cores,
  // bound these kernels: measured against 128 x 128 tiles (interleaved, one
  // box, bitwise identical, both before the XCD balance of the kernel) MoE
  // up 3.32 / 3.50 ms, down 2.08 / 2.16 ms, down Dgrad 1.72 / 1.71 ms.
  using CFG = BigCfg;
  if (G < 0 || M_total < 0 || N < 0 || K < 0 || max_group_rows < 0) return FP8BLK_ERR_INVALID_ARG;
  const bool p2 = (opB & FP8BLK_GEMM_POW2_SCALES) != 0;
  const int ob = (opB & FP8BLK_GEMM_OUT_BF16) != 0;
  opB &= ~(FP8BLK_GEMM_POW2_SCALES | FP8BLK_GEMM_OUT_BF16);
  if (opB != FP8BLK_OP_N && opB != FP8BLK_OP_T) return FP8BLK_ERR_INVALID_ARG;
  if (K % 128 != 0) return FP8BLK_ERR_INVALID_ARG;
  if (G == 0 || M_total == 0 || N == 0) return FP8BLK_OK;
  if (K == 0 || group_offsets == nullptr || !aligned(group_offsets, 4)) return FP8BLK_ERR_INVALID_ARG;
  if (!matrix_ok(A, M_total, K, lda, 1) || !matrix_ok(C, M_total, N, ldc, ob ? 2 : 4)) return FP8BLK_ERR_INVALID_ARG;
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
#define FP8BLK_GROUPED_LAUNCH(T_, P2_, OB_)                                                                      \
  hipLaunchKernelGGL((k_grouped_gemm<CFG, T_, P2_, OB_>), dim3((unsigned)blocks), dim3(CFG::NT), 0, st, G,          \
                     group_offsets, M_total, N, K, A, lda, sA, B, ldb, strideB, sB, stride_sB, sB_ld, C, ldc, tiles_n)
#define FP8BLK_GROUPED_LAUNCH_OB(T_, P2_) \
  if (ob) FP8BLK_GROUPED_LAUNCH(T_, P2_, OUT_BF16); else FP8BLK_GROUPED_LAUNCH(T_, P2_, OUT_F32)
  if (opB == FP8BLK_OP_T) {
    if (p2) { FP8BLK_GROUPED_LAUNCH_OB(true, true); } else { FP8BLK_GROUPED_LAUNCH_OB(true, false); }
  } else {
    if (p2) { FP8BLK_GROUPED_LAUNCH_OB(false, true); } else { FP8BLK_GROUPED_LAUNCH_OB(false, false); }
  }
#undef FP8BLK_GROUPED_LAUNCH_OB
#undef FP8BLK_GROUPED_LAUNCH
  return launch_status();
}

extern "C" fp8blk_status_t fp8blk_grouped_wgrad_fp8_blockscaled(int64_t G, const int32_t* group_offsets, int64_t T,
                                                                int64_t M, int64_t N, const uint8_t* AT,
                                                                int64_t ldaT, const float* sA, const uint8_t* BT,
                                                                int64_t ldbT, const float* sB, uint32_t flags,
                                                                void* C, int64_t ldc, int64_t strideC,
                                                                void* stream) {
  // 128 x 128 tiles: the per-column scales of both operands (ROW128) need the
  // registers of the smaller tile.
  using CFG = RowCfg;
  if (G < 0 || T < 0 || M < 0 || N < 0) return FP8BLK_ERR_INVALID_ARG;
  if (flags & ~(uint32_t)(FP8BLK_GEMM_POW2_SCALES | FP8BLK_GEMM_OUT_BF16)) return FP8BLK_ERR_INVALID_ARG;
  const bool p2 = (flags & FP8BLK_GEMM_POW2_SCALES) != 0;
  const int ob = (flags & FP8BLK_GEMM_OUT_BF16) != 0;
  if (G == 0 || M == 0 || N == 0) return FP8BLK_OK;
  const int64_t slots = fp8blk_token_group_slots(T, G);
  if (group_offsets == nullptr || !aligned(group_offsets, 4)) return FP8BLK_ERR_INVALID_ARG;
  if (T > 0) {  // with no tokens the operands are not read (every dW_e = 0)
    if (!matrix_ok(AT, M, 128 * slots, ldaT, 1) || !matrix_ok(BT, N, 128 * slots, ldbT, 1))
      return FP8BLK_ERR_INVALID_ARG;
    if (!vec_ok(sA, slots * M) || !vec_ok(sB, slots * N)) return FP8BLK_ERR_INVALID_ARG;
  }
  if (!matrix_ok(C, M, N, ldc, ob ? 2 : 4) || strideC < M * ldc || strideC % (ob ? 8 : 4) != 0)
    return FP8BLK_ERR_INVALID_ARG;
  if (ldaT >= kMaxPitch || ldbT >= kMaxPitch || slots > 0x7FFFFFFF / 2) return FP8BLK_ERR_UNSUPPORTED;
  const int64_t tiles_m = ceil_div(M, CFG::BM), tiles_n = ceil_div(N, CFG::BN);
  const int64_t blocks = G * tiles_m * tiles_n;
  if (blocks > 0x7FFFFFFF) return FP8BLK_ERR_UNSUPPORTED;
  hipStream_t st = as_stream(stream);
#define FP8BLK_WGRAD_LAUNCH(P2_, OB_)                                                                             \
  hipLaunchKernelGGL((k_grouped_wgrad<CFG, P2_, OB_>), dim3((unsigned)blocks), dim3(CFG::NT), 0, st, group_offsets, M, \
                     N, AT, ldaT, sA, BT, ldbT, sB, C, ldc, strideC, tiles_m, tiles_n)
  if (p2) {
    if (ob) FP8BLK_WGRAD_LAUNCH(true, OUT_BF16); else FP8BLK_WGRAD_LAUNCH(true, OUT_F32);
  } else {
    if (ob) FP8BLK_WGRAD_LAUNCH(false, OUT_BF16); else FP8BLK_WGRAD_LAUNCH(false, OUT_F32);
  }
#undef FP8BLK_WGRAD_LAUNCH
  return launch_status();
}
