/*
 * libfp8blk — fine-grained (tile/block-scaled) FP8 quantization and FP8 GEMM
 * for AMD Instinct MI355X (gfx950).
 *
 * The method: activations are quantized to E4M3 with one FP32 scale per 1x128
 * tile (one token, 128 channels) and weights with one scale per 128x128 block
 * [p1¶3, the description of Figure 7(a)]; the tile maximum is taken online at
 * quantization time [p2¶4]; E4M3 is used for every tensor [p2¶2]; power-of-two
 * scales are used for some activations [p2¶4]; the GEMM multiplies the FP8
 * codes and promotes each 128-deep K group's partial sum into an FP32
 * accumulator, multiplying in the group's scales there [p2¶3, p2¶4]; Fprop,
 * Dgrad and Wgrad all run in FP8 [p1¶3, Figure 6], Wgrad on operands
 * re-quantized into 128x1 tiles along tokens [p5¶4]; MoE expert projections
 * use a per-expert (grouped) variant [p2¶4].
 *
 * Citations [pN¶k] name the N-th page of the source collection and its k-th
 * paragraph counted from the page heading:
 *   p1 = xn--9g3bo1gtkw0l8ubf92bgle.kr (board qna, wr_id 85187)
 *   p2 = inprokorea.com (board free, wr_id 735329)
 *   p5 = inprokorea.com (board free, wr_id 890463)
 *
 * Numerics fixed by this library where the pages are silent:
 *   E4M3 is OCP "e4m3fn" (bias 7, no infinities, largest finite 448).
 *   scale s = fl32(amax / 448) (IEEE division); with FP8BLK_SCALE_POW2,
 *   s = the smallest power of two >= amax / 448 (exact); amax = 0 gives s = 1.
 *   code q = E4M3(fl32(x / s)), round to nearest even, saturating to +-448,
 *   sign kept for values that round to zero.  Dequantized value: dec(q) * s.
 *
 * Conventions for every entry point:
 *   - All tensor pointers are DEVICE pointers (hipMalloc'd or equivalent) on
 *     the current HIP device.  The caller owns every buffer; the library never
 *     allocates, frees or synchronizes.  Between calls it keeps only two
 *     per-device lookups, each made once and thread-safe: the device's
 *     compute-unit count (which sets the split-K choice) and, for
 *     fp8blk_gemm_fp8_blockscaled_noalloc, the address of its scratch array.
 *   - `stream` is a hipStream_t passed as void* (NULL = the default stream).
 *     All work is enqueued asynchronously on it.
 *   - BF16 inputs are raw bit patterns (uint16_t).  Matrices are row-major
 *     with leading dimension (row pitch) in ELEMENTS.
 *   - Inputs and outputs must not overlap.
 *   - Sizes of zero are valid and enqueue nothing.
 *   - Arguments are validated on the host before anything is enqueued; an
 *     invalid call returns FP8BLK_ERR_INVALID_ARG and touches nothing.
 *     FP8BLK_ERR_LAUNCH reports a failed kernel launch.  Faults inside a
 *     kernel surface at the caller's next synchronization (HIP convention).
 *   - Alignment: every matrix pointer must be 16-byte aligned and every row
 *     pitch a multiple of 16 bytes (8 BF16, 16 FP8 codes, 4 FP32); scale
 *     pointers must be 4-byte aligned.
 *   - Extent: a matrix with R rows and pitch P occupies R*P elements; the
 *     GEMMs may read (never write) the padding between the row length and
 *     the pitch, including that of the last row.
 */
#ifndef LIBFP8BLK_H
#define LIBFP8BLK_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  FP8BLK_OK = 0,
  FP8BLK_ERR_INVALID_ARG = 1, /* null pointer, negative size, bad pitch/alignment, unknown flag/enum */
  FP8BLK_ERR_UNSUPPORTED = 2, /* valid but not implemented combination */
  FP8BLK_ERR_LAUNCH = 3       /* hipGetLastError() reported a failure after a launch */
} fp8blk_status_t;

/* flags for the quantizers */
#define FP8BLK_SCALE_POW2 0x1u /* power-of-two scales [p2¶4] */

/* storage of the GEMM's B operand */
enum { FP8BLK_OP_N = 0, /* B stored [K][N] (row pitch ldb >= N)            */
       FP8BLK_OP_T = 1  /* B stored [N][K] (row pitch ldb >= K)            */ };

/* Flag OR'ed into `opB` of either GEMM: every scale of A and B is a power of
 * two in [2^-126, 2^127] (as written by the quantizers with
 * FP8BLK_SCALE_POW2, which the pages use for some activations [p2¶4]).  The
 * matrix cores then apply the scales themselves as E8M0 block scales and add
 * each group's scaled product to the FP32 accumulator (round to nearest
 * even), so no separate promotion step is needed.  A scale that is not such
 * a power of two is read as 2^(its biased exponent - 127): the result is
 * then wrong, not an error. */
#define FP8BLK_GEMM_POW2_SCALES 0x100
/* Flag OR'ed into `opB` of the dense and grouped GEMMs (and into `flags` of
 * the grouped Wgrad): C is BF16 instead of FP32.  Each output is the same
 * FP32 result rounded to the nearest BF16 (ties to even; NaN stays NaN,
 * values beyond the BF16 range become infinities).  C then holds uint16_t
 * BF16 bit patterns, its pitch ldc (and strideC) counts BF16 elements, and
 * the alignment rules apply to the BF16 matrix (pitch a multiple of 8). */
#define FP8BLK_GEMM_OUT_BF16 0x200

/* B scale layouts */
enum { FP8BLK_BSCALE_BLOCK128 = 0, /* one scale per 128x128 block of B as stored:
                                      [K/128][ceil(N/128)] for OP_N,
                                      [ceil(N/128)][K/128] for OP_T          */
       FP8BLK_BSCALE_ROW128 = 1    /* one scale per column n per K group:
                                      [K/128][N] (B quantized with 128-deep
                                      tiles along K, e.g. by quantize_128x1) */ };

/*
 * 1x128 quantization of activations (per token per 128 channels) [p1¶3],
 * amax taken online per tile [p2¶4].
 *   x   [M][K] BF16, pitch ldx >= K.
 *   q   [M][K] E4M3 codes (uint8), pitch ldq >= K.
 *   s   [ceil(K/128)][M] FP32, dense: s[g*M + m] scales row m, columns
 *       [128g, 128g+128); a partial last group uses the columns present.
 *   flags: 0 or FP8BLK_SCALE_POW2.
 */
fp8blk_status_t fp8blk_quantize_1x128(const uint16_t* x, int64_t M, int64_t K, int64_t ldx,
                                      uint8_t* q, int64_t ldq, float* s, uint32_t flags,
                                      void* stream);

/*
 * 128x1 quantization along tokens with transposed output, the Wgrad operand
 * layout [p5¶4].
 *   x   [T][C] BF16 (tokens x channels), pitch ldx >= C.
 *   qT  [C][T] E4M3 codes, pitch ldqT >= T: qT[c*ldqT + t] is token t, channel c.
 *   s   [ceil(T/128)][C] FP32, dense: s[g*C + c] scales channel c over tokens
 *       [128g, 128g+128).  qT/s equal quantize_1x128 applied to x transposed.
 *   flags: 0 or FP8BLK_SCALE_POW2.
 *   FP8BLK_ERR_UNSUPPORTED if ceil(T/128) > 65535 (T above 8 388 480 tokens:
 *   the token groups are one launch dimension).
 */
fp8blk_status_t fp8blk_quantize_128x1(const uint16_t* x, int64_t T, int64_t C, int64_t ldx,
                                      uint8_t* qT, int64_t ldqT, float* s, uint32_t flags,
                                      void* stream);

/*
 * 128x128 block quantization of weights (per 128 input channels per 128
 * output channels) [p1¶3].
 *   w   [R][C] BF16, pitch ldw >= C.
 *   q   [R][C] E4M3 codes, pitch ldq >= C.
 *   s   [ceil(R/128)][ceil(C/128)] FP32, dense; partial edge blocks use the
 *       elements present.
 *   flags: 0 or FP8BLK_SCALE_POW2.
 */
fp8blk_status_t fp8blk_quantize_block128(const uint16_t* w, int64_t R, int64_t C, int64_t ldw,
                                         uint8_t* q, int64_t ldq, float* s, uint32_t flags,
                                         void* stream);

/*
 * Both operands of an Fprop GEMM in one launch: exactly
 *   fp8blk_quantize_1x128(x, M, K, ldx, qx, ldqx, sx, xflags) and
 *   fp8blk_quantize_block128(w, R, C, ldw, qw, ldqw, sw, wflags)
 * (same arguments, layouts and results, bit for bit), with the two
 * tensors' tiles in one grid so that one launch ramp and tail serve both.
 * The four outputs must not overlap each other or the inputs.  Either
 * tensor may be empty (then only the other is quantized).
 */
fp8blk_status_t fp8blk_quantize_1x128_block128(const uint16_t* x, int64_t M, int64_t K, int64_t ldx,
                                               uint8_t* qx, int64_t ldqx, float* sx, uint32_t xflags,
                                               const uint16_t* w, int64_t R, int64_t C, int64_t ldw,
                                               uint8_t* qw, int64_t ldqw, float* sw, uint32_t wflags,
                                               void* stream);

/*
 * Re-quantization of a cached 1x128-quantized activation into transposed
 * 128x1 tiles: read, dequantize, transpose, re-quantize, store [p5¶4].
 *   q   [T][C] E4M3 codes from fp8blk_quantize_1x128 (pitch ldq >= C),
 *   sq  [ceil(C/128)][T] its FP32 scales.
 *   The dequantized value is fl32(dec(q) * s); it is then quantized exactly
 *   as fp8blk_quantize_128x1 quantizes a value.
 *   qT  [C][T] E4M3 codes (pitch ldqT >= T), sT [ceil(T/128)][C] FP32.
 *   flags: 0 or FP8BLK_SCALE_POW2.
 *   FP8BLK_ERR_UNSUPPORTED if ceil(T/128) > 65535, as for quantize_128x1.
 */
fp8blk_status_t fp8blk_requantize_128x1_from_1x128(const uint8_t* q, const float* sq, int64_t T,
                                                   int64_t C, int64_t ldq, uint8_t* qT,
                                                   int64_t ldqT, float* sT, uint32_t flags,
                                                   void* stream);

/*
 * Block-scaled FP8 GEMM:  C[m][n] = sum_g sA[g][m] * sB(g,n) * P_g[m][n],
 *   P_g[m][n] = sum over the 128-deep K group g of dec(A[m][k]) * dec(B[k][n]).
 * Each group's partial is formed by the matrix cores (one MFMA per 16x16
 * output tile and group) and promoted into an FP32 accumulator with one FMA
 * by the scale product [p2¶3, p2¶4].
 *   A  [M][K] E4M3 codes, pitch lda >= K; sA [K/128][M] FP32 (1x128 scales).
 *   B  [K][N] (opB = FP8BLK_OP_N, pitch ldb >= N) or [N][K] (FP8BLK_OP_T,
 *      pitch ldb >= K) E4M3 codes; sB per `bscale_mode`.
 *   C  [M][N] FP32 (BF16 with FP8BLK_GEMM_OUT_BF16), pitch ldc >= N
 *      (overwritten).
 *   K must be a positive multiple of 128 (M, N arbitrary); lda and ldb
 *   must be below 2^23 (FP8BLK_ERR_UNSUPPORTED otherwise).
 *   Roles: Fprop Y = X W (A = 1x128-quantized X, B = W [K][N] block-scaled,
 *   OP_N); Dgrad dX = dY W^T (A = 1x128-quantized dY, B = the same W read as
 *   OP_T with its own block scales); Wgrad dW = X^T dY (A = 128x1-quantized
 *   X as [d_in][T], B = 128x1-quantized dY as [d_out][T] with OP_T and
 *   FP8BLK_BSCALE_ROW128) [p1¶3; p5¶4].
 *   workspace / workspace_bytes: optional DEVICE scratch (16-byte aligned,
 *   owned by the caller, contents on entry irrelevant) of at least
 *   fp8blk_workspace_bytes(M, N, K, 1) bytes.  When the shape's output
 *   tiles are too few to fill the GPU and such a workspace is given, K is
 *   split into S ranges of whole groups: each range's partial product
 *   (formed exactly as above) goes to the workspace and C is their sum in
 *   range order (S-1 extra FP32 additions per element; deterministic).
 *   NULL/0 (or a smaller workspace) computes C in one pass.  The workspace
 *   must not be used by other work on other streams during the call.
 */
fp8blk_status_t fp8blk_gemm_fp8_blockscaled(int64_t M, int64_t N, int64_t K,
                                            const uint8_t* A, int64_t lda, const float* sA,
                                            const uint8_t* B, int64_t ldb, int opB,
                                            const float* sB, int bscale_mode,
                                            void* C, int64_t ldc,
                                            void* workspace, size_t workspace_bytes,
                                            void* stream);

/*
 * The same GEMM for callers that cannot allocate (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): identical
 * arguments and results to fp8blk_gemm_fp8_blockscaled given a large enough
 * workspace, with the split-K partials in a device array that the library
 * holds on each GPU for the life of the process
 * (FP8BLK_NOALLOC_SCRATCH_BYTES).  It calls no allocating routine; its first
 * call on a device looks the array's address up once.  Shapes whose
 * partials exceed the array return FP8BLK_ERR_UNSUPPORTED before anything is
 * enqueued (with 256 compute units no valid shape does).  Every call on one
 * GPU uses the same array: calls that overlap on one GPU (other streams,
 * other threads) race and give wrong results.
 */
#define FP8BLK_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
fp8blk_status_t fp8blk_gemm_fp8_blockscaled_noalloc(int64_t M, int64_t N, int64_t K,
                                                    const uint8_t* A, int64_t lda, const float* sA,
                                                    const uint8_t* B, int64_t ldb, int opB,
                                                    const float* sB, int bscale_mode,
                                                    void* C, int64_t ldc, void* stream);

/*
 * The same GEMM with its output quantized on store for the next layer's
 * input (the pages quantize activations to FP8 before the next FP8 GEMM
 * and keep such caches in FP8 [p2¶4; p5¶4]): with C the FP32 result
 * defined above,
 *   (Q, sQ) = fp8blk_quantize_1x128 applied to C rounded to BF16 (nearest
 *             even), with flags qflags (0 or FP8BLK_SCALE_POW2),
 * computed in the GEMM's epilogue without writing C.
 *   Q   [M][N] E4M3 codes, pitch ldq >= N; sQ [ceil(N/128)][M] FP32.
 *   B is block-scaled (FP8BLK_BSCALE_BLOCK128 layouts); opB as above,
 *   FP8BLK_GEMM_POW2_SCALES allowed; K a positive multiple of 128; never
 *   split along K.
 */
fp8blk_status_t fp8blk_gemm_fp8_blockscaled_q1x128(int64_t M, int64_t N, int64_t K,
                                                   const uint8_t* A, int64_t lda, const float* sA,
                                                   const uint8_t* B, int64_t ldb, int opB,
                                                   const float* sB, uint8_t* Q, int64_t ldq,
                                                   float* sQ, uint32_t qflags, void* stream);
/*
 * Grouped (per-expert) block-scaled FP8 GEMM for MoE expert projections
 * [p2¶4]: for each expert e,
 *   C[off[e]:off[e+1]][:] = A[off[e]:off[e+1]][:] * B_e
 * with the same arithmetic as fp8blk_gemm_fp8_blockscaled.
 *   group_offsets  DEVICE int32 [G+1], non-decreasing, off[0] = 0,
 *                  off[G] = M_total (rows of A/C ordered by expert; groups
 *                  may be empty).  Read on the device: no host sync.
 *   A   [M_total][K] codes, pitch lda; sA [K/128][M_total].
 *   B   G matrices, expert e at B + e*strideB (elements), each [K][N]
 *       (OP_N, pitch ldb >= N) or [N][K] (OP_T, pitch ldb >= K).
 *   sB  G block-scale tables (BLOCK128 layout of one B_e), expert e at
 *       sB + e*stride_sB (floats).
 *   C   [M_total][N] FP32 (BF16 with FP8BLK_GEMM_OUT_BF16), pitch ldc.
 *   max_group_rows: an upper bound on any group's row count (e.g. M_total),
 *   or 0 if unknown; it only sizes the launch grid.
 *   K must be a positive multiple of 128; lda, ldb below 2^23.
 */
fp8blk_status_t fp8blk_grouped_gemm_fp8_blockscaled(int64_t G, const int32_t* group_offsets,
                                                    int64_t M_total, int64_t max_group_rows,
                                                    int64_t N, int64_t K,
                                                    const uint8_t* A, int64_t lda, const float* sA,
                                                    const uint8_t* B, int64_t ldb, int64_t strideB,
                                                    int opB, const float* sB, int64_t stride_sB,
                                                    void* C, int64_t ldc,
                                                    void* workspace, size_t workspace_bytes,
                                                    void* stream);

/*
 * MoE backward, Wgrad operands: 128x1 quantization along tokens inside each
 * expert's token range (the Wgrad operand tiling [p5¶4] applied per expert of
 * the grouped projections [p2¶4]).  Expert e owns tokens
 * [off[e], off[e+1]) of x; its tokens form ceil(M_e/128) groups of 128
 * starting at its first token (M_e = off[e+1] - off[e]; the last group is
 * partial when 128 does not divide M_e).  The groups of all experts are
 * stored one after another: expert e's first group is slot
 *   PG[e] = sum over e' < e of ceil(M_e'/128),
 * and its token j is column 128*PG[e] + j of qT.
 *   x   [T][C] BF16 (tokens in expert order), pitch ldx >= C.
 *   group_offsets  DEVICE int32 [G+1], non-decreasing, off[0] = 0,
 *                  off[G] = T.  Read on the device: no host sync.
 *   qT  [C][128*S] E4M3 codes, pitch ldqT >= 128*S, S =
 *       fp8blk_token_group_slots(T, G) (an upper bound on the number of
 *       groups).  Columns of a partial group past the expert's last token
 *       hold code 0; columns of slots past the last group are not written.
 *   s   [S][C] FP32, dense: s[g*C + c] scales channel c over the tokens of
 *       group slot g (rows of slots past the last group are not written).
 *   Each group is quantized exactly as fp8blk_quantize_128x1 quantizes a
 *   128-token tile of the expert's tokens.  flags: 0 or FP8BLK_SCALE_POW2.
 *   FP8BLK_ERR_UNSUPPORTED if S > 65535.
 */
fp8blk_status_t fp8blk_quantize_128x1_grouped(const uint16_t* x, int64_t T, int64_t C, int64_t ldx,
                                              int64_t G, const int32_t* group_offsets,
                                              uint8_t* qT, int64_t ldqT, float* s, uint32_t flags,
                                              void* stream);
/* Group slots to allocate for T tokens in G experts: T/128 + G (integer
 * division; 0 for negative arguments).  At least the number of ragged
 * 128-token groups of any split of the T tokens into G experts. */
int64_t fp8blk_token_group_slots(int64_t T, int64_t G);
/*
 * MoE backward, grouped Wgrad: for every expert e,
 *   C_e[m][n] = sum over e's token groups g of sA[g][m] * sB[g][n] * P_g[m][n],
 *   P_g[m][n] = sum over the tokens t of group g of dec(AT[m][t]) * dec(BT[n][t]),
 * i.e. dW_e = X_e^T dY_e with both operands as written by
 * fp8blk_quantize_128x1_grouped (same offsets, same T) [p5¶4; p2¶4].  Each
 * group's partial is formed by the matrix cores and promoted into an FP32
 * accumulator as in fp8blk_gemm_fp8_blockscaled (Wgrad role, ROW128 scales).
 *   group_offsets  the DEVICE offsets given to the quantizer.
 *   AT  [M][128*S] codes (pitch ldaT), sA [S][M]: X quantized, M = X's channels.
 *   BT  [N][128*S] codes (pitch ldbT), sB [S][N]: dY quantized, N = dY's channels.
 *   flags  0, or FP8BLK_GEMM_POW2_SCALES (every scale a power of two, e.g.
 *          both operands quantized with FP8BLK_SCALE_POW2) and/or
 *          FP8BLK_GEMM_OUT_BF16.
 *   C   G matrices [M][N] FP32 (BF16 with FP8BLK_GEMM_OUT_BF16), expert e
 *       at C + e*strideC elements, pitch ldc >= N, strideC >= M*ldc and
 *       16-byte aligned; all overwritten (an expert without tokens gets
 *       zeros).
 *   ldaT, ldbT below 2^23 (FP8BLK_ERR_UNSUPPORTED otherwise).  With T = 0
 *   the operands are not read (and may be NULL); C still gets zeros.
 */
fp8blk_status_t fp8blk_grouped_wgrad_fp8_blockscaled(int64_t G, const int32_t* group_offsets, int64_t T,
                                                     int64_t M, int64_t N,
                                                     const uint8_t* AT, int64_t ldaT, const float* sA,
                                                     const uint8_t* BT, int64_t ldbT, const float* sB,
                                                     uint32_t flags, void* C, int64_t ldc,
                                                     int64_t strideC, void* stream);
/*
 * Diagnostic: one 16x16 tile product over 128 E4M3 k, as the matrix cores
 * compute it, returned unprocessed.  The GEMMs promote each 128-deep group's
 * matrix-core partial into FP32 because the cores add products with limited
 * precision [p2¶3, p5¶4]; this call exposes that behaviour so that it can be
 * measured and pinned.
 *   A, B  DEVICE [16][128] E4M3 codes, row-major, 16-byte aligned.
 *   C     DEVICE [16][16] FP32, C[i][j] = the instruction's result for
 *         sum_k dec(A[i][k]) * dec(B[j][k]) (overwritten).
 *   instr 0: one v_mfma_scale_f32_16x16x128_f8f6f4 (the GEMMs' instruction)
 *            with unit scales from a zero accumulator;
 *         1: four v_mfma_f32_16x16x32_fp8_fp8 (32 k each) chained through
 *            the FP32 accumulator from zero.
 *   FP8BLK_ERR_INVALID_ARG for another instr, a null or misaligned pointer.
 */
fp8blk_status_t fp8blk_mfma_probe(int instr, const uint8_t* A, const uint8_t* B, float* C, void* stream);

/*
 * Diagnostic: a plain streaming kernel with the quantizers' HBM traffic
 * pattern (BF16 in, one byte per element out: 16 bytes read and 8 bytes
 * written per 16-byte chunk), so that a quantizer's time can be set against
 * what a kernel of the same traffic and no tile logic takes on the device.
 *   src     DEVICE, `chunks` 16-byte chunks, 16-byte aligned (read only).
 *   chunks  number of 16-byte chunks, >= 0 (0: nothing is read or written).
 *   dst     DEVICE, 8 * chunks bytes, 8-byte aligned; byte pairs of words
 *           (x ^ y, z ^ w) of each chunk (x, y, z, w its 4-byte words).
 *   FP8BLK_ERR_INVALID_ARG for chunks < 0, a null or misaligned pointer.
 */
fp8blk_status_t fp8blk_stream_probe(const void* src, int64_t chunks, void* dst, void* stream);

/* Workspace that lets fp8blk_gemm_fp8_blockscaled split K for this shape
 * (G = 1), for the current device; 0 when it would not split.  The grouped
 * GEMM (G > 1) needs none. */
size_t fp8blk_workspace_bytes(int64_t M, int64_t N, int64_t K, int64_t G);

/* Human-readable name of a status code (static string). */
const char* fp8blk_status_string(fp8blk_status_t status);

/* ABI version of this header: 6 (2 added the MoE backward entry points, 3 the
 * BF16 output flag and the quantize-on-store GEMM, 4 the matrix-core probe
 * and the allocation-free GEMM, 5 the streaming probe, 6 the two-operand
 * quantizer). */
int fp8blk_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* LIBFP8BLK_H */
