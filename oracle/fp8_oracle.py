"""CPU oracle for fine-grained FP8 (E4M3) quantization and the block-scaled FP8 GEMM.

TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the CPU
baseline leg of the benchmark may import this module.  The product path (the
HIP library and its Python binding) never calls it, and it shares no code,
table or constant generator with that path.

It is deliberately plain and slow: NumPy over whole arrays, no blocking and no
fusion beyond what the definitions below state, so that every function can be
checked against the source pages by eye.

Citations ``[pN¶k]`` name the N-th web page of the source collection and its
k-th paragraph counted from the page heading:
  p1 = xn--9g3bo1gtkw0l8ubf92bgle.kr (board qna, wr_id 85187)
  p2 = inprokorea.com (board free, wr_id 735329)
  p5 = inprokorea.com (board free, wr_id 890463)

What the pages fix, and the readings taken where they are silent:
  * Activations are scaled per 1x128 tile (one token, 128 channels) and
    weights per 128x128 block [p1¶3, the description of Figure 7(a)].
  * The maximum absolute value is taken online, per tile or block, at
    quantization time [p2¶4].
  * All tensors use E4M3 [p2¶2].  Reading: OCP E4M3 ("e4m3fn": bias 7, no
    infinities, 0x7F/0xFF are NaN, largest finite 448).
  * Scales are FP32 and stored alongside the codes [p1¶3]; they multiply the
    codes at dequantization [p2¶4], so x ~= dec(q) * s.
  * Reading: s = fl32(amax / 448) with IEEE division; an all-zero tile gets
    s = 1.  With the power-of-two option (used by the pages for some
    activations [p2¶4]) s is the smallest power of two >= amax / 448,
    compared exactly.
  * Reading: the quotient is y = fl32(x / s) (IEEE division by the stored
    scale), encoded round-to-nearest-even at the 3-bit mantissa, saturating
    |y| > 448 to +-448, keeping the sign of values that round to zero.
  * Wgrad operands use 128x1 tiles along the token dimension and are stored
    transposed [p5¶4].
  * The GEMM sums each 128-deep K group (one scale group) and promotes the
    partial into a full-precision accumulator, multiplying in the group's
    scales [p2¶3, p2¶4].  Here the partial is exact (FP64, see
    ``gemm_blockscaled``) and the accumulator is FP64.
  * Context only, with no HIP counterpart: the limited-accumulation
    emulation at the end of this file.  Its rule is pinned against brute
    force; whether the rule matches the H800 is parity unpinned.
"""
from __future__ import annotations

import numpy as np

E4M3_MAX = 448.0
TILE = 128

# --------------------------------------------------------------------------
# BF16 input handling
# --------------------------------------------------------------------------


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """Widen BF16 bit patterns (uint16) to float32 exactly: BF16 is the upper
    half of an IEEE binary32 word."""
    bits = np.asarray(bits, dtype=np.uint16)
    return (bits.astype(np.uint32) << np.uint32(16)).view(np.float32)


# --------------------------------------------------------------------------
# E4M3 format (OCP "e4m3fn"): 1 sign, 4 exponent (bias 7), 3 mantissa bits
# --------------------------------------------------------------------------


def e4m3_decode(codes: np.ndarray) -> np.ndarray:
    """Value of each E4M3 code as float64, written from the bit-field
    definition: exponent field 0 is subnormal (m/8 * 2^-6), otherwise
    (1 + m/8) * 2^(e-7); codes 0x7F and 0xFF are NaN."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where((c >> 7) & 1, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = (c & 0x7).astype(np.float64)
    mag = np.where(e == 0, m / 8.0 * 2.0 ** -6, (1.0 + m / 8.0) * np.exp2(e - 7.0))
    out = sign * mag
    return np.where((c & 0x7F) == 0x7F, np.nan, out)


def e4m3_encode(y: np.ndarray) -> np.ndarray:
    """Encode float32 values to E4M3 codes: round to nearest, ties to even at
    the 3-bit mantissa (quantum 2^-9 below 2^-6), saturate |y| > 448 to the
    largest finite code 0x7E, keep the sign bit when the result is zero.
    NaN input is outside the contract and maps to 0x7F."""
    y = np.asarray(y, dtype=np.float32)
    neg = np.signbit(y)
    a = np.abs(y).astype(np.float64)  # exact widening
    nan = np.isnan(a)
    a = np.where(nan, 0.0, a)
    sat = a > E4M3_MAX
    a = np.where(sat, E4M3_MAX, a)

    code = np.zeros(a.shape, dtype=np.int64)
    sub = a < 2.0 ** -6
    # Subnormal range: integer multiples of 2^-9.  A count of 8 is 2^-6,
    # whose code (exponent field 1, mantissa 0) is also 8.
    n_sub = np.rint(a * 2.0 ** 9)  # np.rint rounds half to even
    # Normal range: a = f * 2^E with f in [0.5, 1)  =>  binade exponent E-1,
    # quantum 2^(E-1-3).
    f, E = np.frexp(np.where(sub, 1.0, a))
    ex = E.astype(np.int64) - 1
    n = np.rint(a * np.exp2(3.0 - ex))  # in [8, 16]; exact scaling by 2^k
    carry = n >= 16
    ex = np.where(carry, ex + 1, ex)
    n = np.where(carry, n / 2.0, n)
    normal_code = ((ex + 7) << 3) | (n.astype(np.int64) - 8)
    code = np.where(sub, n_sub.astype(np.int64), normal_code)
    code = np.where(neg, code | 0x80, code)
    code = np.where(nan, 0x7F, code)
    return code.astype(np.uint8)


# --------------------------------------------------------------------------
# Tile scale
# --------------------------------------------------------------------------


def tile_scale(amax: np.ndarray, pow2: bool) -> np.ndarray:
    """Per-tile FP32 scale from the tile's maximum absolute value.

    Default: s = fl32(amax / 448) (IEEE float32 division).
    pow2:    s = 2^e with e the smallest integer such that 448 * 2^e >= amax,
             decided by exact comparison in float64 (448 * 2^e is exact).
    amax == 0 gives s = 1 in both modes."""
    amax = np.asarray(amax, dtype=np.float32)
    if not pow2:
        s = amax / np.float32(E4M3_MAX)  # float32 / float32: IEEE RN
    else:
        a = amax.astype(np.float64)
        safe = np.where(a > 0, a, 1.0)
        e = np.ceil(np.log2(safe / E4M3_MAX)).astype(np.int64)
        # correct any off-by-one of log2 by exact comparisons
        e = np.where(E4M3_MAX * np.exp2(e - 1.0) >= safe, e - 1, e)
        e = np.where(E4M3_MAX * np.exp2(e * 1.0) < safe, e + 1, e)
        s = np.exp2(e * 1.0).astype(np.float32)
    return np.where(amax == 0, np.float32(1.0), s).astype(np.float32)


def _encode_tiles(x: np.ndarray, s: np.ndarray) -> np.ndarray:
    """q = enc(fl32(x / s)) elementwise; x and s broadcast, both float32."""
    y = (x.astype(np.float32) / s.astype(np.float32)).astype(np.float32)
    return e4m3_encode(y)


# --------------------------------------------------------------------------
# Quantizers
# --------------------------------------------------------------------------


def quantize_1x128(x_bits: np.ndarray, pow2: bool = False):
    """1x128 tiles (per token per 128 channels) [p1¶3].

    x_bits: uint16 BF16 bits, shape [M][K].
    Returns (q uint8 [M][K], s float32 [ceil(K/128)][M]).  The scale layout is
    K-group-major: s[g][m] scales row m, columns [128g, 128g+128).  A partial
    last group takes its amax over the columns present."""
    x = bf16_bits_to_f32(x_bits)
    M, K = x.shape
    G = -(-K // TILE)
    q = np.empty((M, K), dtype=np.uint8)
    s = np.empty((G, M), dtype=np.float32)
    for g in range(G):
        cols = slice(g * TILE, min(K, (g + 1) * TILE))
        tile = x[:, cols]
        amax = np.max(np.abs(tile), axis=1) if tile.shape[1] else np.zeros(M, np.float32)
        sg = tile_scale(amax, pow2)
        s[g] = sg
        q[:, cols] = _encode_tiles(tile, sg[:, None])
    return q, s


def quantize_128x1(x_bits: np.ndarray, pow2: bool = False):
    """128x1 tiles along the token dimension, codes stored transposed, as
    the pages describe for the Wgrad operands [p5¶4].

    x_bits: uint16 BF16 bits, shape [T][C] (tokens x channels).
    Returns (qT uint8 [C][T], s float32 [ceil(T/128)][C]); s[g][c] scales
    channel c over tokens [128g, 128g+128).  Computed directly over column
    tiles, not by reusing quantize_1x128."""
    x = bf16_bits_to_f32(x_bits)
    T, C = x.shape
    G = -(-T // TILE)
    qT = np.empty((C, T), dtype=np.uint8)
    s = np.empty((G, C), dtype=np.float32)
    for g in range(G):
        rows = slice(g * TILE, min(T, (g + 1) * TILE))
        tile = x[rows, :]  # [<=128][C]
        amax = np.max(np.abs(tile), axis=0) if tile.shape[0] else np.zeros(C, np.float32)
        sg = tile_scale(amax, pow2)
        s[g] = sg
        qT[:, rows] = _encode_tiles(tile, sg[None, :]).T
    return qT, s


def quantize_block128(w_bits: np.ndarray, pow2: bool = False):
    """128x128 blocks (per 128 input channels per 128 output channels)
    [p1¶3].

    w_bits: uint16 BF16 bits, shape [R][C].
    Returns (q uint8 [R][C], s float32 [ceil(R/128)][ceil(C/128)]); partial
    edge blocks take their amax over the elements present."""
    w = bf16_bits_to_f32(w_bits)
    R, C = w.shape
    GR, GC = -(-R // TILE), -(-C // TILE)
    q = np.empty((R, C), dtype=np.uint8)
    s = np.empty((GR, GC), dtype=np.float32)
    for i in range(GR):
        for j in range(GC):
            rs = slice(i * TILE, min(R, (i + 1) * TILE))
            cs = slice(j * TILE, min(C, (j + 1) * TILE))
            blk = w[rs, cs]
            amax = np.float32(np.max(np.abs(blk))) if blk.size else np.float32(0)
            sij = tile_scale(np.array([amax], np.float32), pow2)[0]
            s[i, j] = sij
            q[rs, cs] = _encode_tiles(blk, np.float32(sij))
    return q, s


def dequantize_1x128(q: np.ndarray, s: np.ndarray) -> np.ndarray:
    """dec(q) * s in float64 (exact) for 1x128-scaled codes [M][K], s [G][M]."""
    d = e4m3_decode(q)
    M, K = q.shape
    out = np.empty((M, K), np.float64)
    for g in range(s.shape[0]):
        cols = slice(g * TILE, min(K, (g + 1) * TILE))
        out[:, cols] = d[:, cols] * s[g].astype(np.float64)[:, None]
    return out


def dequantize_block128(q: np.ndarray, s: np.ndarray) -> np.ndarray:
    """dec(q) * s in float64 (exact) for 128x128-scaled codes."""
    d = e4m3_decode(q)
    rep = np.repeat(np.repeat(s.astype(np.float64), TILE, axis=0), TILE, axis=1)
    return d * rep[: q.shape[0], : q.shape[1]]


def requantize_128x1_from_1x128(q: np.ndarray, s: np.ndarray, pow2: bool = False):
    """The pages' Wgrad operand path [p5¶4]: a cached 1x128-quantized
    activation (codes q [T][C], scales s [ceil(C/128)][T]) is read out,
    dequantized, transposed and re-quantized into 128x1 tiles.

    Reading: the dequantized value is fl32(dec(q) * s), one IEEE float32
    multiplication rounded to nearest even (the product of a 4-bit and a
    24-bit significand can need 28 bits), which is then quantized exactly as
    ``quantize_128x1`` quantizes a float32 tensor."""
    T, C = q.shape
    x = np.empty((T, C), np.float32)
    d = e4m3_decode(q)
    for g in range(s.shape[0]):
        cols = slice(g * TILE, min(C, (g + 1) * TILE))
        x[:, cols] = (d[:, cols].astype(np.float32) * s[g][:, None].astype(np.float32))
    G = -(-T // TILE)
    qT = np.empty((C, T), np.uint8)
    sT = np.empty((G, C), np.float32)
    for g in range(G):
        rows = slice(g * TILE, min(T, (g + 1) * TILE))
        tile = x[rows, :]
        amax = np.max(np.abs(tile), axis=0)
        sg = tile_scale(amax, pow2)
        sT[g] = sg
        qT[:, rows] = _encode_tiles(tile, sg[None, :]).T
    return qT, sT


# --------------------------------------------------------------------------
# Block-scaled GEMM
# --------------------------------------------------------------------------

OP_N = 0  # B stored [K][N]
OP_T = 1  # B stored [N][K]
BSCALE_BLOCK128 = 0
BSCALE_ROW128 = 1


def _b_scale_for_group(sB: np.ndarray, g: int, N: int, opB: int, mode: int) -> np.ndarray:
    """Per-column B scale (float64, length N) for K group g.

    BLOCK128: one scale per 128x128 block of the stored B; stored [K/128][N/128]
              for opB=N and [N/128][K/128] for opB=T (the block grid of the
              matrix as stored).
    ROW128:   one scale per output column per K group, stored [K/128][N]
              (B quantized with 128x1 tiles along K)."""
    n_blk = np.arange(N) // TILE
    if mode == BSCALE_ROW128:
        return sB[g, :].astype(np.float64)
    if opB == OP_N:
        return sB[g, n_blk].astype(np.float64)
    return sB[n_blk, g].astype(np.float64)


def gemm_blockscaled(A: np.ndarray, sA: np.ndarray, B: np.ndarray, sB: np.ndarray,
                     opB: int = OP_N, bscale_mode: int = BSCALE_BLOCK128) -> np.ndarray:
    """C[m,n] = sum_g sA[g][m] * sB(g,n) * P_g[m,n],
    P_g[m,n] = sum_{k in group g} dec(A[m,k]) * dec(B[k,n])   [p2¶3, p2¶4].

    A: uint8 codes [M][K], sA float32 [K/128][M].
    B: uint8 codes, [K][N] (opB=N) or [N][K] (opB=T); sB as in
       ``_b_scale_for_group``.
    K must be a multiple of 128.  Returns C as float64 [M][N].

    Exactness: every E4M3 value is an integer multiple of 2^-9 below 2^9, so a
    product of two is a multiple of 2^-18 below 2^18 and a 128-term sum is a
    multiple of 2^-18 below 2^25: fewer than 43 significant bits.  The FP64
    matmul of one group's decoded slices is therefore exact in any summation
    order, which is why a library matmul may serve as the group step.  The
    scale product sA*sB (two float32) is exact in FP64; the product with P_g
    and the running sum over g, in ascending g, round once each in FP64."""
    M, K = A.shape
    assert K % TILE == 0
    Ad = e4m3_decode(A)
    Bd = e4m3_decode(B)
    if opB == OP_T:
        Bd = Bd.T
    assert Bd.shape[0] == K
    N = Bd.shape[1]
    C = np.zeros((M, N), np.float64)
    for g in range(K // TILE):
        ks = slice(g * TILE, (g + 1) * TILE)
        P = Ad[:, ks] @ Bd[ks, :]
        S = sA[g].astype(np.float64)[:, None] * _b_scale_for_group(sB, g, N, opB, bscale_mode)[None, :]
        C += P * S
    return C


def gemm_blockscaled_entries(A, sA, B, sB, rows, cols, opB=OP_N, bscale_mode=BSCALE_BLOCK128):
    """The same sum as ``gemm_blockscaled`` for selected output entries
    (rows[i], cols[i]) only; used to check full-size outputs by sampling."""
    rows = np.asarray(rows)
    cols = np.asarray(cols)
    K = A.shape[1]
    Ar = e4m3_decode(A[rows, :])  # [S][K]
    if opB == OP_N:
        Bc = e4m3_decode(B[:, cols]).T  # [S][K]
        N = B.shape[1]
    else:
        Bc = e4m3_decode(B[cols, :])
        N = B.shape[0]
    out = np.zeros(rows.shape[0], np.float64)
    for g in range(K // TILE):
        ks = slice(g * TILE, (g + 1) * TILE)
        P = np.sum(Ar[:, ks] * Bc[:, ks], axis=1)  # exact, see gemm_blockscaled
        sb = _b_scale_for_group(sB, g, N, opB, bscale_mode)[cols]
        out += P * (sA[g, rows].astype(np.float64) * sb)
    return out


def grouped_gemm_blockscaled(offsets: np.ndarray, A: np.ndarray, sA: np.ndarray,
                             B: np.ndarray, sB: np.ndarray, opB: int = OP_N) -> np.ndarray:
    """Per-expert GEMM: rows [offsets[e], offsets[e+1]) of A times expert e's
    block-scaled weight B[e].  The pages quantize the activation before the
    MoE up-projection and run that projection in FP8 [p2¶4], with all experts
    of a layer on one device [p2¶1].

    A: uint8 [M_total][K], sA float32 [K/128][M_total] (rows in expert order).
    B: uint8 [G][K][N] (opB=N) or [G][N][K] (opB=T); sB: per-expert block
    scales [G][...] in the layout of ``_b_scale_for_group``.
    Returns float64 [M_total][N]."""
    offsets = np.asarray(offsets, np.int64)
    Gn = offsets.shape[0] - 1
    N = B.shape[2] if opB == OP_N else B.shape[1]
    C = np.zeros((A.shape[0], N), np.float64)
    for e in range(Gn):
        r0, r1 = int(offsets[e]), int(offsets[e + 1])
        if r1 == r0:
            continue
        C[r0:r1] = gemm_blockscaled(A[r0:r1], sA[:, r0:r1], B[e], sB[e], opB, BSCALE_BLOCK128)
    return C


def token_group_starts(offsets) -> np.ndarray:
    """Layout of the ragged 128-token groups of MoE experts (reading: the
    pages tile Wgrad operands 128x1 along tokens [p5¶4] and run the expert
    projections per expert [p2¶4]; tiling inside each expert's token range is
    the plainest reading, and a group then never mixes two experts' tokens).
    Expert e owns tokens [offsets[e], offsets[e+1]); they form
    ceil(M_e/128) groups starting at its first token.  Returns PG int64
    [G+1]: expert e's groups are slots PG[e] .. PG[e+1]-1, PG[G] the total."""
    offsets = np.asarray(offsets, np.int64)
    counts = -(-(offsets[1:] - offsets[:-1]) // TILE)
    return np.concatenate([[0], np.cumsum(counts)]).astype(np.int64)


def quantize_128x1_grouped(x_bits: np.ndarray, offsets, pow2: bool = False):
    """128x1 quantization inside each expert's token range, in the slot
    layout of ``token_group_starts``: expert e's token j is column
    128*PG[e] + j.  x_bits: uint16 BF16 [T][C] (tokens in expert order).
    Returns (qT uint8 [C][128*PG[G]], s float32 [PG[G]][C]); columns of a
    partial last group past the expert's tokens hold code 0 (the code of
    +0), so that they add nothing to a product."""
    offsets = np.asarray(offsets, np.int64)
    PG = token_group_starts(offsets)
    C = x_bits.shape[1]
    qT = np.zeros((C, TILE * int(PG[-1])), np.uint8)
    s = np.empty((int(PG[-1]), C), np.float32)
    for e in range(offsets.shape[0] - 1):
        t0, t1 = int(offsets[e]), int(offsets[e + 1])
        if t1 == t0:
            continue
        qe, se = quantize_128x1(x_bits[t0:t1], pow2)
        c0 = TILE * int(PG[e])
        qT[:, c0:c0 + (t1 - t0)] = qe
        s[PG[e]:PG[e + 1]] = se
    return qT, s


def grouped_wgrad_blockscaled(offsets, AT: np.ndarray, sA: np.ndarray, BT: np.ndarray, sB: np.ndarray) -> np.ndarray:
    """MoE grouped Wgrad: for each expert e, the Wgrad-role block-scaled GEMM
    [p1¶3, p5¶4] over that expert's group slots only:
      C_e[m,n] = sum over slots g of e of sA[g][m] * sB[g][n] * P_g[m,n],
      P_g[m,n] = sum over the 128 columns t of slot g of dec(AT[m,t]) * dec(BT[n,t]).
    AT [M][>=128*PG[G]], BT [N][>=128*PG[G]] codes and sA [>=PG[G]][M],
    sB [>=PG[G]][N] as written by ``quantize_128x1_grouped``.  Returns
    float64 [G][M][N]; an expert without tokens gets zeros."""
    offsets = np.asarray(offsets, np.int64)
    PG = token_group_starts(offsets)
    Gn = offsets.shape[0] - 1
    M, N = AT.shape[0], BT.shape[0]
    out = np.zeros((Gn, M, N), np.float64)
    for e in range(Gn):
        g0, g1 = int(PG[e]), int(PG[e + 1])
        if g1 == g0:
            continue
        cols = slice(TILE * g0, TILE * g1)
        out[e] = gemm_blockscaled(AT[:, cols], sA[g0:g1], BT[:, cols], sB[g0:g1], OP_T, BSCALE_ROW128)
    return out


def grouped_wgrad_entries(offsets, AT, sA, BT, sB, experts, rows, cols) -> np.ndarray:
    """The same sum as ``grouped_wgrad_blockscaled`` for selected entries
    (experts[i], rows[i], cols[i]); used to check full-size outputs by
    sampling."""
    PG = token_group_starts(offsets)
    out = np.zeros(len(experts), np.float64)
    for i, (e, m, n) in enumerate(zip(experts, rows, cols)):
        for g in range(int(PG[e]), int(PG[e + 1])):
            ts = slice(TILE * g, TILE * (g + 1))
            P = np.sum(e4m3_decode(AT[m, ts]) * e4m3_decode(BT[n, ts]))  # exact, see gemm_blockscaled
            out[i] += P * (np.float64(sA[g, m]) * np.float64(sB[g, n]))
    return out


def gemm_unquantized(A_bits: np.ndarray, B_bits: np.ndarray, opB: int = OP_N) -> np.ndarray:
    """FP64 product of the BF16 inputs with no quantization; the reference
    for the accumulation/quantization error study."""
    A = bf16_bits_to_f32(A_bits).astype(np.float64)
    B = bf16_bits_to_f32(B_bits).astype(np.float64)
    if opB == OP_T:
        B = B.T
    return A @ B


# --------------------------------------------------------------------------
# Context only: limited-precision accumulation of FP8 products
# --------------------------------------------------------------------------
#
# The pages report that the H800 tensor core adds FP8 products in fixed
# point, aligning them to the largest exponent by right shifts before the
# addition [p5¶4], that the sum keeps only about 14 bits [p2¶3], and that
# over K = 4096 this gives a maximum relative error of nearly 2 % [p2¶2].
# They say neither how many products are aligned together nor whether the
# shifted-out bits are truncated or rounded.  Readings taken here: each step
# adds `width` products and the running accumulator; every one of those
# terms is truncated toward zero (a right shift of a sign-magnitude
# mantissa) to a multiple of 2^(E - bits), where 2^(E-1) <= the largest
# |term| < 2^E; the exact sum of the truncated terms becomes the new FP32
# accumulator.  This models no kernel of this library (the gfx950 MFMA is not
# emulated here); it is context for the accumulation study, and whether it
# matches the H800 is unpinned.


def limited_dot(a: np.ndarray, b: np.ndarray, width: int = 32, bits: int = 14) -> np.ndarray:
    """sum_k a[..., k] * b[..., k] accumulated as described above, in steps
    of `width` products along the last axis (a and b broadcast; their values
    are exact FP8 values, so every product is exact in FP64).  Returns
    float64 holding FP32 values."""
    assert bits + int(np.ceil(np.log2(width + 1))) <= 53, "truncated terms must sum exactly in FP64"
    K = a.shape[-1]
    acc = np.zeros(np.broadcast_shapes(a.shape[:-1], b.shape[:-1]), np.float64)
    for k0 in range(0, K, width):
        prods = a[..., k0:k0 + width] * b[..., k0:k0 + width]
        terms = np.concatenate([acc[..., None], prods], axis=-1)
        _, ex = np.frexp(terms)  # |t| in [2^(ex-1), 2^ex) for t != 0
        ex = np.where(terms != 0, ex, -(1 << 20))
        emax = ex.max(axis=-1)
        zero = emax == -(1 << 20)
        lsb = np.ldexp(1.0, np.where(zero, 0, emax - bits))[..., None]
        kept = np.trunc(terms / lsb) * lsb  # toward zero; exact (lsb is a power of two)
        acc = kept.sum(axis=-1).astype(np.float32).astype(np.float64)
    return acc


def quantize_per_tensor(x_bits: np.ndarray):
    """One scale for the whole tensor, s = fl32(amax / 448), codes
    enc(fl32(x / s)): the tensor-wise scaling the pages contrast with their
    tiles [p2¶2].  Returns (q uint8, s float32 scalar)."""
    x = bf16_bits_to_f32(x_bits)
    amax = np.array([np.max(np.abs(x)) if x.size else 0.0], np.float32)
    s = tile_scale(amax, False)
    return _encode_tiles(x, s[0]), s[0]


def gemm_limited_per_tensor(A: np.ndarray, sA, B: np.ndarray, sB, width: int = 32, bits: int = 14) -> np.ndarray:
    """C = sA * sB * (limited sum over all of K of dec(A[m,k]) * dec(B[k,n])):
    tensor-wise scales and the whole K accumulated in the tensor core, the
    setting of the pages' 2 % figure [p2¶2].  A [M][K], B [K][N] codes."""
    Ad = e4m3_decode(A)
    Bd = e4m3_decode(B)
    P = limited_dot(Ad[:, None, :], Bd.T[None, :, :], width, bits)
    return P * (np.float64(sA) * np.float64(sB))


def gemm_blockscaled_limited(A: np.ndarray, sA: np.ndarray, B: np.ndarray, sB: np.ndarray,
                             width: int = 32, bits: int = 14) -> np.ndarray:
    """The pages' method on the H800 as they describe it: each 128-deep group
    summed in the tensor core with limited accumulation (starting from zero),
    then promoted to FP32 on the vector cores, multiplied by the group's
    scales and added to an FP32 accumulator [p2¶3, p2¶4].  A [M][K] 1x128,
    B [K][N] with 128x128 block scales (opB = N).  Returns float64 holding
    FP32 values."""
    M, K = A.shape
    assert K % TILE == 0
    Ad = e4m3_decode(A)
    Bd = e4m3_decode(B)
    N = Bd.shape[1]
    C = np.zeros((M, N), np.float32)
    for g in range(K // TILE):
        ks = slice(g * TILE, (g + 1) * TILE)
        P = limited_dot(Ad[:, None, ks], Bd[ks, :].T[None, :, :], width, bits).astype(np.float32)
        S = (sA[g].astype(np.float32)[:, None] * _b_scale_for_group(sB, g, N, OP_N, BSCALE_BLOCK128)
             .astype(np.float32)[None, :])
        C = (C + P * S).astype(np.float32)
    return C.astype(np.float64)
