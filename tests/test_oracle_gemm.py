"""Pins for the oracle's block-scaled GEMM (CPU only).

* exact rational brute force (Fraction sums over an enumerated E4M3 value
  set) on tiny shapes with edge codes, for every B layout and scale mode;
* closed forms: an identity B returns the dequantized A; one group with unit
  scales returns the exact dot products; scaling sA by 2^j scales C by 2^j;
* the transposed B storage and the ROW128 scale mode reduce to the plain one;
* the grouped variant equals per-expert GEMMs, with empty experts.
"""
from fractions import Fraction

import numpy as np
import pytest

import oracle
from tests import exact_ref


def _codes(rng, shape, edge=True):
    c = rng.integers(0, 0x7F, size=shape).astype(np.uint8)
    c |= (rng.integers(0, 2, size=shape) << 7).astype(np.uint8)
    if edge:
        flat = c.reshape(-1)
        picks = rng.integers(0, flat.size, size=max(1, flat.size // 8))
        flat[picks] = rng.choice(np.array([0x7E, 0xFE, 0x01, 0x81, 0x00, 0x80, 0x07], np.uint8), size=picks.size)
    return c


def _scales(rng, shape):
    # float32 scales with full 24-bit significands over a wide exponent range
    v = rng.uniform(1.0, 2.0, size=shape) * np.exp2(rng.integers(-30, 10, size=shape))
    return v.astype(np.float32)


def _exact_C(A, sA, B, sB, opB, mode):
    M, K = A.shape
    N = B.shape[1] if opB == oracle.OP_N else B.shape[0]
    out = [[Fraction(0)] * N for _ in range(M)]
    for m in range(M):
        for n in range(N):
            tot = Fraction(0)
            for g in range(K // 128):
                P = Fraction(0)
                for k in range(g * 128, (g + 1) * 128):
                    b = B[k, n] if opB == oracle.OP_N else B[n, k]
                    P += exact_ref.e4m3_value(int(A[m, k])) * exact_ref.e4m3_value(int(b))
                if mode == oracle.BSCALE_ROW128:
                    sb = sB[g, n]
                elif opB == oracle.OP_N:
                    sb = sB[g, n // 128]
                else:
                    sb = sB[n // 128, g]
                tot += Fraction(float(sA[g, m])) * Fraction(float(sb)) * P
            out[m][n] = tot
    return out


CASES = [(oracle.OP_N, oracle.BSCALE_BLOCK128), (oracle.OP_T, oracle.BSCALE_BLOCK128),
         (oracle.OP_N, oracle.BSCALE_ROW128), (oracle.OP_T, oracle.BSCALE_ROW128)]


@pytest.mark.parametrize("K", [128, 256, 384])
@pytest.mark.parametrize("opB,mode", CASES)
def test_gemm_bruteforce(K, opB, mode):
    rng = np.random.default_rng(K + 10 * opB + 100 * mode)
    M, N = 3, 2
    G = K // 128
    A = _codes(rng, (M, K))
    B = _codes(rng, (K, N) if opB == oracle.OP_N else (N, K))
    sA = _scales(rng, (G, M))
    if mode == oracle.BSCALE_ROW128:
        sB = _scales(rng, (G, N))
    else:
        sB = _scales(rng, (G, 1) if opB == oracle.OP_N else (1, G))
    C = oracle.gemm_blockscaled(A, sA, B, sB, opB, mode)
    ex = _exact_C(A, sA, B, sB, opB, mode)
    for m in range(M):
        for n in range(N):
            # each group: one FP64 rounding of P*S and one of the running sum
            bound = Fraction(2 * G) * Fraction(1, 2 ** 52) * sum(
                abs(Fraction(float(sA[g, m]))) * Fraction(2 ** 18 * 128) for g in range(G)) * max(
                abs(Fraction(float(x))) for x in sB.reshape(-1))
            assert abs(Fraction(C[m, n]) - ex[m][n]) <= bound
            # the sampled-entry form gives identical bits
            e = oracle.gemm_blockscaled_entries(A, sA, B, sB, [m], [n], opB, mode)[0]
            assert e == C[m, n]


def test_single_group_unit_scales_exact():
    rng = np.random.default_rng(5)
    A = _codes(rng, (4, 128))
    B = _codes(rng, (128, 3))
    C = oracle.gemm_blockscaled(A, np.ones((1, 4), np.float32), B, np.ones((1, 1), np.float32))
    ex = _exact_C(A, np.ones((1, 4), np.float32), B, np.ones((1, 1), np.float32), oracle.OP_N,
                  oracle.BSCALE_BLOCK128)
    for m in range(4):
        for n in range(3):
            assert Fraction(C[m, n]) == ex[m][n]


def test_identity_b_returns_dequantized_a():
    rng = np.random.default_rng(6)
    M, K = 8, 256
    A = _codes(rng, (M, K), edge=True)
    sA = _scales(rng, (K // 128, M))
    B = np.zeros((K, K), np.uint8)
    B[np.arange(K), np.arange(K)] = 0x38  # E4M3 1.0
    sB = np.ones((K // 128, K // 128), np.float32)
    C = oracle.gemm_blockscaled(A, sA, B, sB)
    assert np.array_equal(C, oracle.dequantize_1x128(A, sA))


def test_power_of_two_linearity():
    rng = np.random.default_rng(7)
    A = _codes(rng, (5, 256))
    B = _codes(rng, (256, 130))
    sA = _scales(rng, (2, 5))
    sB = _scales(rng, (2, 2))
    C = oracle.gemm_blockscaled(A, sA, B, sB)
    C2 = oracle.gemm_blockscaled(A, (sA * np.float32(2.0 ** 9)).astype(np.float32), B, sB)
    assert np.array_equal(C2, C * 2.0 ** 9)


def test_transposed_storage_and_row128_reduce_to_plain():
    rng = np.random.default_rng(8)
    M, K, N = 6, 384, 260
    A = _codes(rng, (M, K))
    B = _codes(rng, (K, N))
    sA = _scales(rng, (3, M))
    sB = _scales(rng, (3, 3))
    C = oracle.gemm_blockscaled(A, sA, B, sB, oracle.OP_N, oracle.BSCALE_BLOCK128)
    CT = oracle.gemm_blockscaled(A, sA, np.ascontiguousarray(B.T), np.ascontiguousarray(sB.T), oracle.OP_T,
                                 oracle.BSCALE_BLOCK128)
    assert np.array_equal(C, CT)
    row = np.repeat(sB, 128, axis=1)[:, :N]
    CR = oracle.gemm_blockscaled(A, sA, B, row, oracle.OP_N, oracle.BSCALE_ROW128)
    assert np.array_equal(C, CR)


def test_grouped_equals_per_expert_with_empty_groups():
    rng = np.random.default_rng(9)
    K, N = 256, 140
    counts = [3, 0, 5, 0, 0, 2]
    off = np.concatenate([[0], np.cumsum(counts)])
    Mt = int(off[-1])
    A = _codes(rng, (Mt, K))
    sA = _scales(rng, (2, Mt))
    B = _codes(rng, (len(counts), K, N))
    sB = _scales(rng, (len(counts), 2, 2))
    C = oracle.grouped_gemm_blockscaled(off, A, sA, B, sB)
    for e in range(len(counts)):
        r0, r1 = off[e], off[e + 1]
        if r1 > r0:
            ref = oracle.gemm_blockscaled(A[r0:r1], sA[:, r0:r1], B[e], sB[e])
            assert np.array_equal(C[r0:r1], ref)
    # a few entries against the exact sum
    for r, n in [(0, 0), (4, 139), (9, 77)]:
        e = int(np.searchsorted(off, r, side="right") - 1)
        ex = _exact_C(A[r:r + 1], sA[:, r:r + 1], B[e][:, n:n + 1], sB[e][:, n // 128:n // 128 + 1],
                      oracle.OP_N, oracle.BSCALE_BLOCK128)[0][0]
        assert abs(Fraction(C[r, n]) - ex) <= abs(ex) * Fraction(1, 2 ** 48) + Fraction(1, 2 ** 200)


def test_unquantized_reference():
    rng = np.random.default_rng(10)
    a = rng.standard_normal((3, 256)).astype(np.float32)
    b = rng.standard_normal((256, 2)).astype(np.float32)
    ab = (a.view(np.uint32) >> 16).astype(np.uint16)
    bb = (b.view(np.uint32) >> 16).astype(np.uint16)
    R = oracle.gemm_unquantized(ab, bb)
    for m in range(3):
        for n in range(2):
            ex = sum(exact_ref.bf16_to_fraction(int(ab[m, k])) * exact_ref.bf16_to_fraction(int(bb[k, n]))
                     for k in range(256))
            assert abs(Fraction(R[m, n]) - ex) <= Fraction(256, 2 ** 52) * sum(
                abs(exact_ref.bf16_to_fraction(int(ab[m, k])) * exact_ref.bf16_to_fraction(int(bb[k, n])))
                for k in range(256))
