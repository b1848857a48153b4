"""Pins for the oracle's limited-accumulation emulation (CPU only; context
for the accumulation study, no HIP counterpart).

The rule it implements is the reading of the pages' description of the
H800's FP8 accumulation: terms aligned to the largest exponent by right
shifts, about 14 bits kept.  Whether that matches the H800 is unpinned; what
is pinned here is that the code computes the rule:

* exact brute force of the rule with Python fractions on tiny random FP8
  dot products (several widths and bit counts, signs, zeros, the accumulator
  taking part in the alignment);
* closed forms: with enough bits and one step it is fl32 of the exact sum;
  small integers lose nothing at 14 bits;
* invariants: odd in either operand, error shrinking as bits grow;
* the pages' point: promoting each 128-deep group to FP32 (their method)
  leaves far less error than accumulating the whole K in the limited format.
"""
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
import synthetic
from synthetic import bf16_bits
from tests import exact_ref


def _fp8_values(rng, shape, zero_frac=0.1):
    codes = rng.integers(0, 256, size=shape).astype(np.uint8)
    codes[(codes & 0x7F) == 0x7F] = 0x3C  # no NaN codes
    codes[rng.random(shape) < zero_frac] = 0
    return oracle.e4m3_decode(codes)


def _brute(a, b, width, bits):
    return exact_ref.limited_dot_exact(a, b, width, bits)


@pytest.mark.parametrize("width,bits", [(1, 3), (4, 5), (8, 14), (32, 14), (7, 20)])
def test_bruteforce(width, bits):
    rng = np.random.default_rng(100 + width + bits)
    for case in range(6):
        K = int(rng.integers(1, 90))
        a = _fp8_values(rng, K)
        b = _fp8_values(rng, K)
        got = oracle.limited_dot(a, b, width, bits)
        assert got == _brute(a, b, width, bits), (case, K)


def test_vectorized_matches_scalar():
    rng = np.random.default_rng(5)
    A = _fp8_values(rng, (6, 200))
    B = _fp8_values(rng, (200, 5))
    M = oracle.limited_dot(A[:, None, :], B.T[None, :, :], 16, 14)
    for i in range(6):
        for j in range(5):
            assert M[i, j] == _brute(A[i], B[:, j], 16, 14)


def test_one_step_with_enough_bits_is_rounded_exact_sum():
    rng = np.random.default_rng(6)
    a = _fp8_values(rng, 64)
    b = _fp8_values(rng, 64)
    exact = sum(Fraction(float(x)) * Fraction(float(y)) for x, y in zip(a, b))
    assert oracle.limited_dot(a, b, 64, 45) == float(np.float32(float(exact)))


def test_small_integers_lose_nothing():
    # |values| <= 15 are exact E4M3 values; 64 products and every partial sum
    # stay below 2^14, so 14 kept bits hold them all
    rng = np.random.default_rng(7)
    a = rng.integers(-15, 16, size=(3, 64)).astype(np.float64)
    b = rng.integers(-15, 16, size=(3, 64)).astype(np.float64)
    assert np.array_equal(oracle.limited_dot(a, b, 32, 14), np.sum(a * b, axis=1))


def test_odd_symmetry_and_error_shrinks_with_bits():
    rng = np.random.default_rng(8)
    a = _fp8_values(rng, (16, 2048), 0.0)
    b = _fp8_values(rng, (16, 2048), 0.0)
    assert np.array_equal(oracle.limited_dot(-a, b), -oracle.limited_dot(a, b))
    assert np.array_equal(oracle.limited_dot(a, -b), -oracle.limited_dot(a, b))
    # all-positive terms: truncation only ever drops magnitude, so the error
    # against the FP64 sum (exact: fewer than 53 significant bits) shrinks
    # strictly as bits are added
    errs = [np.max(np.abs(oracle.limited_dot(np.abs(a), np.abs(b), 32, bits) - np.sum(np.abs(a * b), axis=1)))
            for bits in (10, 14, 18, 22)]
    assert errs[0] > errs[1] > errs[2] > errs[3]


def test_group_promotion_beats_whole_k_accumulation():
    """K = 4096, 1x128 / 128x128 scales promoted per group in FP32 against
    tensor-wise scales accumulated over the whole K, both with 14 kept bits,
    each measured against the exact FP64 sum of its own quantized inputs."""
    A, B = synthetic.accum_study(4096)
    a, b = bf16_bits(A[:32]), bf16_bits(B[:, :32])
    qa, sa = oracle.quantize_per_tensor(a)
    qb, sb = oracle.quantize_per_tensor(b)
    whole = oracle.gemm_limited_per_tensor(qa, sa, qb, sb)
    ref_t = (oracle.e4m3_decode(qa) @ oracle.e4m3_decode(qb)) * (np.float64(sa) * np.float64(sb))
    e_whole = np.max(np.abs(whole - ref_t)) / np.max(np.abs(ref_t))
    qa1, sa1 = oracle.quantize_1x128(a)
    qb1, sb1 = oracle.quantize_block128(b)
    grouped = oracle.gemm_blockscaled_limited(qa1, sa1, qb1, sb1)
    ref_g = oracle.gemm_blockscaled(qa1, sa1, qb1, sb1)
    e_group = np.max(np.abs(grouped - ref_g)) / np.max(np.abs(ref_g))
    assert 1e-3 < e_whole < 0.05
    assert e_group < e_whole / 10


def test_zero_and_empty():
    assert oracle.limited_dot(np.zeros(40), np.ones(40)) == 0.0
    assert oracle.limited_dot(np.zeros(0), np.zeros(0)) == 0.0
    g = torch.Generator().manual_seed(3)
    x = bf16_bits(synthetic.randn_bf16((4, 128), 1.0, g))
    q, s = oracle.quantize_per_tensor(x)
    assert s == np.float32(np.max(np.abs(oracle.bf16_bits_to_f32(x))) / np.float32(448.0))
    assert q.shape == x.shape
