"""Exact pins for the oracle functions that the quantizer and GEMM pins do not
reach (CPU only):

* ``dequantize_block128`` and ``dequantize_1x128``: every element of a
  ragged grid equals dec(q) * s evaluated with Python fractions, where the
  code's value comes from the enumerated E4M3 value set of
  ``tests/exact_ref.py`` (not from the oracle's bit-field decoder) and the
  scale is the stored FP32 value of the element's block or tile;
* ``quantize_per_tensor``: codes and scale equal the exact rational
  quantization of the whole tensor as one tile (tensor-wise scaling, which
  the pages contrast with their tiles);
* ``gemm_limited_per_tensor`` and ``gemm_blockscaled_limited``: every output
  equals the exact evaluation of the limited-accumulation rule
  (``exact_ref.limited_dot_exact``) followed by the scale arithmetic each
  function states, rounded exactly as stated (FP64 for the tensor-wise
  product, binary32 for the per-group promotion).

A dropped scale, a transposed block index, a wrong tile boundary, a code
decoded through the wrong table or a scale applied to the wrong group fails
one of these.
"""
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
from synthetic import bf16_bits, edge_tensor, randn_bf16
from tests import exact_ref


def _codes(rng, shape):
    """Random E4M3 codes without the two NaN codes, some zeros of both signs."""
    q = rng.integers(0, 256, size=shape).astype(np.uint8)
    q[(q & 0x7F) == 0x7F] = 0x7E
    q[rng.random(shape) < 0.05] = 0x00
    q[rng.random(shape) < 0.02] = 0x80
    return q


def _scales(rng, shape):
    """Random positive FP32 scales spanning many binades (normal and subnormal)."""
    mant = rng.random(shape) + 1.0
    ex = rng.integers(-140, 40, size=shape)
    return (mant * np.exp2(ex)).astype(np.float32)


def test_dequantize_block128_exact_ragged():
    rng = np.random.default_rng(41)
    R, C = 130, 140  # 2 x 2 blocks, the last row and column of blocks partial
    q = _codes(rng, (R, C))
    s = _scales(rng, (2, 2))
    s[1, 0] = np.float32(2.0 ** -140)  # a subnormal scale
    d = oracle.dequantize_block128(q, s)
    assert d.shape == (R, C) and d.dtype == np.float64
    for r in range(R):
        for c in range(C):
            want = exact_ref.e4m3_value(int(q[r, c])) * Fraction(float(s[r // 128, c // 128]))
            assert Fraction(float(d[r, c])) == want, (r, c)


def test_dequantize_block128_of_quantized_weight_is_within_half_step():
    """On a quantized BF16 weight: each element is recovered to within half an
    E4M3 step of its block (saturation cannot occur in the default mode)."""
    g = torch.Generator().manual_seed(42)
    w = bf16_bits(randn_bf16((130, 257), 0.006, g))
    q, s = oracle.quantize_block128(w)
    d = oracle.dequantize_block128(q, s)
    x = oracle.bf16_bits_to_f32(w).astype(np.float64)
    # E4M3 relative step is 2^-3 in the normal range; subnormal codes have an
    # absolute step of 2^-9 * s
    sc = np.repeat(np.repeat(s.astype(np.float64), 128, 0), 128, 1)[:130, :257]
    bound = np.maximum(np.abs(x) * 2.0 ** -4, 2.0 ** -10 * sc) * (1 + 2.0 ** -20)
    assert np.all(np.abs(d - x) <= bound)


def test_dequantize_1x128_exact_ragged():
    rng = np.random.default_rng(43)
    M, K = 5, 300  # three groups, the last partial
    q = _codes(rng, (M, K))
    s = _scales(rng, (3, M))
    d = oracle.dequantize_1x128(q, s)
    for m in range(M):
        for k in range(K):
            want = exact_ref.e4m3_value(int(q[m, k])) * Fraction(float(s[k // 128, m]))
            assert Fraction(float(d[m, k])) == want, (m, k)


@pytest.mark.parametrize("seed,edge", [(44, False), (45, True)])
def test_quantize_per_tensor_codes_exact(seed, edge):
    g = torch.Generator().manual_seed(seed)
    shape = (5, 37)
    x = bf16_bits(edge_tensor(shape, seed) if edge else randn_bf16(shape, 3.0, g))
    q, s = oracle.quantize_per_tensor(x)
    codes, sc = exact_ref.quantize_values([int(b) for b in x.reshape(-1)], False)
    assert np.float32(s).view(np.uint32) == np.float32(sc).view(np.uint32)
    assert list(q.reshape(-1)) == codes


def test_quantize_per_tensor_all_zero_and_empty():
    q, s = oracle.quantize_per_tensor(np.array([[0x0000, 0x8000, 0x0000]], np.uint16))
    assert s == np.float32(1.0) and list(q[0]) == [0x00, 0x80, 0x00]
    q, s = oracle.quantize_per_tensor(np.zeros((0, 4), np.uint16))
    assert q.shape == (0, 4) and s == np.float32(1.0)


@pytest.mark.parametrize("width,bits", [(32, 14), (8, 10), (128, 14)])
def test_gemm_limited_per_tensor_exact(width, bits):
    rng = np.random.default_rng(46 + width)
    M, K, N = 3, 200, 2
    A = _codes(rng, (M, K))
    B = _codes(rng, (K, N))
    sA, sB = np.float32(0.0371), np.float32(2.0 ** -7 * 1.3)
    C = oracle.gemm_limited_per_tensor(A, sA, B, sB, width, bits)
    for m in range(M):
        a = [float(exact_ref.e4m3_value(int(c))) for c in A[m]]
        for n in range(N):
            b = [float(exact_ref.e4m3_value(int(c))) for c in B[:, n]]
            p = Fraction(exact_ref.limited_dot_exact(a, b, width, bits))
            want = float(p * Fraction(float(sA)) * Fraction(float(sB)))  # one FP64 rounding
            assert C[m, n] == want, (m, n)


def test_gemm_blockscaled_limited_exact():
    rng = np.random.default_rng(47)
    M, K, N = 2, 384, 130  # three groups; two 128-column scale blocks, the second partial
    A = _codes(rng, (M, K))
    B = _codes(rng, (K, N))
    sA = (rng.random((3, M)) + 1.0).astype(np.float32) * np.float32(2.0 ** -9)
    sB = (rng.random((3, 2)) + 1.0).astype(np.float32) * np.float32(2.0 ** -6)
    C = oracle.gemm_blockscaled_limited(A, sA, B, sB, 32, 14)
    for m in range(M):
        for n in (0, 1, 77, 127, 128, 129):
            acc = Fraction(0)
            for g in range(3):
                a = [float(exact_ref.e4m3_value(int(c))) for c in A[m, 128 * g:128 * g + 128]]
                b = [float(exact_ref.e4m3_value(int(c))) for c in B[128 * g:128 * g + 128, n]]
                p = Fraction(exact_ref.limited_dot_exact(a, b, 32, 14))
                sc = Fraction(exact_ref.round_to_f32(Fraction(float(sA[g, m])) * Fraction(float(sB[g, n // 128]))))
                t = Fraction(exact_ref.round_to_f32(p * sc))
                acc = Fraction(exact_ref.round_to_f32(acc + t))
            assert Fraction(float(C[m, n])) == acc, (m, n)
