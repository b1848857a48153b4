"""Pins for the oracle's quantizers (CPU only).

* hand-derived worked cases (tests/golden/quant_cases.json);
* exact rational brute force (tests/exact_ref.py) on tiny tensors;
* invariants that the definitions fix: E4M3-representable tiles round-trip,
  a tile's amax maps to +-448, power-of-two scales rescale exactly, scaling by
  2^j and negation act on codes and scales as they must, row permutation
  commutes, 128x1 equals 1x128 of the transpose, and a block scale is the
  max of its rows' tile scales.
"""
import numpy as np
import pytest

import oracle
from synthetic import bf16_bits, edge_tensor, randn_bf16
from tests import exact_ref
from tests.golden_cases import load_cases

import torch

QUANT = {"1x128": oracle.quantize_1x128, "128x1": oracle.quantize_128x1,
         "block128": oracle.quantize_block128}


@pytest.mark.parametrize("case", load_cases(), ids=lambda c: c["name"][:40])
def test_golden_cases(case):
    q, s = QUANT[case["kind"]](case["x"], pow2=case["pow2"])
    assert np.array_equal(s.view(np.uint32), case["scale_bits"]), (s.view(np.uint32), case["scale_bits"])
    for r, c, code in case["codes"]:
        assert q[r, c] == code, (r, c, hex(q[r, c]), hex(code))


def _bits(shape, seed, edge=False):
    g = torch.Generator().manual_seed(seed)
    if edge:
        return bf16_bits(edge_tensor(shape, seed))
    return bf16_bits(randn_bf16(shape, 1.0, g, outlier_cols=2, outlier_factor=40.0))


@pytest.mark.parametrize("pow2", [False, True])
@pytest.mark.parametrize("edge", [False, True])
def test_1x128_bruteforce(pow2, edge):
    x = _bits((3, 200), 11 + edge, edge)
    q, s = oracle.quantize_1x128(x, pow2)
    for m in range(3):
        for g, (c0, c1) in enumerate([(0, 128), (128, 200)]):
            codes, sc = exact_ref.quantize_values([int(b) for b in x[m, c0:c1]], pow2)
            assert s[g, m] == np.float32(sc), (m, g, s[g, m], sc)
            assert list(q[m, c0:c1]) == codes


@pytest.mark.parametrize("pow2", [False, True])
def test_128x1_bruteforce(pow2):
    x = _bits((150, 3), 21, edge=True)
    qT, s = oracle.quantize_128x1(x, pow2)
    for c in range(3):
        for g, (t0, t1) in enumerate([(0, 128), (128, 150)]):
            codes, sc = exact_ref.quantize_values([int(b) for b in x[t0:t1, c]], pow2)
            assert s[g, c] == np.float32(sc)
            assert list(qT[c, t0:t1]) == codes


@pytest.mark.parametrize("pow2", [False, True])
def test_block128_bruteforce(pow2):
    x = _bits((130, 140), 31, edge=True)
    q, s = oracle.quantize_block128(x, pow2)
    for i, (r0, r1) in enumerate([(0, 128), (128, 130)]):
        for j, (c0, c1) in enumerate([(0, 128), (128, 140)]):
            blk = [int(b) for b in x[r0:r1, c0:c1].reshape(-1)]
            codes, sc = exact_ref.quantize_values(blk, pow2)
            assert s[i, j] == np.float32(sc)
            assert list(q[r0:r1, c0:c1].reshape(-1)) == codes


def _representable_tile_bits(rng, rows, cols, j):
    """Tiles of E4M3 values times 2^j, each row containing +-448*2^j."""
    codes = rng.integers(0, 0x7F, size=(rows, cols)).astype(np.uint8)
    codes |= (rng.integers(0, 2, size=(rows, cols)) << 7).astype(np.uint8)
    codes[:, ::128] = 0x7E  # every 1x128 tile and every column tile holds 448
    v = (oracle.e4m3_decode(codes) * 2.0 ** j).astype(np.float32)
    bits = (v.view(np.uint32) >> 16).astype(np.uint16)
    assert np.array_equal(oracle.bf16_bits_to_f32(bits), v)  # exact in BF16
    return bits, codes


@pytest.mark.parametrize("j", [-20, -3, 0, 5, 40])
def test_roundtrip_representable(j):
    rng = np.random.default_rng(100 + j)
    bits, codes = _representable_tile_bits(rng, 4, 256, j)
    for pow2 in (False, True):
        q, s = oracle.quantize_1x128(bits, pow2)
        assert np.all(s == np.float32(2.0 ** j))
        assert np.array_equal(q, codes)
        assert np.array_equal(oracle.dequantize_1x128(q, s), oracle.bf16_bits_to_f32(bits).astype(np.float64))


def test_amax_maps_to_448_default_mode():
    x = _bits((64, 1024), 5, edge=False)
    q, s = oracle.quantize_1x128(x, False)
    xf = oracle.bf16_bits_to_f32(x)
    for g in range(8):
        tile = xf[:, g * 128:(g + 1) * 128]
        idx = np.argmax(np.abs(tile), axis=1)
        picked = q[np.arange(64), g * 128 + idx]
        assert np.all(picked & 0x7F == 0x7E)
        assert np.all((picked >> 7) == np.signbit(tile[np.arange(64), idx]))


def test_pow2_amax_code_range_and_exactness():
    x = _bits((64, 1024), 6, edge=False)
    q, s = oracle.quantize_1x128(x, True)
    mant = s.view(np.uint32) & 0x7FFFFF
    assert np.all(mant == 0), "power-of-two scales"
    xf = oracle.bf16_bits_to_f32(x)
    for g in range(8):
        tile = xf[:, g * 128:(g + 1) * 128]
        amax = np.max(np.abs(tile), axis=1)
        y = amax / s[g]
        assert np.all((y > 224) & (y <= 448))
        # division by a power of two is exact: fl32(x/s) * s == x
        yy = (tile / s[g][:, None]).astype(np.float32)
        assert np.array_equal(yy * s[g][:, None], tile)


@pytest.mark.parametrize("pow2", [False, True])
def test_equivariance_scale_and_sign(pow2):
    x = _bits((16, 512), 7, edge=False)
    xf = oracle.bf16_bits_to_f32(x)
    q, s = oracle.quantize_1x128(x, pow2)
    for j in (-7, 3, 11):
        xs = (xf * np.float32(2.0 ** j)).astype(np.float32)
        bits = (xs.view(np.uint32) >> 16).astype(np.uint16)
        q2, s2 = oracle.quantize_1x128(bits, pow2)
        assert np.array_equal(q2, q)
        assert np.array_equal(s2, (s * np.float32(2.0 ** j)).astype(np.float32))
    qn, sn = oracle.quantize_1x128(x ^ np.uint16(0x8000), pow2)
    assert np.array_equal(qn, q ^ np.uint8(0x80))
    assert np.array_equal(sn, s)


def test_row_permutation_commutes():
    x = _bits((40, 384), 8, edge=True)
    perm = np.random.default_rng(0).permutation(40)
    q, s = oracle.quantize_1x128(x)
    qp, sp = oracle.quantize_1x128(x[perm])
    assert np.array_equal(qp, q[perm]) and np.array_equal(sp, s[:, perm])


@pytest.mark.parametrize("pow2", [False, True])
def test_128x1_is_1x128_of_transpose(pow2):
    x = _bits((300, 70), 9, edge=True)
    qT, s = oracle.quantize_128x1(x, pow2)
    q2, s2 = oracle.quantize_1x128(np.ascontiguousarray(x.T), pow2)
    assert np.array_equal(qT, q2) and np.array_equal(s, s2)


def test_block_scale_is_max_of_row_tiles():
    x = _bits((256, 384), 10, edge=False)
    qb, sb = oracle.quantize_block128(x)
    _, s1 = oracle.quantize_1x128(x)  # [3][256]
    xf = oracle.bf16_bits_to_f32(x)
    for i in range(2):
        for j in range(3):
            row_amax = np.max(np.abs(xf[i * 128:(i + 1) * 128, j * 128:(j + 1) * 128]), axis=1)
            assert np.array_equal(row_amax / np.float32(448), s1[j, i * 128:(i + 1) * 128])
            assert sb[i, j] == np.float32(np.max(row_amax)) / np.float32(448)
            assert sb[i, j] == np.max(s1[j, i * 128:(i + 1) * 128])


def test_requantize_from_1x128_exact_case():
    """When the 1x128 codes are exact (E4M3 values times a power of two per
    row tile), dequantizing and re-quantizing 128x1 must equal quantizing the
    original tensor 128x1."""
    rng = np.random.default_rng(3)
    bits, _ = _representable_tile_bits(rng, 256, 256, 0)
    q, s = oracle.quantize_1x128(bits)
    for pow2 in (False, True):
        qT, sT = oracle.requantize_128x1_from_1x128(q, s, pow2)
        qT2, sT2 = oracle.quantize_128x1(bits, pow2)
        assert np.array_equal(qT, qT2) and np.array_equal(sT, sT2)


def test_requantize_from_1x128_bruteforce():
    x = _bits((130, 140), 12, edge=False)
    q, s = oracle.quantize_1x128(x)
    qT, sT = oracle.requantize_128x1_from_1x128(q, s)
    from fractions import Fraction
    for c in (0, 77, 139):
        g1 = c // 128
        deq = [exact_ref.round_to_f32(exact_ref.e4m3_value(int(q[t, c])) * Fraction(float(s[g1, t])),
                                      negative_zero=bool(q[t, c] & 0x80)) for t in range(130)]
        for g, (t0, t1) in enumerate([(0, 128), (128, 130)]):
            vals = deq[t0:t1]
            amax = max(abs(Fraction(v)) for v in vals)
            sc = exact_ref.scale_of(amax, False)
            assert sT[g, c] == np.float32(sc)
            for t in range(t0, t1):
                y = exact_ref.round_to_f32(Fraction(vals[t - t0]) / Fraction(sc),
                                           negative_zero=np.signbit(vals[t - t0]))
                assert qT[c, t] == exact_ref.e4m3_nearest(y)


def test_empty_inputs():
    q, s = oracle.quantize_1x128(np.zeros((0, 256), np.uint16))
    assert q.shape == (0, 256) and s.shape == (2, 0)
    qT, s = oracle.quantize_128x1(np.zeros((0, 5), np.uint16))
    assert qT.shape == (5, 0) and s.shape == (0, 5)
