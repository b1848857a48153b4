"""Pins for the oracle's E4M3 encoder and decoder (CPU only).

The encoder is checked exhaustively against torch's ``float8_e4m3fn`` cast (a
library routine that rounds to nearest even and keeps the sign of zero) over
every binary32 value with 2^-11 <= |y| < 464, and separately for saturation,
which torch does not do (it returns NaN from 464 up).  The decoder is checked
against the same library type and against closed forms.
"""
import math

import numpy as np
import pytest
import torch

import oracle
from tests import exact_ref


def test_decode_all_codes_match_library():
    codes = np.arange(256, dtype=np.uint8)
    ours = oracle.e4m3_decode(codes)
    lib = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    nan_ours = np.isnan(ours)
    assert np.array_equal(nan_ours, np.isnan(lib))
    assert set(np.nonzero(nan_ours)[0]) == {0x7F, 0xFF}
    assert np.array_equal(ours[~nan_ours], lib[~nan_ours])
    assert np.array_equal(np.signbit(ours[~nan_ours]), np.signbit(lib[~nan_ours]))


def test_decode_closed_forms():
    d = oracle.e4m3_decode
    assert d(np.uint8(0x7E)) == 448.0
    assert d(np.uint8(0xFE)) == -448.0
    assert d(np.uint8(0x01)) == 2.0 ** -9
    assert d(np.uint8(0x07)) == 7 * 2.0 ** -9
    assert d(np.uint8(0x08)) == 2.0 ** -6
    assert d(np.uint8(0x38)) == 1.0
    assert np.signbit(d(np.uint8(0x80))) and d(np.uint8(0x80)) == 0.0
    pos = d(np.arange(0x7F, dtype=np.uint8))
    assert np.all(np.diff(pos) > 0), "positive codes must increase strictly"
    assert np.isfinite(d(np.arange(256, dtype=np.uint8))).sum() == 254
    # the enumeration used by the brute-force reference agrees
    assert [float(v) for v in exact_ref.E4M3_POS] == list(pos)


def _positive_f32_range(lo_bits, hi_bits, chunk=1 << 24):
    b = lo_bits
    while b < hi_bits:
        e = min(hi_bits, b + chunk)
        yield np.arange(b, e, dtype=np.uint32).view(np.float32)
        b = e


def test_encode_exhaustive_against_library():
    lo = int(np.float32(2.0 ** -11).view(np.uint32))
    hi = int(np.float32(464.0).view(np.uint32))  # exclusive
    n = 0
    for y in _positive_f32_range(lo, hi):
        ours = oracle.e4m3_encode(y)
        lib = torch.from_numpy(y).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
        bad = np.nonzero(ours != lib)[0]
        assert bad.size == 0, f"mismatch at y={y[bad[0]]!r}: {ours[bad[0]]:#x} vs {lib[bad[0]]:#x}"
        n += y.size
    assert n > 1.5e8


def test_encode_sign_symmetry_and_tiny():
    rng = np.random.default_rng(1)
    bits = rng.integers(0, 0x43E80000, size=2_000_000, dtype=np.uint32)  # |y| < 464
    y = bits.view(np.float32)
    pos = oracle.e4m3_encode(y)
    neg = oracle.e4m3_encode(-y)
    assert np.array_equal(neg, pos | 0x80)
    lib = torch.from_numpy(-y).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(neg, lib)
    # everything at or below 2^-10 rounds to a zero code, keeping the sign
    tiny = np.array([0.0, 2.0 ** -149, 2.0 ** -20, 2.0 ** -10], np.float32)
    assert np.array_equal(oracle.e4m3_encode(tiny), np.zeros(4, np.uint8))
    assert np.array_equal(oracle.e4m3_encode(-tiny), np.full(4, 0x80, np.uint8))
    assert oracle.e4m3_encode(np.float32(np.nextafter(np.float32(2 ** -10), np.float32(1)))) == 0x01


def test_encode_saturates():
    big = np.array([np.nextafter(np.float32(448), np.float32(1e9)), 463.99997, 464.0, 480.0,
                    1e6, 3.4028235e38, np.inf], np.float32)
    assert np.all(oracle.e4m3_encode(big) == 0x7E)
    assert np.all(oracle.e4m3_encode(-big) == 0xFE)


def test_encode_decode_roundtrip_all_codes():
    codes = np.array([c for c in range(256) if c & 0x7F != 0x7F], np.uint8)
    vals = oracle.e4m3_decode(codes).astype(np.float32)
    assert np.array_equal(oracle.e4m3_encode(vals), codes)


def test_encode_ties_go_to_even():
    pos = oracle.e4m3_decode(np.arange(0x7F, dtype=np.uint8))
    mids = ((pos[:-1] + pos[1:]) / 2).astype(np.float32)
    assert np.array_equal(mids.astype(np.float64), (pos[:-1] + pos[1:]) / 2), "midpoints exact in f32"
    enc = oracle.e4m3_encode(mids)
    lo = np.arange(0x7E)
    want = np.where(lo % 2 == 0, lo, lo + 1)
    assert np.array_equal(enc, want.astype(np.uint8))


@pytest.mark.parametrize("seed", [0, 1])
def test_encode_matches_bruteforce_sample(seed):
    rng = np.random.default_rng(seed)
    y = (rng.standard_normal(400) * np.exp2(rng.integers(-14, 10, 400))).astype(np.float32)
    y[:6] = [0.0, -0.0, 448.0, -500.0, 2.0 ** -10, -(2.0 ** -10)]
    ours = oracle.e4m3_encode(y)
    for v, c in zip(y, ours):
        assert c == exact_ref.e4m3_nearest(float(v)), (v, c)
