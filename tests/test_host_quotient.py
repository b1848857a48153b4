"""The requantizer's default-mode quotient, checked on the host.

The GPU re-quantizer (128x1 tiles from cached 1x128 codes) forms the IEEE
FP32 quotient fl32(x / s) of a dequantized value x and its tile scale s as
fl32(x * r) with r = fl64(1 / s) and the product in FP64.  The argument:
x and s have 24-bit significands, so x / s is never exactly a midpoint
between two FP32 values and lies at least 2^-49 (relative) away from every
midpoint, while x * r is within about 2^-52 of x / s; both therefore round
to the same FP32 value.  numpy's FP64 and FP32 arithmetic is IEEE with
round-to-nearest-even, as the device's is, so these cases check the
argument (not the kernel, which the GPU tests compare with the oracle).
"""
import numpy as np


def _route(x: np.ndarray, s: np.ndarray) -> np.ndarray:
    return (x.astype(np.float64) * (1.0 / s.astype(np.float64))).astype(np.float32)


def _same(a: np.ndarray, b: np.ndarray) -> bool:
    return bool(np.array_equal(a.view(np.uint32), b.view(np.uint32)))


def test_requantizer_domain():
    """x = fl32(e4m3 value * 1x128 scale), s = fl32(amax / 448) with amax >= |x|,
    scales over the whole FP32 range including subnormal ones."""
    rng = np.random.default_rng(0)
    n = 1_000_000
    codes = rng.integers(0, 256, n).astype(np.uint8)
    codes[(codes & 0x7F) == 0x7F] = 0
    e = ((codes >> 3) & 0xF).astype(np.int64)
    m = (codes & 7).astype(np.float64)
    d = np.where(e == 0, m * 2.0 ** -9, (1 + m / 8) * 2.0 ** (e - 7)) * np.where(codes & 0x80, -1, 1)
    so = (rng.random(n) * 2.0 ** rng.integers(-149, 120, n)).astype(np.float32)
    so[so == 0] = np.float32(2.0 ** -149)
    with np.errstate(under="ignore"):
        x = (d.astype(np.float32) * so).astype(np.float32)
        amax = (np.abs(x) * (1 + rng.random(n) * 8).astype(np.float32)).astype(np.float32)
        s = (amax / np.float32(448)).astype(np.float32)
    s[s == 0] = 1
    assert np.sum(s < 2.0 ** -126) > 1000
    with np.errstate(under="ignore"):
        assert _same(_route(x, s), (x / s).astype(np.float32))


def test_arbitrary_finite_pairs():
    rng = np.random.default_rng(1)
    n = 1_000_000
    x = rng.integers(0, 0x7F000000, n, dtype=np.uint32).view(np.float32)
    s = rng.integers(1, 0x7F000000, n, dtype=np.uint32).view(np.float32)
    with np.errstate(over="ignore", under="ignore"):
        ref = (x / s).astype(np.float32)
        got = _route(x, s)
    keep = np.isfinite(ref) & (np.abs(ref) < 2.0 ** 127)
    assert _same(got[keep], ref[keep])


def test_quotients_next_to_midpoints():
    """The hardest cases: x = fl32(m * s) for m a midpoint between two FP32
    values, so that x / s lies within about 2^-24 (relative) of m."""
    rng = np.random.default_rng(2)
    n = 1_000_000
    mid = (rng.integers(2 ** 24, 2 ** 25, n) | 1).astype(np.float64) * 2.0 ** rng.integers(-40, 8, n)
    s = (1 + rng.random(n)).astype(np.float32) * np.float32(2.0) ** rng.integers(-60, 60, n).astype(np.float32)
    x = (mid * s.astype(np.float64)).astype(np.float32)
    with np.errstate(over="ignore", under="ignore"):
        ref = (x / s).astype(np.float32)
        got = _route(x, s)
    keep = np.isfinite(ref)
    assert keep.mean() > 0.99
    assert _same(got[keep], ref[keep])
