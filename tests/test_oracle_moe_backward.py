"""Pins for the oracle's MoE backward functions (CPU only): the ragged
per-expert 128x1 quantization of Wgrad operands and the grouped Wgrad.

* the group-slot layout on a hand-worked offset list;
* exact rational brute force (tests/exact_ref.py) of every ragged group's
  codes and scale, including experts with 0, 1, 127, 128 and 129 tokens;
* special case: experts whose token counts are multiples of 128 reduce to
  the dense 128x1 quantizer of the whole tensor;
* closed form: integer inputs with power-of-two scales quantize exactly, so
  each expert's grouped Wgrad equals the integer product X_e^T dY_e;
* brute force of the grouped Wgrad on a tiny ragged case (Fraction sums), and
  the sampled-entry form agreeing bit for bit with the full form.
"""
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
from synthetic import bf16_bits, edge_tensor, randn_bf16
from tests import exact_ref


def test_token_group_starts_worked_example():
    # experts with 0, 5, 128, 128, 39 tokens: 0, 1, 1, 1, 1 groups
    assert list(oracle.token_group_starts([0, 0, 5, 133, 261, 300])) == [0, 0, 1, 2, 3, 4]
    # 129 tokens need two groups, 256 exactly two, 1 one
    assert list(oracle.token_group_starts([0, 129, 385, 386])) == [0, 2, 4, 5]
    assert list(oracle.token_group_starts([0])) == [0]


@pytest.mark.parametrize("pow2", [False, True])
def test_grouped_128x1_bruteforce(pow2):
    counts = [1, 0, 129, 127, 128, 3]
    off = np.concatenate([[0], np.cumsum(counts)])
    T, C = int(off[-1]), 3
    x = bf16_bits(edge_tensor((T, C), 31 + pow2))
    qT, s = oracle.quantize_128x1_grouped(x, off, pow2)
    PG = oracle.token_group_starts(off)
    assert qT.shape == (C, 128 * int(PG[-1])) and s.shape == (int(PG[-1]), C)
    for e in range(len(counts)):
        for g in range(int(PG[e + 1] - PG[e])):
            t0 = int(off[e]) + 128 * g
            t1 = min(t0 + 128, int(off[e + 1]))
            slot = int(PG[e]) + g
            for c in range(C):
                codes, sc = exact_ref.quantize_values([int(b) for b in x[t0:t1, c]], pow2)
                assert s[slot, c] == np.float32(sc), (e, g, c)
                col = 128 * slot
                assert list(qT[c, col:col + (t1 - t0)]) == codes, (e, g, c)
                assert not qT[c, col + (t1 - t0):col + 128].any(), "padding must be code 0"


@pytest.mark.parametrize("pow2", [False, True])
def test_grouped_128x1_aligned_reduces_to_dense(pow2):
    counts = [256, 0, 128, 384]
    off = np.concatenate([[0], np.cumsum(counts)])
    g = torch.Generator().manual_seed(7)
    x = bf16_bits(randn_bf16((int(off[-1]), 200), 1.0, g, outlier_cols=3, outlier_factor=30.0))
    qg, sg = oracle.quantize_128x1_grouped(x, off, pow2)
    qd, sd = oracle.quantize_128x1(x, pow2)
    assert np.array_equal(qg, qd)
    assert np.array_equal(sg.view(np.uint32), sd.view(np.uint32))


def test_grouped_wgrad_integer_closed_form():
    # integers |v| <= 15 have at most four significant bits; with power-of-two
    # scales every one of them is an exact E4M3 value times the scale, so the
    # quantized product is the exact integer product
    rng = np.random.default_rng(3)
    counts = [5, 0, 130, 128, 1, 61]
    off = np.concatenate([[0], np.cumsum(counts)])
    T, M, N = int(off[-1]), 40, 33
    X = rng.integers(-15, 16, size=(T, M))
    dY = rng.integers(-15, 16, size=(T, N))
    xb = bf16_bits(torch.tensor(X, dtype=torch.bfloat16))
    yb = bf16_bits(torch.tensor(dY, dtype=torch.bfloat16))
    AT, sA = oracle.quantize_128x1_grouped(xb, off, pow2=True)
    BT, sB = oracle.quantize_128x1_grouped(yb, off, pow2=True)
    W = oracle.grouped_wgrad_blockscaled(off, AT, sA, BT, sB)
    assert W.shape == (len(counts), M, N)
    for e in range(len(counts)):
        t0, t1 = off[e], off[e + 1]
        ref = X[t0:t1].T.astype(np.int64) @ dY[t0:t1].astype(np.int64)
        assert np.array_equal(W[e], ref.astype(np.float64)), e


def test_grouped_wgrad_bruteforce_and_entries():
    rng = np.random.default_rng(4)
    counts = [130, 0, 7]
    off = np.concatenate([[0], np.cumsum(counts)])
    T, M, N = int(off[-1]), 2, 3
    x = bf16_bits(edge_tensor((T, M), 41))
    y = bf16_bits(edge_tensor((T, N), 42))
    AT, sA = oracle.quantize_128x1_grouped(x, off)
    BT, sB = oracle.quantize_128x1_grouped(y, off)
    W = oracle.grouped_wgrad_blockscaled(off, AT, sA, BT, sB)
    PG = oracle.token_group_starts(off)
    assert not W[1].any()
    for e in (0, 2):
        for m in range(M):
            for n in range(N):
                ex = Fraction(0)
                for g in range(int(PG[e]), int(PG[e + 1])):
                    P = sum(exact_ref.e4m3_value(int(AT[m, t])) * exact_ref.e4m3_value(int(BT[n, t]))
                            for t in range(128 * g, 128 * g + 128))
                    ex += Fraction(float(sA[g, m])) * Fraction(float(sB[g, n])) * P
                assert abs(Fraction(W[e, m, n]) - ex) <= abs(ex) * Fraction(1, 2 ** 48) + Fraction(1, 2 ** 300)
                got = oracle.grouped_wgrad_entries(off, AT, sA, BT, sB, [e], [m], [n])[0]
                assert got == W[e, m, n]
