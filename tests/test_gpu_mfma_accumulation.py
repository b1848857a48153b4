"""How the gfx950 matrix cores add FP8 products, pinned on the device.

The pages promote matrix-core partial sums into FP32 at a fixed K interval
because the tensor cores they used add FP8 products with limited precision,
aligned to the largest term (inprokorea.com wr_id 735329, third paragraph;
wr_id 890463, fourth paragraph).  The GEMMs here promote every 128-deep
group, and their element-wise error bound (``tests/gpu_util.mfma_error_bound``)
rests on a model of one matrix-core instruction measured on the device:

  * the products are added in blocks of 8 consecutive k;
  * in each block every product is truncated toward zero to a multiple of
    2^(E - 13), E = the largest sum of the two operands' exponents over the
    block's products (a subnormal code counts as exponent -6), i.e. the
    alignment follows the exponent fields, not the normalized product, whose
    magnitude lies in [2^E, 2^(E+2));
  * the block sums are then combined at FP32 precision.

``fp8blk_mfma_probe`` returns one 16x16 tile product over 128 k as the
instruction computes it.  Structured operands separate the model from exact
arithmetic (a small product beside 2^16 is dropped in its block and kept in
the next one; each truncated term is dropped on its own; truncation is toward
zero; the quantum follows the block maximum's exponent); random operands are
checked against an exact evaluation of the model.  The same cases run on the
older K = 32 FP8 instruction (four chained through the FP32 accumulator): it
reads the same OCP E4M3 codes and adds in the same way, so it would give no
precision back for its lower rate.

Through the public GEMM: a single 128-deep group with unit scales returns
the instruction's result bit for bit (the fold multiplies by 1.0 and adds to
zero), and the FP32 accumulator across groups rounds to nearest even in both
scale paths (2^24 + 1 -> 2^24, 2^24 + 3 -> 2^24 + 4).
"""
from fractions import Fraction

import numpy as np
import pytest
import torch

import fp8_fine_grained_quantize_amd as fb
import oracle
from tests import exact_ref
from tests.gpu_util import f32_dev, np_f32, u8_dev

pytestmark = pytest.mark.gpu

F8 = torch.float8_e4m3fn


def _code(v: float) -> int:
    c = int(torch.tensor([v], dtype=torch.float32).to(F8).view(torch.uint8)[0])
    assert float(exact_ref.e4m3_value(c)) == v, v
    return c


def _probe(pairs, instr):
    """Row 0 of A and of B hold the (k, a, b) values, everything else zero;
    returns C[0][0]."""
    A = np.zeros((16, 128), np.uint8)
    B = np.zeros((16, 128), np.uint8)
    for k, a, b in pairs:
        A[0, k] = _code(a)
        B[0, k] = _code(b)
    C = fb.mfma_probe(torch.from_numpy(A).cuda(), torch.from_numpy(B).cuda(), instr)
    torch.cuda.synchronize()
    return float(C[0, 0])


# (name, [(k, a, b), ...], result the model gives); 2^16 = 256 * 256
CASES = [
    ("2^16 + 4 in one block: 4 below the quantum 8 is dropped", [(0, 256, 256), (1, 2, 2)], 65536.0),
    ("2^16 + 4, the 4 seven k away (same block)", [(0, 256, 256), (7, 2, 2)], 65536.0),
    ("2^16 + 4, the 4 in the next block of 8", [(0, 256, 256), (8, 2, 2)], 65540.0),
    ("4 in the first block, 2^16 in the second", [(0, 2, 2), (8, 256, 256)], 65540.0),
    ("2^16 + 8: the quantum itself is kept", [(0, 256, 256), (1, 2, 4)], 65544.0),
    ("2^16 + 12 truncated to 2^16 + 8", [(0, 256, 256), (1, 2, 6)], 65544.0),
    ("2^16 - 4: truncation toward zero drops it", [(0, 256, 256), (1, -2, 2)], 65536.0),
    ("2^16 - 8 kept", [(0, 256, 256), (1, -2, 4)], 65528.0),
    ("2^16 + 4 + 4: each term truncated on its own", [(0, 256, 256), (1, 2, 2), (2, 2, 2)], 65536.0),
    ("1.5 * 2^16 + 4: quantum from the exponent of the maximum", [(0, 384, 256), (1, 2, 2)], 98304.0),
    ("1.5 * 2^16 + 8", [(0, 384, 256), (1, 2, 4)], 98312.0),
    ("2.25 * 2^16 + 8: quantum from the exponent sum (16), not log2 (17)", [(0, 384, 384), (1, 2, 4)], 147464.0),
    ("2.25 * 2^16 + 4 dropped", [(0, 384, 384), (1, 2, 2)], 147456.0),
    ("two blocks of 2^16, the second with a dropped 4", [(0, 256, 256), (8, 256, 256), (9, 2, 2)], 131072.0),
    ("2^16 + 1", [(0, 256, 256), (1, 1, 1)], 65536.0),
    ("2^16 + 16", [(0, 256, 256), (1, 4, 4)], 65552.0),
    ("subnormal code times one", [(0, 2.0 ** -9, 1)], 2.0 ** -9),
    ("448 * 1", [(0, 448, 1)], 448.0),
    ("-3 * 5", [(0, -3, 5)], -15.0),
]


@pytest.mark.parametrize("instr", [0, 1], ids=["k128_scaled", "k32_x4"])
@pytest.mark.parametrize("case", CASES, ids=[c[0][:40] for c in CASES])
def test_structured_accumulation(case, instr):
    name, pairs, want = case
    exact = sum(a * b for _, a, b in pairs)
    got = _probe(pairs, instr)
    print(f"[mfma] instr={instr} {name}: got {got} exact {exact}", flush=True)
    assert got == want


def _exponent(code: int) -> int:
    """Unbiased exponent of an E4M3 code from its bit fields (subnormals -6)."""
    e = (int(code) >> 3) & 0xF
    return -6 if e == 0 else e - 7


def _model(A: np.ndarray, B: np.ndarray) -> np.ndarray:
    """The model, evaluated exactly: D[i][j] from codes A [16][128], B [16][128]
    (values from the enumerated E4M3 set of tests/exact_ref.py)."""
    D = np.zeros((16, 16))
    for i in range(16):
        for j in range(16):
            total = Fraction(0)
            for b in range(16):
                ks = range(8 * b, 8 * b + 8)
                p = [exact_ref.e4m3_value(int(A[i, k])) * exact_ref.e4m3_value(int(B[j, k])) for k in ks]
                if all(t == 0 for t in p):
                    continue
                E = max(_exponent(A[i, k]) + _exponent(B[j, k]) for k, t in zip(ks, p) if t != 0)
                q = Fraction(2) ** (E - 13)
                total += sum(int(t / q) * q for t in p)  # int() truncates toward zero
            D[i, j] = float(total)
    return D


@pytest.mark.parametrize("instr", [0, 1], ids=["k128_scaled", "k32_x4"])
def test_random_operands_follow_the_model(instr):
    """Random codes over the whole E4M3 range: the instruction's result
    equals the exactly evaluated block sums up to the FP32 rounding of their
    combination (at most 16 roundings of the running sum)."""
    rng = np.random.default_rng(11 + instr)
    A = rng.integers(0, 256, (16, 128)).astype(np.uint8)
    B = rng.integers(0, 256, (16, 128)).astype(np.uint8)
    A[(A & 0x7F) == 0x7F] = 0x7E
    B[(B & 0x7F) == 0x7F] = 0x7E
    C = np_f32(fb.mfma_probe(torch.from_numpy(A).cuda(), torch.from_numpy(B).cuda(), instr)).astype(np.float64)
    Ad, Bd = oracle.e4m3_decode(A), oracle.e4m3_decode(B)
    M = _model(A, B)
    exact = Ad @ Bd.T
    mag = np.abs(Ad) @ np.abs(Bd).T
    assert np.all(np.abs(C - M) <= 16 * 2.0 ** -24 * mag + 1e-300)
    # and the model is not exact arithmetic on these operands
    assert np.any(M != exact)


def test_single_group_gemm_returns_the_instruction_result():
    """K = 128 with unit scales: C = fl32(P * 1.0 + 0) = P, the raw matrix-core
    result, bit for bit (the GEMM computes C^T tiles: its B fragment is the
    instruction's first operand)."""
    rng = np.random.default_rng(12)
    A = rng.integers(0, 256, (16, 128)).astype(np.uint8)
    Bt = rng.integers(0, 256, (16, 128)).astype(np.uint8)  # B stored [N][K]
    A[(A & 0x7F) == 0x7F] = 0x00
    Bt[(Bt & 0x7F) == 0x7F] = 0x00
    sA = np.ones((1, 16), np.float32)
    sB = np.ones((1, 1), np.float32)
    C = fb.gemm_fp8_blockscaled(u8_dev(A), f32_dev(sA), u8_dev(Bt), f32_dev(sB), opB=fb.OP_T)
    P = fb.mfma_probe(torch.from_numpy(Bt).cuda(), torch.from_numpy(A).cuda(), 0)  # P[n][m]
    torch.cuda.synchronize()
    assert np.array_equal(np_f32(C).view(np.uint32), np_f32(P).T.copy().view(np.uint32))


@pytest.mark.parametrize("pow2", [False, True])
@pytest.mark.parametrize("small,want", [(1, 2.0 ** 24), (3, 2.0 ** 24 + 4)])
def test_fp32_accumulator_rounds_to_nearest_even(pow2, small, want):
    """Two groups: 2^24 from group 0 (256 * 256 with a row scale 2^8), then
    `small` from group 1 (1 * small, unit scales).  2^24 + 1 and 2^24 + 3 are
    halfway cases: the FP32 running sum rounds them to even."""
    A = np.zeros((16, 256), np.uint8)
    B = np.zeros((256, 16), np.uint8)
    A[0, 0], B[0, 0] = _code(256), _code(256)
    A[0, 128], B[128, 0] = _code(1), _code(small)
    sA = np.ones((2, 16), np.float32)
    sA[0, 0] = 2.0 ** 8
    sB = np.ones((2, 1), np.float32)
    C = fb.gemm_fp8_blockscaled(u8_dev(A), f32_dev(sA), u8_dev(B), f32_dev(sB), opB=fb.OP_N, pow2_scales=pow2,
                                split_k=False)
    torch.cuda.synchronize()
    assert float(np_f32(C)[0, 0]) == want
