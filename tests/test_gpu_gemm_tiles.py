"""GPU parity of the dense GEMM's tile shapes against each other and the oracle.

The dense GEMM takes 256x256 tiles, 224x256 tiles (when they need fewer
tile rows per CU: e.g. a 7168 x 2048 output is 224 tiles of 256 rows on 256
CUs, one launch wave with 32 CUs idle, or exactly 256 tiles of 224 rows) or
128x128 tiles (too few big tiles to fill the GPU).  Every tile shape computes
an output element with the same instructions in the same order (one MFMA per
128-deep K group, the same scale fold), so a GEMM whose rows are split over
calls small enough to take the 128x128 tiles must give a bitwise identical
result.  The shapes below are chosen, for 256 CUs, so that:
  4000 x 4000: 256 tiles of 256x256 (224x256 would need 288, two waves);
  6994 / 7091 x 2008: 224 tiles of 256x256 or 256 of 224x256 -> 224x256, with
    a ragged last row tile of 50 rows (its second wave row idle) or 147 rows,
    and a ragged last column tile of 216 columns;
  row slices of at most 1792 rows x 2008 or 1000 x 4000: 128x128 tiles.
"""
import numpy as np
import pytest
import torch

import fp8_fine_grained_quantize_amd as fb
import oracle
import synthetic
from synthetic import bf16_bits
from tests.gpu_util import e_norm, f32_dev, np_f32, u8_dev

pytestmark = pytest.mark.gpu

CASES = [(oracle.OP_N, oracle.BSCALE_BLOCK128), (oracle.OP_T, oracle.BSCALE_BLOCK128),
         (oracle.OP_N, oracle.BSCALE_ROW128), (oracle.OP_T, oracle.BSCALE_ROW128)]


def _small_int_codes(rng, shape):
    vals = np.array([0x00, 0x38, 0x40, 0x48, 0xB8, 0xC0, 0xC8], np.uint8)  # 0, +-1, +-2, +-4
    return vals[rng.integers(0, vals.size, size=shape)]


def _operands(M, N, K, opB, mode, pow2, seed):
    """Oracle-quantized operands in the layouts of the four GEMM modes."""
    g = torch.Generator().manual_seed(seed)
    A = synthetic.randn_bf16((M, K), 1.0, g, outlier_cols=3, outlier_factor=30.0)
    qA, sA = oracle.quantize_1x128(bf16_bits(A), pow2)
    if opB == oracle.OP_N:
        B = synthetic.randn_bf16((K, N), 0.02, g)
        if mode == oracle.BSCALE_BLOCK128:
            qB, sB = oracle.quantize_block128(bf16_bits(B), pow2)
        else:
            qBT, sB = oracle.quantize_128x1(bf16_bits(B), pow2)
            qB = np.ascontiguousarray(qBT.T)
    else:
        B = synthetic.randn_bf16((N, K), 0.02, g)
        qB, sB = (oracle.quantize_block128(bf16_bits(B), pow2) if mode == oracle.BSCALE_BLOCK128 else
                  oracle.quantize_1x128(bf16_bits(B), pow2))
    return qA, sA, qB, sB


def _gemm(qA, sA, qB, sB, opB, mode, pow2, out_dtype=torch.float32):
    C = fb.gemm_fp8_blockscaled(u8_dev(qA), f32_dev(np.ascontiguousarray(sA)), u8_dev(qB), f32_dev(sB), opB=opB,
                                bscale_mode=mode, pow2_scales=pow2, out_dtype=out_dtype)
    torch.cuda.synchronize()
    return C.cpu()


def _by_row_slices(qA, sA, qB, sB, opB, mode, pow2, rows, out_dtype=torch.float32):
    M = qA.shape[0]
    parts = [_gemm(qA[r0:r0 + rows], sA[:, r0:r0 + rows], qB, sB, opB, mode, pow2, out_dtype)
             for r0 in range(0, M, rows)]
    return torch.cat(parts, 0)


def _bits(C):
    return C.view(torch.int32 if C.dtype == torch.float32 else torch.int16).numpy()


@pytest.mark.parametrize("pow2", [False, True])
@pytest.mark.parametrize("opB,mode", CASES)
@pytest.mark.parametrize("M,N", [(4000, 4000), (7091, 2008)])
def test_exact_small_integers_bitwise_big_tiles(M, N, opB, mode, pow2):
    """Small-integer codes with power-of-two scales (every product and sum
    exact) on the 256x256 and the 224x256 tiles: equal to the oracle."""
    rng = np.random.default_rng(17)
    K = 384
    G = K // 128
    qA = _small_int_codes(rng, (M, K))
    qB = _small_int_codes(rng, (K, N) if opB == oracle.OP_N else (N, K))
    sA = np.exp2(rng.integers(-3, 4, size=(G, M))).astype(np.float32)
    NB = -(-N // 128)
    if mode == oracle.BSCALE_ROW128:
        sB = np.exp2(rng.integers(-3, 4, size=(G, N))).astype(np.float32)
    else:
        sB = np.exp2(rng.integers(-3, 4, size=(G, NB) if opB == oracle.OP_N else (NB, G))).astype(np.float32)
    print(f"[tiles] exact {M}x{N}x{K} opB={opB} mode={mode} pow2={pow2}", flush=True)
    C = _gemm(qA, sA, qB, sB, opB, mode, pow2).numpy()
    R = oracle.gemm_blockscaled(qA, sA, qB, sB, opB, mode)
    assert np.array_equal(C.astype(np.float64), R)


@pytest.mark.parametrize("pow2", [False, True])
@pytest.mark.parametrize("opB,mode", CASES)
def test_224_row_tiles_bitwise_vs_128_tiles_and_oracle(opB, mode, pow2):
    """Random operands on the 224x256 tiles (5 K groups: an odd last group):
    bitwise equal to the same rows computed on 128x128 tiles, FP32 and BF16
    output, and within the oracle gate."""
    M, N, K = 6994, 2008, 640
    qA, sA, qB, sB = _operands(M, N, K, opB, mode, pow2, 31 + opB + 2 * mode)
    print(f"[tiles] 224x256 {M}x{N}x{K} opB={opB} mode={mode} pow2={pow2}", flush=True)
    C = _gemm(qA, sA, qB, sB, opB, mode, pow2)
    Cs = _by_row_slices(qA, sA, qB, sB, opB, mode, pow2, 1792)
    assert np.array_equal(_bits(C), _bits(Cs))
    Cb = _gemm(qA, sA, qB, sB, opB, mode, pow2, torch.bfloat16)
    Cbs = _by_row_slices(qA, sA, qB, sB, opB, mode, pow2, 1792, torch.bfloat16)
    assert np.array_equal(_bits(Cb), _bits(Cbs))
    assert np.array_equal(_bits(Cb), _bits(C.to(torch.bfloat16)))
    R = oracle.gemm_blockscaled(qA, sA, qB, sB, opB, mode)
    en = e_norm(C.numpy(), R)
    print(f"[tiles] E_norm={en:.3e}", flush=True)
    assert en <= 1e-3


@pytest.mark.parametrize("pow2", [False, True])
@pytest.mark.parametrize("opB,mode", CASES)
def test_256_row_tiles_bitwise_vs_128_tiles(opB, mode, pow2):
    """The same cross-check on the 256x256 tiles."""
    M, N, K = 4000, 4000, 384
    qA, sA, qB, sB = _operands(M, N, K, opB, mode, pow2, 41 + opB + 2 * mode)
    print(f"[tiles] 256x256 {M}x{N}x{K} opB={opB} mode={mode} pow2={pow2}", flush=True)
    C = _gemm(qA, sA, qB, sB, opB, mode, pow2)
    Cs = _by_row_slices(qA, sA, qB, sB, opB, mode, pow2, 1000)
    assert np.array_equal(_bits(C), _bits(Cs))
