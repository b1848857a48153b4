"""GPU checks of the BF16-output epilogue (FP8BLK_GEMM_OUT_BF16): every BF16
output is the kernel's own FP32 result rounded to nearest even — compared
bit for bit with torch's float32 -> bfloat16 conversion (round to nearest
even) of the FP32 output of the same call without the flag — and the BF16
result stays within the FP32 gate plus the BF16 rounding (2^-8 relative) of
the oracle.  Dense (including a split-K shape and ragged edges), grouped
and grouped Wgrad.
"""
import numpy as np
import pytest
import torch

import fp8_fine_grained_quantize_amd as fb
import oracle
import synthetic
from synthetic import bf16_bits
from tests.gpu_util import e_norm, f32_dev, np_f32, np_u8, quantized_operands, u8_dev

pytestmark = pytest.mark.gpu

TOL = 1e-3 + 2.0 ** -8   # BF16 keeps 8 significant bits: rounding is within 2^-8 relative


def _bf16_np(t):
    return t.float().cpu().numpy().astype(np.float64)


@pytest.mark.parametrize("M,N,K,opB,mode,pow2", [
    (300, 200, 384, oracle.OP_N, oracle.BSCALE_BLOCK128, False),
    (257, 136, 256, oracle.OP_T, oracle.BSCALE_BLOCK128, True),
    (200, 264, 512, oracle.OP_T, oracle.BSCALE_ROW128, False),
    (1024, 1024, 4096, oracle.OP_N, oracle.BSCALE_BLOCK128, False),   # split-K: BF16 from the reduction
    (4096, 4096, 1024, oracle.OP_N, oracle.BSCALE_BLOCK128, False),   # 256x256 tiles
    (4096, 4096, 1024, oracle.OP_N, oracle.BSCALE_BLOCK128, True),
])
def test_dense_bf16_out(M, N, K, opB, mode, pow2):
    print(f"[bf16-out] dense {M}x{N}x{K} opB={opB} mode={mode} pow2={pow2}", flush=True)
    g = torch.Generator().manual_seed(M + N + K)
    A = synthetic.randn_bf16((M, K), 1.0, g, outlier_cols=2, outlier_factor=30.0)
    Bsh = (K, N) if opB == oracle.OP_N else (N, K)
    B = synthetic.randn_bf16(Bsh, 0.02, g)
    row128 = mode == oracle.BSCALE_ROW128
    if pow2:
        qA, sA = oracle.quantize_1x128(bf16_bits(A), True)
        qB, sB = oracle.quantize_block128(bf16_bits(B), True)
    else:
        qA, sA, qB, sB = quantized_operands(bf16_bits(A), bf16_bits(B), opB, row128)
    args = (u8_dev(qA), f32_dev(sA), u8_dev(qB), f32_dev(sB))
    C32 = fb.gemm_fp8_blockscaled(*args, opB=opB, bscale_mode=mode, pow2_scales=pow2)
    C16 = fb.gemm_fp8_blockscaled(*args, opB=opB, bscale_mode=mode, pow2_scales=pow2, out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    assert C16.dtype == torch.bfloat16
    assert torch.equal(C16.cpu().view(torch.int16), C32.to(torch.bfloat16).cpu().view(torch.int16))
    if M * N * K <= 1024 * 1024 * 4096:
        R = oracle.gemm_blockscaled(qA, sA, qB, sB, opB, mode)
        assert e_norm(_bf16_np(C16), R) <= TOL


# FP32 results exact products dec(A) * sA (identity B) chosen to land on the
# BF16 rounding's edge cases: ties to even in both directions, just off a tie,
# FP32 subnormals (BF16 subnormals, and values rounding to zero), values
# rounding up to the largest finite BF16 and past it to infinity.
EDGE_SCALES = [1 + 2.0 ** -8, 1 + 3 * 2.0 ** -8, 1 + 2.0 ** -8 + 2.0 ** -23, 1 + 2.0 ** -8 - 2.0 ** -23,
               2.0 ** -130, 1.5 * 2.0 ** -133, 2.0 ** -149 * 3, 3.3895e38 / 448, 3.3961e38 / 448, 3.4e38 / 448,
               1.0, 2.0 ** -126]


@pytest.mark.parametrize("M,K", [(64, 128), (4096, 4096), (1024, 1024)])
def test_bf16_epilogue_rounding_edges(M, K):
    """Identity B (E4M3 1.0, unit scale): the FP32 output is the exact
    product dec(A[m][k]) * sA[m] rounded once, so the BF16 outputs (256x256
    tiles at 4096 x 4096, the split-K reduction at 1024 x 1024, a single
    128x128 tile at 64 rows) meet every rounding edge case; each must equal
    torch's conversion of the FP32 output bit for bit, and the fused 1x128
    quantization must equal quantize_1x128 of that BF16 matrix."""
    rng = np.random.default_rng(M + K)
    qA = rng.integers(0x01, 0x7F, size=(M, K)).astype(np.uint8) | (rng.integers(0, 2, (M, K)) << 7).astype(np.uint8)
    qA[:, :8] = 0x38  # 1.0: the scale itself
    qA[:, 8:12] = 0xB8  # -1.0
    qA[:, 12:16] = 0x7E  # 448
    sA = np.array([EDGE_SCALES[m % len(EDGE_SCALES)] for m in range(M)], np.float32)
    sA = np.tile(sA, (K // 128, 1))
    qB = np.zeros((K, K), np.uint8)
    qB[np.arange(K), np.arange(K)] = 0x38
    sB = np.ones((K // 128, K // 128), np.float32)
    print(f"[bf16-out] rounding edges {M}x{K}x{K}", flush=True)
    args = (u8_dev(qA), f32_dev(sA), u8_dev(qB), f32_dev(sB))
    C32 = fb.gemm_fp8_blockscaled(*args)
    C16 = fb.gemm_fp8_blockscaled(*args, out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    want = C32.to(torch.bfloat16)
    assert torch.equal(C16.view(torch.int16), want.view(torch.int16))
    assert torch.isinf(want.float()).any() and (want.float().abs() < 2.0 ** -126).logical_and(want != 0).any()
    # quantize-on-store never splits K: compare with the one-pass FP32 result
    # (split partials can turn an underflowed -0 into +0, and the quantizer
    # keeps the sign of zero)
    want1 = fb.gemm_fp8_blockscaled(*args, split_k=False).to(torch.bfloat16)
    for pow2 in (False, True):
        Q, sQ = fb.gemm_fp8_blockscaled_q1x128(*args, pow2=pow2)
        q2, s2 = fb.quantize_1x128(want1, pow2=pow2)
        torch.cuda.synchronize()
        finite = torch.isfinite(want1.float()).all(dim=1).cpu().numpy()
        assert np.array_equal(np_u8(Q)[finite], np_u8(q2)[finite])
        assert np.array_equal(np_f32(sQ)[:, finite].view(np.uint32), np_f32(s2)[:, finite].view(np.uint32))


@pytest.mark.parametrize("opB", [oracle.OP_N, oracle.OP_T])
def test_grouped_bf16_out(opB):
    counts = [3, 0, 130, 257, 64]
    off = np.concatenate([[0], np.cumsum(counts)]).astype(np.int64)
    Mt, K, N = int(off[-1]), 256, 200
    g = torch.Generator().manual_seed(90 + opB)
    qA, sA = oracle.quantize_1x128(bf16_bits(synthetic.randn_bf16((Mt, K), 1.0, g)))
    Bs, sBs = [], []
    for e in range(len(counts)):
        qB, sB = oracle.quantize_block128(bf16_bits(synthetic.randn_bf16((K, N) if opB == oracle.OP_N else (N, K),
                                                                         0.02, g)))
        Bs.append(qB)
        sBs.append(sB)
    B, sB = np.stack(Bs), np.stack(sBs)
    offs = torch.from_numpy(off.astype(np.int32)).cuda()
    args = (offs, u8_dev(qA), f32_dev(sA), u8_dev(B), f32_dev(sB))
    C32 = fb.grouped_gemm_fp8_blockscaled(*args, opB=opB)
    C16 = fb.grouped_gemm_fp8_blockscaled(*args, opB=opB, out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    assert torch.equal(C16.cpu().view(torch.int16), C32.to(torch.bfloat16).cpu().view(torch.int16))
    R = oracle.grouped_gemm_blockscaled(off, qA, sA, B, sB, opB)
    assert e_norm(_bf16_np(C16), R) <= TOL


@pytest.mark.parametrize("pow2", [False, True])
def test_grouped_wgrad_bf16_out(pow2):
    counts = [1, 0, 129, 300]
    off = np.concatenate([[0], np.cumsum(counts)]).astype(np.int64)
    offs = torch.from_numpy(off.astype(np.int32)).cuda()
    T, M, N = int(off[-1]), 256, 136
    g = torch.Generator().manual_seed(95)
    X = synthetic.randn_bf16((T, M), 1.0, g)
    dY = synthetic.randn_bf16((T, N), 1e-3, g)
    AT, sA = fb.quantize_128x1_grouped(X.cuda(), offs, pow2=pow2)
    BT, sB = fb.quantize_128x1_grouped(dY.cuda(), offs, pow2=pow2)
    W32 = fb.grouped_wgrad_fp8_blockscaled(offs, T, AT, sA, BT, sB, pow2_scales=pow2)
    W16 = fb.grouped_wgrad_fp8_blockscaled(offs, T, AT, sA, BT, sB, pow2_scales=pow2, out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    assert torch.equal(W16.cpu().view(torch.int16), W32.to(torch.bfloat16).cpu().view(torch.int16))
    rA, rsA = oracle.quantize_128x1_grouped(bf16_bits(X), off, pow2)
    rB, rsB = oracle.quantize_128x1_grouped(bf16_bits(dY), off, pow2)
    R = oracle.grouped_wgrad_blockscaled(off, rA, rsA, rB, rsB)
    for e in range(len(counts)):
        if counts[e]:
            assert e_norm(_bf16_np(W16[e]), R[e]) <= TOL
        else:
            assert not W16[e].float().any()
