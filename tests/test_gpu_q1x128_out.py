"""GPU checks of the quantize-on-store GEMM (fp8blk_gemm_fp8_blockscaled_q1x128):
its codes and scales equal, bit for bit, quantize_1x128 applied to the same
GEMM's BF16 output (two library paths, each checked against the oracle on
its own: the BF16 GEMM output to its gate, the quantizer bit for bit), over
both tile configurations, both B layouts, both scale modes of the inputs and
of the output, and ragged M and N (a partial last 128-column group).  The
dequantized output is also held against the oracle's GEMM within the BF16
and E4M3 rounding it adds.
"""
import numpy as np
import pytest
import torch

import fp8_fine_grained_quantize_amd as fb
import oracle
import synthetic
from synthetic import bf16_bits
from tests.gpu_util import f32_dev, np_f32, np_u8, u8_dev

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("M,N,K", [(300, 200, 384), (4096, 4096, 512), (257, 456, 256)])
@pytest.mark.parametrize("opB", [oracle.OP_N, oracle.OP_T])
@pytest.mark.parametrize("p2_in,p2_out", [(False, False), (False, True), (True, True)])
def test_q1x128_matches_bf16_then_quantize(M, N, K, opB, p2_in, p2_out):
    print(f"[q-out] {M}x{N}x{K} opB={opB} pow2 in={p2_in} out={p2_out}", flush=True)
    g = torch.Generator().manual_seed(M + N + K + opB)
    A = synthetic.randn_bf16((M, K), 1.0, g, outlier_cols=2, outlier_factor=30.0)
    B = synthetic.randn_bf16((K, N) if opB == oracle.OP_N else (N, K), 0.02, g)
    qA, sA = oracle.quantize_1x128(bf16_bits(A), p2_in)
    qB, sB = oracle.quantize_block128(bf16_bits(B), p2_in)
    args = (u8_dev(qA), f32_dev(sA), u8_dev(qB), f32_dev(sB))
    Q, sQ = fb.gemm_fp8_blockscaled_q1x128(*args, opB=opB, pow2_scales=p2_in, pow2=p2_out)
    Cb = fb.gemm_fp8_blockscaled(*args, opB=opB, pow2_scales=p2_in, out_dtype=torch.bfloat16, split_k=False)
    Q2, sQ2 = fb.quantize_1x128(Cb, pow2=p2_out)
    torch.cuda.synchronize()
    assert np.array_equal(np_u8(Q), np_u8(Q2))
    assert np.array_equal(np_f32(sQ).view(np.uint32), np_f32(sQ2).view(np.uint32))
    if M * N * K <= 300 * 456 * 384:
        R = oracle.gemm_blockscaled(qA, sA, qB, sB, opB)
        codes = torch.from_numpy(np_u8(Q).copy()).view(torch.float8_e4m3fn).to(torch.float64).numpy()
        deq = codes * np.repeat(np_f32(sQ).T.astype(np.float64), 128, axis=1)[:, :N]
        # BF16 rounding (2^-8), E4M3 rounding (2^-4 of the value, or half the
        # smallest spacing s * 2^-10 below the normal range) and the GEMM gate
        s_full = np.repeat(np_f32(sQ).T.astype(np.float64), 128, axis=1)[:, :N]
        bound = np.abs(R) * (2.0 ** -8 + 2.0 ** -4) + s_full * 2.0 ** -10 + 1e-3 * np.max(np.abs(R))
        assert np.all(np.abs(deq - R) <= bound)


def test_q1x128_matches_sampled_full_size():
    """The dense Fprop workload: fused output equals GEMM(BF16) -> quantize."""
    A, W = synthetic.dense_fprop()
    qA, sA = fb.quantize_1x128(A.cuda())
    qW, sW = fb.quantize_block128(W.cuda())
    for p2_out in (False, True):
        print(f"[q-out] dense fprop 4096x4096x7168 pow2 out={p2_out}", flush=True)
        Q, sQ = fb.gemm_fp8_blockscaled_q1x128(qA, sA, qW, sW, pow2=p2_out)
        Cb = fb.gemm_fp8_blockscaled(qA, sA, qW, sW, out_dtype=torch.bfloat16)
        Q2, sQ2 = fb.quantize_1x128(Cb, pow2=p2_out)
        torch.cuda.synchronize()
        assert torch.equal(Q, Q2)
        assert torch.equal(sQ.view(torch.int32), sQ2.view(torch.int32))
