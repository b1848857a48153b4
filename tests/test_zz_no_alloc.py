"""GPU test of the allocation-free dense GEMM entry point,
fp8blk_gemm_fp8_blockscaled_noalloc, called through the C ABI.

It must give exactly what fp8blk_gemm_fp8_blockscaled gives with a large
enough workspace (the same kernels and split choice, its split-K partials
taken from the library's per-device scratch array instead of the caller's
workspace): the outputs are compared bit for bit, and against the oracle
(E_norm <= 1e-3).  Two calls in a row, the second on a smaller shape, so the
second call reuses an array that holds the first call's partials; further
calls cover a shape that does not split, N not a multiple of 4, BF16 output
and power-of-two scales.
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


def _operands(M, N, K, seed, pow2=False):
    g = torch.Generator().manual_seed(seed)
    A = synthetic.randn_bf16((M, K), 1.0, g, outlier_cols=2, outlier_factor=30.0)
    B = synthetic.randn_bf16((K, N), 0.02, g)
    qA, sA = oracle.quantize_1x128(bf16_bits(A), pow2)
    qB, sB = oracle.quantize_block128(bf16_bits(B), pow2)
    return qA, sA, qB, sB


def _both(qA, sA, qB, sB, out_dtype=torch.float32, pow2=False):
    dA, dsA, dB, dsB = u8_dev(qA), f32_dev(sA), u8_dev(qB), f32_dev(sB)
    M, N = qA.shape[0], qB.shape[1]
    C_ws = fb.gemm_fp8_blockscaled(dA, dsA, dB, dsB, out_dtype=out_dtype, pow2_scales=pow2)
    C_na = fb.empty_pitched(M, N, out_dtype)
    fb.gemm_fp8_blockscaled_noalloc(dA, dsA, dB, dsB, C_na, pow2_scales=pow2)
    torch.cuda.synchronize()
    return C_ws, C_na


@pytest.mark.parametrize("pow2", [False, True])
def test_noalloc_equals_workspace_entry_point_two_calls(pow2):
    # first call: the accumulation-study shape (split over the scratch array)
    M, N, K = 1024, 1024, 4096
    assert fb.workspace_bytes(M, N, K) > 0
    print(f"[noalloc] {M}x{N}x{K} pow2={pow2}", flush=True)
    ops = _operands(M, N, K, 1, pow2)
    C_ws, C_na = _both(*ops, pow2=pow2)
    assert torch.equal(C_ws.view(torch.int32), C_na.view(torch.int32))
    # second call, smaller, N not a multiple of 4 (the array still holds the
    # first call's partials)
    M, N, K = 300, 202, 2048
    assert fb.workspace_bytes(M, N, K) > 0
    print(f"[noalloc] {M}x{N}x{K} pow2={pow2}", flush=True)
    qA, sA, qB, sB = _operands(M, N, K, 2, pow2)
    C_ws, C_na = _both(qA, sA, qB, sB, pow2=pow2)
    assert torch.equal(C_ws.view(torch.int32), C_na.view(torch.int32))
    R = oracle.gemm_blockscaled(qA, sA, qB, sB)
    assert e_norm(np_f32(C_na), R) <= 1e-3


def test_noalloc_bf16_output_and_unsplit_shape():
    M, N, K = 520, 384, 1024
    print(f"[noalloc] {M}x{N}x{K} bf16", flush=True)
    ops = _operands(M, N, K, 3)
    C_ws, C_na = _both(*ops, out_dtype=torch.bfloat16)
    assert torch.equal(C_ws.view(torch.int16), C_na.view(torch.int16))
    # a shape whose tiles fill the GPU: no split, no scratch
    M, N, K = 2048, 4096, 512
    assert fb.workspace_bytes(M, N, K) == 0
    print(f"[noalloc] {M}x{N}x{K} unsplit", flush=True)
    ops = _operands(M, N, K, 4)
    C_ws, C_na = _both(*ops)
    assert torch.equal(C_ws.view(torch.int32), C_na.view(torch.int32))


def test_noalloc_rejects_bad_arguments():
    A = torch.zeros(128, 128, dtype=torch.uint8, device="cuda")
    s = torch.ones(1, 128, device="cuda")
    sb = torch.ones(1, 1, device="cuda")
    C = torch.empty(128, 128, device="cuda")
    L = fb.lib()
    st = torch.cuda.current_stream().cuda_stream
    # K not a multiple of 128
    assert L.fp8blk_gemm_fp8_blockscaled_noalloc(128, 128, 100, A.data_ptr(), 128, s.data_ptr(), A.data_ptr(), 128,
                                                 0, sb.data_ptr(), 0, C.data_ptr(), 128, st) == 1
    # unknown B layout
    assert L.fp8blk_gemm_fp8_blockscaled_noalloc(128, 128, 128, A.data_ptr(), 128, s.data_ptr(), A.data_ptr(), 128,
                                                 5, sb.data_ptr(), 0, C.data_ptr(), 128, st) == 1
