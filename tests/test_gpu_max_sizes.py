"""Index range: every kernel family on operands past 2^31 elements (so any
32-bit element or byte offset would wrap), checked on samples against the
oracle.

* 1x128: A [32800][65960] BF16 (2.16e9 elements, a 40-column tail group); whole rows at both ends
  and in the middle (codes and scales bit for bit; the tiles of a row do not
  depend on other rows).
* 128x1: X [65581][32800] (ragged token tail); whole channels (a channel's
  tiles depend on that channel only), transposed codes and scales bit for bit.
* 128x128: W [32800][65600]; whole blocks at the corners and inside.
* GEMM: C [65666][32848] FP32 and BF16 (2.16e9 outputs) from K = 256 random
  codes and scales; sampled entries against the oracle's exact sums (E_norm
  <= 1e-3; BF16 adds its own rounding of 2^-8).

Inputs come from the seeded device generators in `synthetic`; roughly 20 GB
of GPU memory at most, released after each test.
"""
import numpy as np
import pytest
import torch

import fp8_fine_grained_quantize_amd as fb
import oracle
import synthetic
from synthetic import bf16_bits
from tests.gpu_util import np_f32, np_u8

pytestmark = pytest.mark.gpu


def _free():
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


def test_1x128_rows_past_2g_elements():
    M, K = 32800, 65960
    assert M * K > 2 ** 31
    print(f"[max] quantize_1x128 [{M}][{K}]", flush=True)
    x = synthetic.large_bf16((M, K), 11)
    q, s = fb.quantize_1x128(x)
    torch.cuda.synchronize()
    for r in [0, 1, 96 * 97, M // 2, M - 2, M - 1]:
        qo, so = oracle.quantize_1x128(bf16_bits(x[r:r + 1].cpu()))
        assert np.array_equal(np_u8(q[r:r + 1]), qo), r
        assert np.array_equal(np_f32(s[:, r:r + 1]).view(np.uint32), so.view(np.uint32)), r
    del x, q, s
    _free()


def test_128x1_channels_past_2g_elements():
    T, C = 65581, 32800
    assert T * C > 2 ** 31
    print(f"[max] quantize_128x1 [{T}][{C}]", flush=True)
    x = synthetic.large_bf16((T, C), 12)
    qT, s = fb.quantize_128x1(x)
    torch.cuda.synchronize()
    for c in [0, 5, C // 2 + 3, C - 2, C - 1]:
        qo, so = oracle.quantize_128x1(bf16_bits(x[:, c:c + 1].cpu()))
        assert np.array_equal(np_u8(qT[c:c + 1]), qo), c
        assert np.array_equal(np_f32(s[:, c:c + 1]).view(np.uint32), so.view(np.uint32)), c
    del x, qT, s
    _free()


def test_block128_past_2g_elements():
    R, C = 32800, 65600
    assert R * C > 2 ** 31
    print(f"[max] quantize_block128 [{R}][{C}]", flush=True)
    x = synthetic.large_bf16((R, C), 13)
    q, s = fb.quantize_block128(x)
    torch.cuda.synchronize()
    GR, GC = -(-R // 128), -(-C // 128)
    for bi, bj in [(0, 0), (0, GC - 1), (GR - 1, 0), (GR - 1, GC - 1), (GR // 2, GC // 3)]:
        rs, cs = slice(128 * bi, min(R, 128 * bi + 128)), slice(128 * bj, min(C, 128 * bj + 128))
        qo, so = oracle.quantize_block128(bf16_bits(x[rs, cs].cpu()))
        assert np.array_equal(np_u8(q[rs, cs]), qo), (bi, bj)
        assert np_f32(s[bi, bj]).view(np.uint32) == so[0, 0].view(np.uint32), (bi, bj)
    del x, q, s
    _free()


@pytest.mark.parametrize("pow2", [False, True])
def test_block128_large_ragged_pitched(pow2):
    """quantize_block128 on 6241 blocks: ragged
    row and column edges (10013 columns: the last block's rows end 1-7
    elements into a 16-byte chunk), a pitched view, outlier columns, both
    scale modes; every code and scale against the oracle."""
    R, C = 10000, 10013
    assert (-(-R // 128)) * (-(-C // 128)) == 6241 and C % 8 != 0
    print(f"[max] quantize_block128 large ragged pitched [{R}][{C}] pow2={pow2}", flush=True)
    g = torch.Generator().manual_seed(31)
    x_cpu = synthetic.randn_bf16((R, C), 1.0, g, outlier_cols=3, outlier_factor=60.0)
    x = fb.as_pitched(x_cpu.cuda())
    q, s = fb.quantize_block128(x, pow2=pow2)
    torch.cuda.synchronize()
    qo, so = oracle.quantize_block128(bf16_bits(x_cpu), pow2=pow2)
    assert np.array_equal(np_u8(q), qo)
    assert np.array_equal(np_f32(s).view(np.uint32), so.view(np.uint32))
    del x, q, s
    _free()


def test_block128_stacked_expert_weights():
    """The 256 down-projection weights of the MoE workload quantized in one
    launch on their stacked [256*2048][7168] tensor (57344 blocks) equal each expert's own quantization: 2048 is a multiple
    of 128, so the block grids coincide and the stacked scales are the
    per-expert tables back to back.  Checked against the oracle on four
    experts (first, last, two others)."""
    G, K, N = 256, 2048, 7168
    W = torch.empty(G * K, N, dtype=torch.bfloat16, device="cuda")
    for e in range(G):
        W[e * K:(e + 1) * K] = synthetic.expert_weight("down", e, device="cuda")
    print(f"[max] quantize_block128 stacked expert weights [{G * K}][{N}]", flush=True)
    q, s = fb.quantize_block128(W)
    torch.cuda.synchronize()
    for e in (0, 97, 200, G - 1):
        qo, so = oracle.quantize_block128(bf16_bits(W[e * K:(e + 1) * K].cpu()))
        assert np.array_equal(np_u8(q[e * K:(e + 1) * K]), qo), e
        assert np.array_equal(np_f32(s[e * (K // 128):(e + 1) * (K // 128)]).view(np.uint32), so.view(np.uint32)), e
    del W, q, s
    _free()


@pytest.mark.parametrize("out", ["fp32", "bf16"])
def test_gemm_output_past_2g_elements(out):
    M, N, K = 65666, 32848, 256
    assert M * N > 2 ** 31
    print(f"[max] gemm {M}x{N}x{K} out={out}", flush=True)
    A = synthetic.random_codes((M, K), 21)
    B = synthetic.random_codes((K, N), 22)
    sA = synthetic.random_scales((K // 128, M), 23)
    sB = synthetic.random_scales((K // 128, -(-N // 128)), 24)
    C = fb.gemm_fp8_blockscaled(A, sA, B, sB, out_dtype=torch.bfloat16 if out == "bf16" else torch.float32)
    torch.cuda.synchronize()
    rng = np.random.default_rng(5)
    rows = np.concatenate([[0, M - 1, M - 1, 0], rng.integers(0, M, 60)])
    cols = np.concatenate([[0, N - 1, 0, N - 1], rng.integers(0, N, 60)])
    R = oracle.gemm_blockscaled_entries(np_u8(A), np_f32(sA), np_u8(B), np_f32(sB), rows, cols)
    got = C[torch.from_numpy(rows).cuda(), torch.from_numpy(cols).cuda()].float().cpu().numpy().astype(np.float64)
    tol = 1e-3 + (2.0 ** -8 if out == "bf16" else 0.0)
    assert np.max(np.abs(got - R)) / np.max(np.abs(R)) <= tol
    del A, B, sA, sB, C
    _free()
