"""GPU parity of the block-scaled FP8 GEMM (dense) against the oracle.

Gate: E_norm = max|C - R| / max|R| <= 1e-3 with R the oracle's exact-partial
FP64 result.  A second, element-wise check bounds |C - R| by the measured
error model of the gfx950 FP8 matrix-core instruction (see
gpu_util.mfma_error_bound).  Exact special cases are compared bitwise:
small-integer codes with power-of-two scales (no rounding anywhere), an
identity B (C = fl32(dec(A) * sA)), and power-of-two rescaling of sA.
"""
import numpy as np
import pytest
import torch

import fp8_fine_grained_quantize_amd as fb
import oracle
import synthetic
from synthetic import bf16_bits
from tests.gpu_util import e_norm, f32_dev, mfma_error_bound, np_f32, quantized_operands, u8_dev

pytestmark = pytest.mark.gpu

CASES = [(oracle.OP_N, oracle.BSCALE_BLOCK128), (oracle.OP_T, oracle.BSCALE_BLOCK128),
         (oracle.OP_N, oracle.BSCALE_ROW128), (oracle.OP_T, oracle.BSCALE_ROW128)]


def _run(qA, sA, qB, sB, opB, mode):
    C = fb.gemm_fp8_blockscaled(u8_dev(qA), f32_dev(sA), u8_dev(qB), f32_dev(sB), opB=opB, bscale_mode=mode)
    torch.cuda.synchronize()
    return np_f32(C)


def _scale_products(sA, sB, N, opB, mode):
    G, M = sA.shape
    S = np.empty((G, M, N))
    for g in range(G):
        sb = oracle.fp8_oracle._b_scale_for_group(sB, g, N, opB, mode)
        S[g] = sA[g].astype(np.float64)[:, None] * sb[None, :]
    return S


@pytest.mark.parametrize("opB,mode", CASES)
@pytest.mark.parametrize("M,N,K", [(300, 200, 384), (128, 128, 128), (17, 257, 256), (520, 384, 640)])
def test_ragged_multi_tile(M, N, K, opB, mode):
    print(f"[gemm] M={M} N={N} K={K} opB={opB} mode={mode}", flush=True)
    g = torch.Generator().manual_seed(M + N + K)
    A = synthetic.randn_bf16((M, K), 1.0, g, outlier_cols=3, outlier_factor=30.0)
    Bshape = (K, N) if opB == oracle.OP_N else (N, K)
    B = synthetic.randn_bf16(Bshape, 0.02, g)
    qA, sA, qB, sB = quantized_operands(bf16_bits(A), bf16_bits(B), opB, mode == oracle.BSCALE_ROW128)
    C = _run(qA, sA, qB, sB, opB, mode)
    R = oracle.gemm_blockscaled(qA, sA, qB, sB, opB, mode)
    assert e_norm(C, R) <= 1e-3
    Ad = oracle.e4m3_decode(qA)
    Bd = oracle.e4m3_decode(qB if opB == oracle.OP_N else qB.T)
    bound = mfma_error_bound(Ad, Bd, _scale_products(sA, sB, N, opB, mode))
    over = np.abs(C.astype(np.float64) - R) - bound
    assert np.all(over <= 0), f"{np.sum(over > 0)} entries beyond the error model"


def test_single_gemm_full():
    A, B = synthetic.single_gemm()
    qA, sA, qB, sB = quantized_operands(bf16_bits(A), bf16_bits(B))
    C = _run(qA, sA, qB, sB, oracle.OP_N, oracle.BSCALE_BLOCK128)
    R = oracle.gemm_blockscaled(qA, sA, qB, sB)
    en = e_norm(C, R)
    print(f"[gemm] single 256x512x1024 E_norm={en:.3e}", flush=True)
    assert en <= 1e-3


def _small_int_codes(rng, shape):
    vals = np.array([0x00, 0x38, 0x40, 0x48, 0xB8, 0xC0, 0xC8], np.uint8)  # 0, +-1, +-2, +-4
    return vals[rng.integers(0, vals.size, size=shape)]


@pytest.mark.parametrize("opB,mode", CASES)
def test_exact_small_integers_bitwise(opB, mode):
    rng = np.random.default_rng(11)
    M, N, K = 256, 384, 512
    G = K // 128
    qA = _small_int_codes(rng, (M, K))
    qB = _small_int_codes(rng, (K, N) if opB == oracle.OP_N else (N, K))
    sA = np.exp2(rng.integers(-3, 4, size=(G, M))).astype(np.float32)
    if mode == oracle.BSCALE_ROW128:
        sB = np.exp2(rng.integers(-3, 4, size=(G, N))).astype(np.float32)
    else:
        shape = (G, 3) if opB == oracle.OP_N else (3, G)
        sB = np.exp2(rng.integers(-3, 4, size=shape)).astype(np.float32)
    C = _run(qA, sA, qB, sB, opB, mode)
    R = oracle.gemm_blockscaled(qA, sA, qB, sB, opB, mode)
    assert np.array_equal(C.astype(np.float64), R)


@pytest.mark.parametrize("pow2", [False, True])
@pytest.mark.parametrize("opB,mode", CASES)
def test_exact_small_integers_bitwise_256x256_tiles(opB, mode, pow2):
    """The same exact case on a shape whose big tiles fill the GPU (the
    row-pipelined loop; at 4100 x 2050 on 256 CUs the 224 x 256 tiles, the
    256 x 256 ones are covered in test_gpu_gemm_tiles.py), fold and
    power-of-two paths, with ragged edges."""
    rng = np.random.default_rng(13)
    M, N, K = 4100, 2050, 384
    G = K // 128
    qA = _small_int_codes(rng, (M, K))
    qB = _small_int_codes(rng, (K, N) if opB == oracle.OP_N else (N, K))
    sA = np.exp2(rng.integers(-3, 4, size=(G, M))).astype(np.float32)
    NB = -(-N // 128)
    if mode == oracle.BSCALE_ROW128:
        sB = np.exp2(rng.integers(-3, 4, size=(G, N))).astype(np.float32)
    else:
        sB = np.exp2(rng.integers(-3, 4, size=(G, NB) if opB == oracle.OP_N else (NB, G))).astype(np.float32)
    print(f"[gemm] exact 256x256 tiles {M}x{N}x{K} opB={opB} mode={mode} pow2={pow2}", flush=True)
    C = fb.gemm_fp8_blockscaled(u8_dev(qA), f32_dev(sA), u8_dev(qB), f32_dev(sB), opB=opB, bscale_mode=mode,
                                pow2_scales=pow2)
    torch.cuda.synchronize()
    R = oracle.gemm_blockscaled(qA, sA, qB, sB, opB, mode)
    assert np.array_equal(np_f32(C).astype(np.float64), R)


def test_identity_b_bitwise():
    rng = np.random.default_rng(12)
    M, K = 200, 384
    qA = rng.integers(0, 0x7F, size=(M, K)).astype(np.uint8) | (rng.integers(0, 2, (M, K)) << 7).astype(np.uint8)
    sA = (rng.uniform(1, 2, (K // 128, M)) * np.exp2(rng.integers(-20, 5, (K // 128, M)))).astype(np.float32)
    qB = np.zeros((K, K), np.uint8)
    qB[np.arange(K), np.arange(K)] = 0x38
    sB = np.ones((K // 128, K // 128), np.float32)
    C = _run(qA, sA, qB, sB, oracle.OP_N, oracle.BSCALE_BLOCK128)
    want = oracle.dequantize_1x128(qA, sA).astype(np.float32)  # one rounding of an exact product
    # equal as numbers: a zero code gives -0.0 in the oracle and +0.0 from the
    # matrix cores (the sign of an exact zero sum is not part of the result)
    assert np.array_equal(C, want)
    # the same through the transposed-B path
    C2 = _run(qA, sA, np.ascontiguousarray(qB.T), sB, oracle.OP_T, oracle.BSCALE_BLOCK128)
    assert np.array_equal(C2, want)


def test_pow2_rescaling_and_determinism():
    g = torch.Generator().manual_seed(13)
    A = synthetic.randn_bf16((384, 512), 1.0, g)
    B = synthetic.randn_bf16((512, 256), 0.02, g)
    qA, sA, qB, sB = quantized_operands(bf16_bits(A), bf16_bits(B))
    C1 = _run(qA, sA, qB, sB, oracle.OP_N, oracle.BSCALE_BLOCK128)
    C2 = _run(qA, sA, qB, sB, oracle.OP_N, oracle.BSCALE_BLOCK128)
    assert np.array_equal(C1.view(np.uint32), C2.view(np.uint32))
    C3 = _run(qA, (sA * np.float32(2.0 ** 7)).astype(np.float32), qB, sB, oracle.OP_N, oracle.BSCALE_BLOCK128)
    assert np.array_equal(C3, (C1 * np.float32(2.0 ** 7)).astype(np.float32))


@pytest.mark.parametrize("opB,mode", CASES)
@pytest.mark.parametrize("M,N,K", [(256, 256, 2048), (300, 200, 3072), (64, 1000, 4096), (300, 202, 2048)])
def test_split_k(M, N, K, opB, mode):
    """Shapes with too few tiles to fill the GPU split K over a workspace:
    the result still meets the oracle gate, stays within a few FP32 ulps of
    the one-pass result (S-1 extra additions), and is deterministic."""
    assert fb.workspace_bytes(M, N, K, 1) > 0
    g = torch.Generator().manual_seed(M + N + K)
    A = synthetic.randn_bf16((M, K), 1.0, g)
    if opB == oracle.OP_N:
        B = synthetic.randn_bf16((K, N), 0.02, g)
        qA, sA = oracle.quantize_1x128(bf16_bits(A))
        if mode == oracle.BSCALE_BLOCK128:
            qB, sB = oracle.quantize_block128(bf16_bits(B))
        else:  # 128-deep tiles along K per column: 128x1 of B [K][N], codes back in [K][N]
            qBT, sB = oracle.quantize_128x1(bf16_bits(B))
            qB = np.ascontiguousarray(qBT.T)
    else:
        B = synthetic.randn_bf16((N, K), 0.02, g)
        qA, sA = oracle.quantize_1x128(bf16_bits(A))
        qB, sB = (oracle.quantize_block128(bf16_bits(B)) if mode == oracle.BSCALE_BLOCK128 else
                  oracle.quantize_1x128(bf16_bits(B)))
    dev = [u8_dev(qA), f32_dev(sA), u8_dev(qB), f32_dev(sB)]
    print(f"[gemm] split-K {M}x{N}x{K} opB={opB} mode={mode}", flush=True)
    C1 = np_f32(fb.gemm_fp8_blockscaled(*dev, opB=opB, bscale_mode=mode, split_k=False))
    Cs = np_f32(fb.gemm_fp8_blockscaled(*dev, opB=opB, bscale_mode=mode))
    Cs2 = np_f32(fb.gemm_fp8_blockscaled(*dev, opB=opB, bscale_mode=mode))
    torch.cuda.synchronize()
    R = oracle.gemm_blockscaled(qA, sA, qB, sB, opB, mode)
    assert e_norm(Cs, R) <= 1e-3
    assert np.array_equal(Cs.view(np.uint32), Cs2.view(np.uint32))
    assert float(np.max(np.abs(Cs.astype(np.float64) - C1)) / np.max(np.abs(R))) <= 1e-5


def _sampled(C, qA, sA, qB, sB, opB, mode, n=4096, seed=0):
    rng = np.random.default_rng(seed)
    M, N = C.shape
    rows = rng.integers(0, M, n)
    cols = rng.integers(0, N, n)
    rows[:4] = [0, M - 1, 0, M - 1]
    cols[:4] = [0, N - 1, N - 1, 0]
    R = oracle.gemm_blockscaled_entries(qA, sA, qB, sB, rows, cols, opB, mode)
    got = C[rows, cols].astype(np.float64)
    return float(np.max(np.abs(got - R)) / np.max(np.abs(R)))


def test_dense_fprop_full_size_sampled():
    A, W = synthetic.dense_fprop()
    for pow2 in (False, True):
        qA, sA = oracle.quantize_1x128(bf16_bits(A), pow2)
        qB, sB = oracle.quantize_block128(bf16_bits(W))
        print(f"[gemm] dense fprop 4096x4096x7168 pow2={pow2}", flush=True)
        C = _run(qA, sA, qB, sB, oracle.OP_N, oracle.BSCALE_BLOCK128)
        en = _sampled(C, qA, sA, qB, sB, oracle.OP_N, oracle.BSCALE_BLOCK128)
        print(f"[gemm] sampled E_norm={en:.3e}", flush=True)
        assert en <= 1e-3
        assert np.all(np.isfinite(C))


@pytest.mark.parametrize("K", [4096, 8192, 16384])
def test_accumulation_study_full(K):
    A, B = synthetic.accum_study(K)
    qA, sA, qB, sB = quantized_operands(bf16_bits(A), bf16_bits(B))
    print(f"[gemm] accumulation study 1024x1024x{K}", flush=True)
    C = _run(qA, sA, qB, sB, oracle.OP_N, oracle.BSCALE_BLOCK128)
    R = oracle.gemm_blockscaled(qA, sA, qB, sB)
    U = oracle.gemm_unquantized(bf16_bits(A), bf16_bits(B))
    en = e_norm(C, R)
    eu = e_norm(C, U)
    # componentwise: |C - R| against |A_hat| |B_hat| (the dequantized operands'
    # magnitudes), and the median element-wise relative error
    mag = np.abs(oracle.dequantize_1x128(qA, sA)) @ np.abs(oracle.dequantize_block128(qB, sB))
    d = np.abs(C.astype(np.float64) - R)
    e_comp = float(np.max(d / mag))
    nz = R != 0
    med = float(np.median(d[nz] / np.abs(R[nz])))
    print(f"[gemm] K={K}: E_norm vs oracle {en:.3e}; E_comp {e_comp:.3e}; median element-wise {med:.3e}; "
          f"vs unquantized FP64 {eu:.3e}", flush=True)
    assert en <= 1e-3
    assert eu < 0.1
    # the matrix-core model (products truncated to 2^-13 of their block of 8's
    # maximum) bounds E_comp by 8 * 2^-13 plus the FP32 roundings of the fold
    assert e_comp <= 8 * 2.0 ** -13 + (K // 128 + 2) * 2.0 ** -23


def test_backward_full_size_sampled():
    X, W, dY = synthetic.backward()
    # Dgrad: dX[4096][7168] = dY[4096][2048] . W^T, W stored [7168][2048] read as OP_T
    qA, sA = oracle.quantize_1x128(bf16_bits(dY))
    qW, sW = oracle.quantize_block128(bf16_bits(W))
    print("[gemm] dgrad 4096x7168x2048", flush=True)
    C = _run(qA, sA, qW, sW, oracle.OP_T, oracle.BSCALE_BLOCK128)
    assert _sampled(C, qA, sA, qW, sW, oracle.OP_T, oracle.BSCALE_BLOCK128) <= 1e-3
    # Wgrad: dW[7168][2048] = X^T . dY, both quantized 128x1 along tokens
    qX, sX = oracle.quantize_128x1(bf16_bits(X))     # [7168][4096], [32][7168]
    qD, sD = oracle.quantize_128x1(bf16_bits(dY))    # [2048][4096], [32][2048]
    print("[gemm] wgrad 7168x2048x4096", flush=True)
    C = _run(qX, sX, qD, sD, oracle.OP_T, oracle.BSCALE_ROW128)
    assert _sampled(C, qX, sX, qD, sD, oracle.OP_T, oracle.BSCALE_ROW128) <= 1e-3


def test_empty_is_noop():
    A = torch.empty(0, 256, dtype=torch.uint8, device="cuda")
    B = torch.empty(256, 128, dtype=torch.uint8, device="cuda")
    C = fb.gemm_fp8_blockscaled(A, torch.empty(2, 0, device="cuda"), B, torch.ones(2, 1, device="cuda"))
    torch.cuda.synchronize()
    assert C.shape == (0, 128)


def _pow2_operands(M, N, K, opB, mode, seed):
    """Both operands quantized with power-of-two scales, in the layouts the
    four GEMM modes take."""
    g = torch.Generator().manual_seed(seed)
    A = synthetic.randn_bf16((M, K), 1.0, g)
    qA, sA = oracle.quantize_1x128(bf16_bits(A), True)
    if opB == oracle.OP_N:
        B = synthetic.randn_bf16((K, N), 0.02, g)
        if mode == oracle.BSCALE_BLOCK128:
            qB, sB = oracle.quantize_block128(bf16_bits(B), True)
        else:
            qBT, sB = oracle.quantize_128x1(bf16_bits(B), True)
            qB = np.ascontiguousarray(qBT.T)
    else:
        B = synthetic.randn_bf16((N, K), 0.02, g)
        qB, sB = (oracle.quantize_block128(bf16_bits(B), True) if mode == oracle.BSCALE_BLOCK128 else
                  oracle.quantize_1x128(bf16_bits(B), True))
    return qA, sA, qB, sB


@pytest.mark.parametrize("opB,mode", CASES)
@pytest.mark.parametrize("M,N,K", [(300, 200, 384), (520, 384, 640), (256, 256, 2048)])
def test_pow2_scales_in_matrix_cores(M, N, K, opB, mode):
    """GEMM_POW2_SCALES: scales applied as E8M0 block scales by the MFMA and
    groups accumulated in its FP32 accumulator.  Same gate against the
    oracle; within FP32 rounding of the separate-fold path."""
    qA, sA, qB, sB = _pow2_operands(M, N, K, opB, mode, M * 7 + K)
    dev = [u8_dev(qA), f32_dev(sA), u8_dev(qB), f32_dev(sB)]
    print(f"[gemm] pow2 scales in MFMA {M}x{N}x{K} opB={opB} mode={mode}", flush=True)
    Cp = np_f32(fb.gemm_fp8_blockscaled(*dev, opB=opB, bscale_mode=mode, pow2_scales=True))
    Cf = np_f32(fb.gemm_fp8_blockscaled(*dev, opB=opB, bscale_mode=mode))
    torch.cuda.synchronize()
    R = oracle.gemm_blockscaled(qA, sA, qB, sB, opB, mode)
    assert e_norm(Cp, R) <= 1e-3
    assert float(np.max(np.abs(Cp.astype(np.float64) - Cf)) / np.max(np.abs(R))) <= 1e-5


@pytest.mark.parametrize("opB,mode", CASES)
def test_pow2_scales_exact_small_integers(opB, mode):
    """Small-integer codes with power-of-two scales: every product and sum is
    exact, so the matrix-core scaling must reproduce the oracle exactly."""
    rng = np.random.default_rng(21)
    M, N, K = 256, 384, 512
    G = K // 128
    qA = _small_int_codes(rng, (M, K))
    qB = _small_int_codes(rng, (K, N) if opB == oracle.OP_N else (N, K))
    sA = np.exp2(rng.integers(-3, 4, size=(G, M))).astype(np.float32)
    if mode == oracle.BSCALE_ROW128:
        sB = np.exp2(rng.integers(-3, 4, size=(G, N))).astype(np.float32)
    else:
        shape = (G, 3) if opB == oracle.OP_N else (3, G)
        sB = np.exp2(rng.integers(-3, 4, size=shape)).astype(np.float32)
    C = np_f32(fb.gemm_fp8_blockscaled(u8_dev(qA), f32_dev(sA), u8_dev(qB), f32_dev(sB), opB=opB, bscale_mode=mode,
                                       pow2_scales=True))
    torch.cuda.synchronize()
    R = oracle.gemm_blockscaled(qA, sA, qB, sB, opB, mode)
    assert np.array_equal(C.astype(np.float64), R)


def test_pow2_scales_dense_fprop_full_size_sampled():
    A, W = synthetic.dense_fprop()
    qA, sA = oracle.quantize_1x128(bf16_bits(A), True)
    qB, sB = oracle.quantize_block128(bf16_bits(W), True)
    print("[gemm] dense fprop 4096x4096x7168, power-of-two scales in the MFMA", flush=True)
    C = np_f32(fb.gemm_fp8_blockscaled(u8_dev(qA), f32_dev(sA), u8_dev(qB), f32_dev(sB), pow2_scales=True))
    torch.cuda.synchronize()
    en = _sampled(C, qA, sA, qB, sB, oracle.OP_N, oracle.BSCALE_BLOCK128)
    print(f"[gemm] sampled E_norm={en:.3e}", flush=True)
    assert en <= 1e-3
    assert np.all(np.isfinite(C))
