"""Helpers shared by the GPU parity tests (no method arithmetic here)."""
import numpy as np
import pytest
import torch

import oracle

requires_gpu = pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")


def dev(t: torch.Tensor) -> torch.Tensor:
    """Copy to the GPU into a matrix whose rows sit at a 16-byte pitch."""
    import fp8_fine_grained_quantize_amd as fb
    return fb.as_pitched(t.to("cuda")) if t.dim() == 2 else t.to("cuda")


def np_u8(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().numpy().astype(np.uint8, copy=False)


def np_f32(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().numpy().astype(np.float32, copy=False)


def u8_dev(a: np.ndarray) -> torch.Tensor:
    """uint8 array -> GPU; 2-D and 3-D arrays get a 16-byte row pitch."""
    t = torch.from_numpy(np.ascontiguousarray(a))
    if t.dim() < 2 or t.shape[-1] % 16 == 0:
        return t.to("cuda")
    pad = -(-t.shape[-1] // 16) * 16
    out = torch.zeros(*t.shape[:-1], pad, dtype=torch.uint8, device="cuda")[..., :t.shape[-1]]
    out.copy_(t)
    return out


def f32_dev(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to("cuda")


def e_norm(C: np.ndarray, R: np.ndarray) -> float:
    """max|C - R| / max|R| (the GEMM tolerance measure)."""
    return float(np.max(np.abs(C.astype(np.float64) - R)) / max(np.max(np.abs(R)), 1e-300))


def _e4m3_exponent(v: np.ndarray) -> np.ndarray:
    """Exponent field (unbiased) of exact E4M3 values: floor(log2|v|) for
    normal values, -6 for subnormals; zero gets a very small sentinel."""
    a = np.abs(v)
    e = np.floor(np.log2(np.where(a > 0, a, 1.0)))
    return np.where(a == 0, -1000.0, np.where(a < 2.0 ** -6, -6.0, e))


def mfma_error_bound(Ad: np.ndarray, Bd: np.ndarray, S: np.ndarray, rows=None, cols=None, safety=2.0):
    """Element-wise bound on |C_gpu - C_exact| for the matrix-core partials.

    Ad [M][K], Bd [K][N] decoded (float64); S [G][M][N] scale products.
    Model (measured on gfx950, pinned in test_gpu_mfma_accumulation.py): each
    16x16x128 FP8 MFMA adds its products in blocks of 8 consecutive k; in a
    block every product is truncated toward zero to a multiple of 2^(E-13),
    E the largest sum of the operands' exponents over the block's nonzero
    products; block sums are then combined in FP32; the group result is
    folded with one FMA into an FP32 accumulator.  The bound charges each of
    a block's 8 products one quantum 2^(E-13) (times `safety`), plus FP32
    rounding of the block sums' combination, of every partial and of the
    running sum."""
    M, K = Ad.shape
    N = Bd.shape[1]
    G = K // 128
    ea = _e4m3_exponent(Ad)
    eb = _e4m3_exponent(Bd)
    bound = np.zeros((M, N))
    absC = np.zeros((M, N))
    for g in range(G):
        Sg = np.abs(S[g])
        e_g = np.zeros((M, N))
        sabs = np.zeros((M, N))
        for b in range(16):
            ks = slice(g * 128 + 8 * b, g * 128 + 8 * b + 8)
            P = np.abs(Ad[:, None, ks] * Bd.T[None, :, ks])  # [M][N][8]
            E = np.max(ea[:, None, ks] + eb.T[None, :, ks], axis=2)
            E = np.where(np.any(P > 0, axis=2), E, -1000.0)
            e_g += 8 * np.exp2(E - 13) * safety
            sabs += P.sum(axis=2)
        bound += Sg * (e_g + sabs * 2.0 ** -22)
        absC += Sg * sabs
    return bound + absC * (G + 2) * 2.0 ** -23


def quantized_operands(A_bits, B_bits, opB=oracle.OP_N, row128=False):
    """Oracle quantization of BF16 operands: A 1x128, B block128 or 128-deep
    column tiles (ROW128).  B_bits is [K][N] for OP_N, [N][K] for OP_T."""
    qA, sA = oracle.quantize_1x128(A_bits)
    if row128:
        if opB == oracle.OP_T:
            qB, sB = oracle.quantize_1x128(B_bits)      # [N][K], scales [K/128][N]
        else:
            qBT, sB = oracle.quantize_128x1(B_bits)     # B [K][N] -> codes [N][K]
            qB = np.ascontiguousarray(qBT.T)
    else:
        qB, sB = oracle.quantize_block128(B_bits)
    return qA, sA, qB, sB
