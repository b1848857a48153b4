"""GPU parity of the grouped (per-expert) block-scaled FP8 GEMM.

Small cases are compared with the oracle in full and bitwise with a loop of
dense GPU calls (same tiles, same arithmetic); the MoE-shaped case (256
experts, skewed top-8 routing over 8192 tokens) is checked on sampled
outputs of every expert.
"""
import numpy as np
import pytest
import torch

import fp8_fine_grained_quantize_amd as fb
import oracle
import synthetic
from synthetic import bf16_bits
from tests.gpu_util import e_norm, f32_dev, np_f32, np_u8, u8_dev

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("opB", [oracle.OP_N, oracle.OP_T])
@pytest.mark.parametrize("counts", [[3, 0, 130, 0, 0, 257], [0, 0, 0, 5], [128, 128, 1], [0, 0]])
def test_grouped_small(opB, counts):
    print(f"[grouped] counts={counts} opB={opB}", flush=True)
    K, N = 256, 200
    rng = np.random.default_rng(len(counts) + opB)
    off = np.concatenate([[0], np.cumsum(counts)]).astype(np.int64)
    Mt = int(off[-1])
    g = torch.Generator().manual_seed(21)
    A = synthetic.randn_bf16((max(Mt, 1), K), 1.0, g)[:Mt]
    qA, sA = oracle.quantize_1x128(bf16_bits(A)) if Mt else (np.zeros((0, K), np.uint8), np.zeros((2, 0), np.float32))
    Bs, sBs = [], []
    for e in range(len(counts)):
        Bshape = (K, N) if opB == oracle.OP_N else (N, K)
        qB, sB = oracle.quantize_block128(bf16_bits(synthetic.randn_bf16(Bshape, 0.02, g)))
        Bs.append(qB)
        sBs.append(sB)
    B = np.stack(Bs)
    sB = np.stack(sBs)
    offs = torch.from_numpy(off.astype(np.int32)).cuda()
    C = fb.grouped_gemm_fp8_blockscaled(offs, u8_dev(qA), f32_dev(sA), u8_dev(B), f32_dev(sB), opB=opB)
    torch.cuda.synchronize()
    Cg = np_f32(C)
    if Mt == 0:
        return
    # the caller's bound on any expert's rows sizes the grid from it (here
    # often the tighter bound): the same result
    Cm = fb.grouped_gemm_fp8_blockscaled(offs, u8_dev(qA), f32_dev(sA), u8_dev(B), f32_dev(sB), opB=opB,
                                         max_group_rows=max(counts))
    torch.cuda.synchronize()
    assert np.array_equal(np_f32(Cm).view(np.uint32), Cg.view(np.uint32))
    R = oracle.grouped_gemm_blockscaled(off, qA, sA, B, sB, opB)
    assert e_norm(Cg, R) <= 1e-3
    for e in range(len(counts)):
        r0, r1 = off[e], off[e + 1]
        if r1 == r0:
            continue
        Cd = fb.gemm_fp8_blockscaled(u8_dev(qA[r0:r1]), f32_dev(sA[:, r0:r1]), u8_dev(B[e]), f32_dev(sB[e]), opB=opB,
                                     split_k=False)
        torch.cuda.synchronize()
        assert np.array_equal(np_f32(Cd).view(np.uint32), Cg[r0:r1].view(np.uint32)), f"expert {e}"


@pytest.mark.parametrize("G", [63, 64, 65, 256, 257, 300])
def test_grouped_many_experts(G):
    """Expert counts around the 64-expert chunks of the kernel's tile lookup
    and past the 256 experts whose tile counts it keeps in registers (beyond
    them it walks the offsets chunk by chunk): the oracle gate over the whole
    output and bit equality with one dense call per expert."""
    print(f"[grouped] {G} experts", flush=True)
    K, N = 256, 144
    rng = np.random.default_rng(G)
    counts = rng.integers(0, 24, size=G)
    counts[rng.integers(0, G, size=3)] = [0, 300, 257]  # some empty, two spanning several row tiles
    off = np.concatenate([[0], np.cumsum(counts)]).astype(np.int64)
    Mt = int(off[-1])
    g = torch.Generator().manual_seed(G)
    A = synthetic.randn_bf16((Mt, K), 1.0, g)
    qA, sA = oracle.quantize_1x128(bf16_bits(A))
    W = synthetic.randn_bf16((G * K, N), 0.02, g)
    qW, sW = oracle.quantize_block128(bf16_bits(W))      # the experts' [K][N] weights stacked
    B = qW.reshape(G, K, N)
    sB = sW.reshape(G, K // 128, -1)
    offs = torch.from_numpy(off.astype(np.int32)).cuda()
    C = fb.grouped_gemm_fp8_blockscaled(offs, u8_dev(qA), f32_dev(sA), u8_dev(B), f32_dev(sB))
    Cm = fb.grouped_gemm_fp8_blockscaled(offs, u8_dev(qA), f32_dev(sA), u8_dev(B), f32_dev(sB),
                                         max_group_rows=int(counts.max()))
    torch.cuda.synchronize()
    Cg = np_f32(C)
    assert np.array_equal(np_f32(Cm).view(np.uint32), Cg.view(np.uint32))
    R = oracle.grouped_gemm_blockscaled(off, qA, sA, B, sB, oracle.OP_N)
    assert e_norm(Cg, R) <= 1e-3
    dA, dsA = u8_dev(qA), f32_dev(sA)
    for e in range(G):
        r0, r1 = int(off[e]), int(off[e + 1])
        if r1 == r0:
            continue
        Cd = fb.gemm_fp8_blockscaled(dA[r0:r1], dsA[:, r0:r1].contiguous(), u8_dev(B[e]), f32_dev(sB[e]),
                                     split_k=False)
        torch.cuda.synchronize()
        assert np.array_equal(np_f32(Cd).view(np.uint32), Cg[r0:r1].view(np.uint32)), f"expert {e}"


def test_moe_up_projection_sampled():
    """256 experts, top-8 of 8192 tokens, K=7168 -> N=4096, weights drawn on
    the device per expert; X quantized 1x128 with power-of-two scales before
    the row gather (the pages quantize before dispatch)."""
    r = synthetic.moe_routing()
    X, tok, off = r["X"], r["token_of_row"], r["offsets"]
    G, K, N = 256, 7168, 4096
    qX, sX = oracle.quantize_1x128(bf16_bits(X), pow2=True)
    tok_np = tok.numpy()
    qA = qX[tok_np]
    sA = np.ascontiguousarray(sX[:, tok_np])
    qB_dev = torch.empty(G, K, N, dtype=torch.uint8, device="cuda")
    sB_dev = torch.empty(G, K // 128, N // 128, dtype=torch.float32, device="cuda")
    for e in range(G):
        W = synthetic.expert_weight("up", e, device="cuda")
        fb.quantize_block128(W, q=qB_dev[e], s=sB_dev[e])
    torch.cuda.synchronize()
    offs = off.to(torch.int32).cuda()
    print("[grouped] moe up 65536x4096x7168, 256 experts", flush=True)
    C = fb.grouped_gemm_fp8_blockscaled(offs, u8_dev(qA), f32_dev(sA), qB_dev, sB_dev, opB=oracle.OP_N)
    torch.cuda.synchronize()
    rng = np.random.default_rng(1)
    off_np = off.numpy()
    worst = 0.0
    for e in rng.choice(G, 8, replace=False):
        r0, r1 = int(off_np[e]), int(off_np[e + 1])
        if r1 == r0:
            continue
        # weights: the oracle quantizes the same BF16 draw (copied bit-exact
        # from the device); the GPU-quantized weight must equal it bit for bit
        W = synthetic.expert_weight("up", int(e), device="cuda").cpu()
        qB, sB = oracle.quantize_block128(bf16_bits(W))
        assert np.array_equal(np_u8(qB_dev[e]), qB), f"expert {e} weight codes"
        assert np.array_equal(np_f32(sB_dev[e]).view(np.uint32), sB.view(np.uint32)), f"expert {e} weight scales"
        rows = rng.integers(r0, r1, 64)
        cols = rng.integers(0, N, 64)
        Rv = oracle.gemm_blockscaled_entries(qA[r0:r1], sA[:, r0:r1], qB, sB, rows - r0, cols)
        got = C[torch.from_numpy(rows).cuda(), torch.from_numpy(cols).cuda()].cpu().numpy().astype(np.float64)
        worst = max(worst, float(np.max(np.abs(got - Rv)) / np.max(np.abs(Rv))))
    print(f"[grouped] sampled E_norm={worst:.3e}", flush=True)
    assert worst <= 1e-3


def test_moe_down_projection_sampled():
    """The down projection at its full shape: 256 experts over the 65,536
    expert-ordered rows of the top-8 routing, K = 2048 -> N = 7168, the
    input H [65536][2048] quantized 1x128 (default scales) and every expert's
    W_down[e] [2048][7168] quantized 128x128 on the GPU into one stacked
    tensor, one grouped launch.  Checked on the largest and the smallest
    non-empty expert and six random ones: their weight codes and scales bit
    for bit against the oracle's quantization of the same BF16 draw, their
    rows of H likewise, and 64 sampled outputs each against the oracle's
    exact-partial sums (gate E_norm <= 1e-3 over the samples)."""
    r = synthetic.moe_routing()
    off = r["offsets"]
    off_np = off.numpy().astype(np.int64)
    Mt = int(off_np[-1])
    G, K, N = 256, 2048, 7168
    H = synthetic.moe_grad("h", Mt, device="cuda")
    qH, sH = fb.quantize_1x128(H)
    qD = torch.empty(G, K, N, dtype=torch.uint8, device="cuda")
    sD = torch.empty(G, K // 128, N // 128, dtype=torch.float32, device="cuda")
    for e in range(G):
        fb.quantize_block128(synthetic.expert_weight("down", e, device="cuda"), q=qD[e], s=sD[e])
    offs = off.to(torch.int32).cuda()
    print(f"[grouped] moe down {Mt}x{N}x{K}, {G} experts", flush=True)
    C = fb.grouped_gemm_fp8_blockscaled(offs, qH, sH, qD, sD, opB=oracle.OP_N)
    torch.cuda.synchronize()
    counts = np.diff(off_np)
    nonempty = np.flatnonzero(counts > 0)
    rng = np.random.default_rng(2)
    picks = [int(np.argmax(counts)), int(nonempty[np.argmin(counts[nonempty])])]
    picks += [int(e) for e in rng.choice(np.setdiff1d(nonempty, picks), 6, replace=False)]
    H_cpu = H.cpu()
    worst = 0.0
    for e in picks:
        r0, r1 = int(off_np[e]), int(off_np[e + 1])
        qHo, sHo = oracle.quantize_1x128(bf16_bits(H_cpu[r0:r1]))
        assert np.array_equal(np_u8(qH[r0:r1]), qHo), f"expert {e} input codes"
        assert np.array_equal(np_f32(sH[:, r0:r1]).view(np.uint32), sHo.view(np.uint32)), f"expert {e} input scales"
        W = synthetic.expert_weight("down", e, device="cuda").cpu()
        qB, sB = oracle.quantize_block128(bf16_bits(W))
        assert np.array_equal(np_u8(qD[e]), qB), f"expert {e} weight codes"
        assert np.array_equal(np_f32(sD[e]).view(np.uint32), sB.view(np.uint32)), f"expert {e} weight scales"
        rows = rng.integers(r0, r1, 64)
        cols = rng.integers(0, N, 64)
        Rv = oracle.gemm_blockscaled_entries(qHo, sHo, qB, sB, rows - r0, cols)
        got = C[torch.from_numpy(rows).cuda(), torch.from_numpy(cols).cuda()].cpu().numpy().astype(np.float64)
        err = float(np.max(np.abs(got - Rv)) / np.max(np.abs(Rv)))
        print(f"[grouped] down expert {e} rows {r1 - r0} E_norm={err:.3e}", flush=True)
        worst = max(worst, err)
    assert worst <= 1e-3


@pytest.mark.parametrize("opB", [oracle.OP_N, oracle.OP_T])
def test_grouped_pow2_scales(opB):
    """Power-of-two scales applied in the matrix cores, per expert."""
    counts = [3, 0, 130, 257, 64]
    print(f"[grouped] pow2 scales counts={counts} opB={opB}", flush=True)
    K, N = 384, 256
    off = np.concatenate([[0], np.cumsum(counts)]).astype(np.int64)
    Mt = int(off[-1])
    g = torch.Generator().manual_seed(33)
    qA, sA = oracle.quantize_1x128(bf16_bits(synthetic.randn_bf16((Mt, K), 1.0, g)), True)
    Bs, sBs = [], []
    for e in range(len(counts)):
        Bshape = (K, N) if opB == oracle.OP_N else (N, K)
        qB, sB = oracle.quantize_block128(bf16_bits(synthetic.randn_bf16(Bshape, 0.02, g)), True)
        Bs.append(qB)
        sBs.append(sB)
    B, sB = np.stack(Bs), np.stack(sBs)
    offs = torch.from_numpy(off.astype(np.int32)).cuda()
    C = fb.grouped_gemm_fp8_blockscaled(offs, u8_dev(qA), f32_dev(sA), u8_dev(B), f32_dev(sB), opB=opB,
                                        pow2_scales=True)
    torch.cuda.synchronize()
    R = oracle.grouped_gemm_blockscaled(off, qA, sA, B, sB, opB)
    assert e_norm(np_f32(C), R) <= 1e-3
