"""GPU parity of the MoE backward path: ragged per-expert 128x1
quantization, the grouped Wgrad, and the grouped Dgrad (the grouped GEMM
with the expert weights read transposed).

Small ragged cases are compared with the oracle in full (codes and scales
bit for bit, GEMM outputs within E_norm 1e-3, integer cases exactly); the
MoE-shaped case (256 experts, skewed top-8 routing over 8192 tokens, the
shapes the benchmark times) is checked on sampled experts and entries.
"""
import numpy as np
import pytest
import torch

import fp8_fine_grained_quantize_amd as fb
import oracle
import synthetic
from synthetic import bf16_bits, edge_tensor
from tests.gpu_util import dev, e_norm, f32_dev, np_f32, np_u8, u8_dev

pytestmark = pytest.mark.gpu

RAGGED = [[1, 0, 129, 127, 128, 3], [0, 0, 0], [300], [128, 0, 256, 5, 0], [0, 77, 0]]


def _offs(counts):
    off = np.concatenate([[0], np.cumsum(counts)]).astype(np.int64)
    return off, torch.from_numpy(off.astype(np.int32)).cuda()


def _gpu_quant(x_bits_t, offs, pow2):
    qT, s = fb.quantize_128x1_grouped(dev(x_bits_t), offs, pow2=pow2)
    torch.cuda.synchronize()
    return qT, s


@pytest.mark.parametrize("pow2", [False, True])
@pytest.mark.parametrize("counts", RAGGED)
@pytest.mark.parametrize("C", [200, 256])
def test_grouped_128x1_bitwise(counts, C, pow2):
    print(f"[moe-bwd] quantize_128x1_grouped counts={counts} C={C} pow2={pow2}", flush=True)
    off, offs = _offs(counts)
    T = int(off[-1])
    x = edge_tensor((max(T, 1), C), 50 + len(counts) + C)[:T]
    qT, s = _gpu_quant(x, offs, pow2)
    rq, rs = oracle.quantize_128x1_grouped(bf16_bits(x), off, pow2)
    ng = rs.shape[0]
    assert qT.shape[1] == 128 * fb.token_group_slots(T, len(counts))
    assert np.array_equal(np_u8(qT[:, :128 * ng]), rq)
    assert np.array_equal(np_f32(s[:ng]).view(np.uint32), rs.view(np.uint32))


def test_grouped_128x1_aligned_equals_dense():
    counts = [256, 128, 0, 384]
    off, offs = _offs(counts)
    T = int(off[-1])
    g = torch.Generator().manual_seed(8)
    x = synthetic.randn_bf16((T, 384), 1.0, g, outlier_cols=3, outlier_factor=30.0)
    qg, sg = _gpu_quant(x, offs, False)
    qd, sd = fb.quantize_128x1(dev(x))
    torch.cuda.synchronize()
    assert torch.equal(qg[:, :T].cpu(), qd.cpu())
    assert torch.equal(sg[:T // 128].cpu(), sd.cpu())


@pytest.mark.parametrize("pow2", [False, True])
@pytest.mark.parametrize("counts", [[1, 0, 129, 127, 128, 3], [300], [0, 77, 0], [640, 1, 1000]])
def test_grouped_wgrad_small(counts, pow2):
    print(f"[moe-bwd] grouped wgrad counts={counts} pow2={pow2}", flush=True)
    off, offs = _offs(counts)
    T, M, N = int(off[-1]), 256, 200
    g = torch.Generator().manual_seed(60 + len(counts))
    X = synthetic.randn_bf16((T, M), 1.0, g, outlier_cols=2, outlier_factor=20.0)
    dY = synthetic.randn_bf16((T, N), 1e-3, g)
    AT, sA = _gpu_quant(X, offs, pow2)
    BT, sB = _gpu_quant(dY, offs, pow2)
    W = fb.grouped_wgrad_fp8_blockscaled(offs, T, AT, sA, BT, sB, pow2_scales=pow2)
    torch.cuda.synchronize()
    rA, rsA = oracle.quantize_128x1_grouped(bf16_bits(X), off, pow2)
    rB, rsB = oracle.quantize_128x1_grouped(bf16_bits(dY), off, pow2)
    R = oracle.grouped_wgrad_blockscaled(off, rA, rsA, rB, rsB)
    Wg = np_f32(W)
    for e in range(len(counts)):
        if counts[e] == 0:
            assert not Wg[e].any(), f"expert {e} has no tokens: dW must be zero"
        else:
            assert e_norm(Wg[e], R[e]) <= 1e-3, e


@pytest.mark.parametrize("pow2_flag", [False, True])
def test_grouped_wgrad_integers_exact(pow2_flag):
    """Integer inputs with power-of-two scales quantize exactly; every partial
    and sum stays an integer times 2^-8 below 2^24, so both GEMM paths return
    the integer product X_e^T dY_e bit for bit."""
    counts = [5, 0, 130, 128, 1, 61]
    off, offs = _offs(counts)
    T, M, N = int(off[-1]), 160, 144
    rng = np.random.default_rng(12)
    X = rng.integers(-15, 16, size=(T, M))
    dY = rng.integers(-15, 16, size=(T, N))
    AT, sA = _gpu_quant(torch.tensor(X, dtype=torch.bfloat16), offs, True)
    BT, sB = _gpu_quant(torch.tensor(dY, dtype=torch.bfloat16), offs, True)
    W = np_f32(fb.grouped_wgrad_fp8_blockscaled(offs, T, AT, sA, BT, sB, pow2_scales=pow2_flag))
    for e in range(len(counts)):
        t0, t1 = off[e], off[e + 1]
        ref = (X[t0:t1].T.astype(np.int64) @ dY[t0:t1].astype(np.int64)).astype(np.float32)
        assert np.array_equal(W[e], ref), e


def test_grouped_wgrad_no_tokens_writes_zeros():
    off, offs = _offs([0, 0, 0])
    C = torch.full((3, 128, 144), 7.0, device="cuda")
    AT = torch.empty(128, 0, dtype=torch.uint8, device="cuda")
    BT = torch.empty(144, 0, dtype=torch.uint8, device="cuda")
    none = torch.empty(0, device="cuda")
    fb.grouped_wgrad_fp8_blockscaled(offs, 0, AT, none, BT, none, C=C)
    torch.cuda.synchronize()
    assert not C.any()


@pytest.mark.parametrize("pow2", [False, True])
def test_grouped_dgrad_small(pow2):
    """Dgrad of the up projection: dX_e = dH_e . W_e^T with W_e [7168-like K][N]
    stored as for Fprop and read transposed (OP_T) with its own block scales."""
    counts = [3, 0, 130, 257, 64]
    print(f"[moe-bwd] grouped dgrad counts={counts} pow2={pow2}", flush=True)
    off, offs = _offs(counts)
    Mt, Kw, Nw = int(off[-1]), 384, 256      # W_e [Kw][Nw]; dgrad contracts over Nw
    g = torch.Generator().manual_seed(70)
    dH = synthetic.randn_bf16((Mt, Nw), 1e-3, g)
    qA, sA = oracle.quantize_1x128(bf16_bits(dH), pow2)
    Ws, sWs = [], []
    for e in range(len(counts)):
        qW, sW = oracle.quantize_block128(bf16_bits(synthetic.randn_bf16((Kw, Nw), 0.02, g)), pow2)
        Ws.append(qW)
        sWs.append(sW)
    Wq, sWq = np.stack(Ws), np.stack(sWs)
    C = fb.grouped_gemm_fp8_blockscaled(offs, u8_dev(qA), f32_dev(sA), u8_dev(Wq), f32_dev(sWq), opB=oracle.OP_T,
                                        pow2_scales=pow2)
    torch.cuda.synchronize()
    R = oracle.grouped_gemm_blockscaled(off, qA, sA, Wq, sWq, oracle.OP_T)
    assert e_norm(np_f32(C), R) <= 1e-3


def test_moe_wgrad_down_projection_sampled():
    """dW_down[e] [2048][7168] = H_e^T dOut_e over 256 experts (top-8 of 8192
    tokens, 65,536 expert rows), both operands quantized per expert along
    tokens on the GPU; sampled experts' codes and scales are checked bit for
    bit against the oracle, then sampled entries of dW against the oracle's
    sums over the oracle's own codes."""
    r = synthetic.moe_routing(with_x=False)
    off = r["offsets"].numpy()
    offs = r["offsets"].to(torch.int32).cuda()
    T, G = int(off[-1]), 256
    H = synthetic.moe_grad("h", T, device="cuda")
    dO = synthetic.moe_grad("dout", T, device="cuda")
    print("[moe-bwd] quantize H [65536][2048], dOut [65536][7168] per expert", flush=True)
    AT, sA = fb.quantize_128x1_grouped(H, offs)
    BT, sB = fb.quantize_128x1_grouped(dO, offs)
    print("[moe-bwd] grouped wgrad 256 x [2048][7168]", flush=True)
    W = fb.grouped_wgrad_fp8_blockscaled(offs, T, AT, sA, BT, sB)
    torch.cuda.synchronize()
    PG = oracle.token_group_starts(off)
    counts = off[1:] - off[:-1]
    rng = np.random.default_rng(2)
    picks = [int(np.argmax(counts)), int(np.argmin(np.where(counts > 0, counts, 1 << 30)))]
    picks += [int(e) for e in rng.choice(G, 3, replace=False)]
    worst = 0.0
    for e in picks:
        t0, t1 = int(off[e]), int(off[e + 1])
        if t1 == t0:
            assert not W[e].any()
            continue
        one = np.array([0, t1 - t0])
        hq, hs = oracle.quantize_128x1_grouped(bf16_bits(H[t0:t1].cpu()), one)
        dq, ds = oracle.quantize_128x1_grouped(bf16_bits(dO[t0:t1].cpu()), one)
        c0, c1 = 128 * int(PG[e]), 128 * int(PG[e + 1])
        assert np.array_equal(np_u8(AT[:, c0:c1]), hq), e
        assert np.array_equal(np_u8(BT[:, c0:c1]), dq), e
        assert np.array_equal(np_f32(sA[PG[e]:PG[e + 1]]).view(np.uint32), hs.view(np.uint32)), e
        assert np.array_equal(np_f32(sB[PG[e]:PG[e + 1]]).view(np.uint32), ds.view(np.uint32)), e
        rows = rng.integers(0, 2048, 48)
        cols = rng.integers(0, 7168, 48)
        Rv = oracle.grouped_wgrad_entries(one, hq, hs, dq, ds, [0] * 48, rows, cols)
        got = W[e][torch.from_numpy(rows).cuda(), torch.from_numpy(cols).cuda()].cpu().numpy().astype(np.float64)
        worst = max(worst, float(np.max(np.abs(got - Rv)) / np.max(np.abs(Rv))))
    print(f"[moe-bwd] sampled E_norm={worst:.3e} over experts {picks}", flush=True)
    assert worst <= 1e-3
