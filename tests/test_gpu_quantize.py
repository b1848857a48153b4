"""GPU parity of the quantizers: codes and scales bit-exact against the oracle.

Inputs are the seeded synthetic tensors at the workloads' full sizes (or row /
tile samples of the largest), ragged shapes that span several tiles with a
partial tail, tensors mixing zeros, negative zeros, subnormals and huge
values, pitched views and empty inputs.  A dedicated case quantizes every
BF16 value of magnitude <= 448 with scale 1, so the hardware conversion is
checked against the oracle's encoder on each of them.
"""
import numpy as np
import pytest
import torch

import fp8_fine_grained_quantize_amd as fb
import oracle
import synthetic
from synthetic import bf16_bits
from tests.gpu_util import dev, np_f32, np_u8, u8_dev

pytestmark = pytest.mark.gpu

GPU_Q = {"1x128": fb.quantize_1x128, "128x1": fb.quantize_128x1, "block128": fb.quantize_block128}
ORA_Q = {"1x128": oracle.quantize_1x128, "128x1": oracle.quantize_128x1, "block128": oracle.quantize_block128}


def _check(kind, x_cpu, pow2, x_dev=None):
    print(f"[quant] {kind} shape={tuple(x_cpu.shape)} pow2={pow2}", flush=True)
    xd = dev(x_cpu) if x_dev is None else x_dev
    q, s = GPU_Q[kind](xd, pow2=pow2)
    torch.cuda.synchronize()
    qo, so = ORA_Q[kind](bf16_bits(x_cpu), pow2)
    qg, sg = np_u8(q), np_f32(s)
    assert qg.shape == qo.shape and sg.shape == so.shape
    bad = np.argwhere(qg != qo)
    assert bad.size == 0, f"{len(bad)} code mismatches, first at {bad[0]}: gpu {qg[tuple(bad[0])]:#x} oracle {qo[tuple(bad[0])]:#x}"
    assert np.array_equal(sg.view(np.uint32), so.view(np.uint32)), "scale mismatch"


@pytest.mark.parametrize("pow2", [False, True])
@pytest.mark.parametrize("kind", ["1x128", "128x1", "block128"])
@pytest.mark.parametrize("shape", [(130, 200), (1, 7), (300, 70), (129, 255), (256, 1024), (5, 129)])
def test_ragged_edge_values(kind, shape, pow2):
    _check(kind, synthetic.edge_tensor(shape, seed=shape[0] * 7 + shape[1]), pow2)


@pytest.mark.parametrize("pow2", [False, True])
@pytest.mark.parametrize("kind", ["1x128", "128x1", "block128"])
def test_gaussian_ragged(kind, pow2):
    g = torch.Generator().manual_seed(3)
    x = synthetic.randn_bf16((1000, 900), 1.0, g, outlier_cols=9, outlier_factor=30.0)
    _check(kind, x, pow2)


@pytest.mark.parametrize("pow2", [False, True])
def test_single_gemm_inputs(pow2):
    A, B = synthetic.single_gemm()
    _check("1x128", A, pow2)
    _check("block128", B, pow2)


@pytest.mark.parametrize("pow2", [False, True])
def test_dense_fprop_full_size(pow2):
    A, W = synthetic.dense_fprop()
    _check("1x128", A, pow2)
    _check("block128", W, pow2)


def test_backward_full_size():
    X, W, dY = synthetic.backward()
    _check("1x128", dY, False)
    _check("block128", W, False)
    _check("128x1", X, False)
    _check("128x1", dY, False)


def test_every_bf16_value_through_the_converter():
    """Rows of 128: one +-448 (so s = 1 and y = x) and 127 BF16 values; all
    BF16 magnitudes <= 448, both signs.  Then the same values doubled with a
    896 tile maximum (s = 2)."""
    mags = np.arange(0, 0x43E1, dtype=np.uint16)  # 0 .. 448 in BF16 bits
    vals = np.concatenate([mags, mags | np.uint16(0x8000)])
    rows = -(-vals.size // 127)
    body = np.zeros(rows * 127, np.uint16)
    body[:vals.size] = vals
    x = np.concatenate([np.full((rows, 1), 0x43E0, np.uint16), body.reshape(rows, 127)], axis=1)
    t = torch.from_numpy(x.view(np.int16)).view(torch.bfloat16)
    for pow2 in (False, True):
        _check("1x128", t, pow2)
    t2 = (t.float() * 2).to(torch.bfloat16)  # exact: doubling
    _check("1x128", t2, False)
    # a scale that is not a power of two: tile maximum 1
    small = np.arange(0, 0x3F81, dtype=np.uint16)
    sv = np.concatenate([small, small | np.uint16(0x8000)])
    r2 = -(-sv.size // 127)
    b2 = np.zeros(r2 * 127, np.uint16)
    b2[:sv.size] = sv
    x3 = np.concatenate([np.full((r2, 1), 0x3F80, np.uint16), b2.reshape(r2, 127)], axis=1)
    _check("1x128", torch.from_numpy(x3.view(np.int16)).view(torch.bfloat16), False)


def test_pitched_views():
    g = torch.Generator().manual_seed(5)
    base = synthetic.randn_bf16((200, 520), 1.0, g)
    view_cpu = base[:, 8:392]  # pitch 520, 16-byte aligned start
    base_dev = base.to("cuda")  # pitch 520 elements = 1040 bytes
    _check("1x128", view_cpu.contiguous(), False, x_dev=base_dev[:, 8:392])
    _check("block128", view_cpu.contiguous(), True, x_dev=base_dev[:, 8:392])
    _check("128x1", view_cpu.contiguous(), False, x_dev=base_dev[:, 8:392])


def test_moe_activation_rows_sampled():
    """The MoE input X [8192][7168] with power-of-two scales: 1x128
    quantization is row-wise, so a sample of rows is checked against the
    oracle on those rows."""
    r = synthetic.moe_routing()
    X = r["X"]
    q, s = fb.quantize_1x128(dev(X), pow2=True)
    torch.cuda.synchronize()
    rows = np.random.default_rng(0).choice(X.shape[0], 512, replace=False)
    qo, so = oracle.quantize_1x128(bf16_bits(X)[rows], True)
    assert np.array_equal(np_u8(q)[rows], qo)
    assert np.array_equal(np_f32(s)[:, rows].view(np.uint32), so.view(np.uint32))


def test_requantize_from_1x128():
    for shape, pow2 in [((300, 200), False), ((4096, 2048), False), ((257, 384), True), ((130, 129), False)]:
        g = torch.Generator().manual_seed(shape[0])
        x = synthetic.randn_bf16(shape, 1e-3, g, outlier_cols=3, outlier_factor=20.0)
        qo, so = oracle.quantize_1x128(bf16_bits(x))
        print(f"[requant] shape={shape} pow2={pow2}", flush=True)
        qT, sT = fb.requantize_128x1_from_1x128(u8_dev(qo), torch.from_numpy(so).cuda(), pow2=pow2)
        torch.cuda.synchronize()
        qTo, sTo = oracle.requantize_128x1_from_1x128(qo, so, pow2)
        assert np.array_equal(np_u8(qT), qTo)
        assert np.array_equal(np_f32(sT).view(np.uint32), sTo.view(np.uint32))


@pytest.mark.parametrize("pow2", [False, True])
def test_requantize_wide_range_and_subnormal_scales(pow2):
    """Token rows scaled by 10^u, u uniform in [-30, 30], so that one 128-token
    column tile mixes dequantized values of every magnitude (general FP32
    quotients), and a 128 x 128 corner near the bottom of the BF16 range, so
    that its 1x128 scales and its 128x1 scales are subnormal (the clamped
    quotient).  Codes and scales bit for bit against the oracle."""
    T, C = 640, 384
    g = torch.Generator().manual_seed(41 + pow2)
    mag = torch.pow(10.0, torch.rand(T, 1, generator=g) * 60 - 30)
    x = (torch.randn(T, C, generator=g) * mag).to(torch.bfloat16)
    x[:128, :128] = (torch.randn(128, 128, generator=g) * 1e-38).to(torch.bfloat16)
    qo, so = oracle.quantize_1x128(bf16_bits(x))
    assert np.any(so[0, :128] < np.float32(2.0 ** -126))
    print(f"[requant] wide range pow2={pow2}", flush=True)
    qT, sT = fb.requantize_128x1_from_1x128(u8_dev(qo), torch.from_numpy(so).cuda(), pow2=pow2)
    torch.cuda.synchronize()
    qTo, sTo = oracle.requantize_128x1_from_1x128(qo, so, pow2)
    assert np.all(sTo[0, :128] < np.float32(2.0 ** -126))
    assert np.array_equal(np_u8(qT), qTo)
    assert np.array_equal(np_f32(sT).view(np.uint32), sTo.view(np.uint32))


@pytest.mark.parametrize("pow2_x,pow2_w", [(False, False), (True, False), (False, True), (True, True)])
@pytest.mark.parametrize("xshape,wshape", [((300, 520), (130, 140)), ((10, 100), (7168, 4096)),
                                           ((4096, 7168), (257, 384)), ((33, 129), (1, 8))])
def test_two_operand_quantizer(xshape, wshape, pow2_x, pow2_w):
    """quantize_1x128_block128 equals the two separate quantizers bit for bit
    (an odd number of 1x128 bands leaves half a workgroup idle), and the
    oracle on every code and scale."""
    g = torch.Generator().manual_seed(xshape[0] + wshape[1])
    x = synthetic.randn_bf16(xshape, 1.0, g, outlier_cols=2, outlier_factor=30.0)
    w = synthetic.randn_bf16(wshape, 0.02, g)
    print(f"[quant] two-operand x={xshape} w={wshape} pow2={pow2_x},{pow2_w}", flush=True)
    qx, sx, qw, sw = fb.quantize_1x128_block128(dev(x), dev(w), pow2_x, pow2_w)
    qx1, sx1 = fb.quantize_1x128(dev(x), pow2=pow2_x)
    qw1, sw1 = fb.quantize_block128(dev(w), pow2=pow2_w)
    torch.cuda.synchronize()
    assert torch.equal(qx, qx1) and torch.equal(sx, sx1) and torch.equal(qw, qw1) and torch.equal(sw, sw1)
    if xshape[0] * xshape[1] <= 300 * 520:
        qo, so = oracle.quantize_1x128(bf16_bits(x), pow2_x)
        assert np.array_equal(np_u8(qx), qo) and np.array_equal(np_f32(sx).view(np.uint32), so.view(np.uint32))
    if wshape[0] * wshape[1] <= 257 * 384:
        qo, so = oracle.quantize_block128(bf16_bits(w), pow2_w)
        assert np.array_equal(np_u8(qw), qo) and np.array_equal(np_f32(sw).view(np.uint32), so.view(np.uint32))


def test_two_operand_quantizer_one_side_empty():
    g = torch.Generator().manual_seed(3)
    x = synthetic.randn_bf16((64, 256), 1.0, g)
    w = synthetic.randn_bf16((256, 128), 0.02, g)
    e = torch.empty(0, 256, dtype=torch.bfloat16)
    qx, sx, qw, sw = fb.quantize_1x128_block128(dev(x), dev(e))
    qx1, sx1 = fb.quantize_1x128(dev(x))
    qx2, sx2, qw2, sw2 = fb.quantize_1x128_block128(dev(e), dev(w))
    qw1, sw1 = fb.quantize_block128(dev(w))
    torch.cuda.synchronize()
    assert torch.equal(qx, qx1) and torch.equal(sx, sx1) and qw.shape == (0, 256)
    assert torch.equal(qw2, qw1) and torch.equal(sw2, sw1) and qx2.shape == (0, 256)


def test_empty_inputs_are_noops():
    x = torch.empty(0, 256, dtype=torch.bfloat16, device="cuda")
    q, s = fb.quantize_1x128(x)
    qT, sT = fb.quantize_128x1(x)
    qb, sb = fb.quantize_block128(x)
    torch.cuda.synchronize()
    assert q.shape == (0, 256) and qT.shape == (256, 0) and sb.shape == (0, 2)


def test_deterministic():
    A, _ = synthetic.single_gemm()
    d = dev(A)
    q1, s1 = fb.quantize_1x128(d)
    q2, s2 = fb.quantize_1x128(d)
    torch.cuda.synchronize()
    assert torch.equal(q1, q2) and torch.equal(s1, s2)
