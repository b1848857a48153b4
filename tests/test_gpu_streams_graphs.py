"""GPU checks that the library keeps no state between calls and can be
captured into a HIP graph: every kernel goes on the caller's stream, and a
call allocates, fills and copies nothing.

* Two streams at once: the Fprop path (two-operand quantizer, then the GEMM
  on 256x256 tiles) on one stream and the Wgrad path (two 128x1 quantizers,
  then the ROW128 GEMM on 224x256 tiles) on another give, bit for bit, what
  the same calls give one after another.
* Graph capture: the two-operand quantizer, the GEMM, the split-K GEMM (its
  partial products into a caller workspace, then the reduction launch) and
  the allocation-free GEMM (partials in the library's scratch array) are
  captured into one graph.  Each of several replays, with the inputs
  rewritten in place before some of them and unrelated eager calls between
  them, must equal the eager calls on the same inputs, bit for bit; the first
  replay's Fprop output also meets the oracle gate.
"""
import numpy as np
import pytest
import torch

import fp8_fine_grained_quantize_amd as fb
import oracle
import synthetic
from tests.gpu_util import e_norm

pytestmark = pytest.mark.gpu


def _bf16(shape, std, seed, outliers=0):
    g = torch.Generator().manual_seed(seed)
    t = synthetic.randn_bf16(shape, std, g, outlier_cols=outliers, outlier_factor=30.0) if outliers else \
        synthetic.randn_bf16(shape, std, g)
    return t.cuda()


def _bits(t):
    return t.contiguous().view(torch.int32 if t.element_size() == 4 else
                               torch.int16 if t.element_size() == 2 else torch.uint8).cpu().numpy()


def _fprop(X, W):
    qx, sx, qw, sw = fb.quantize_1x128_block128(X, W)
    return fb.gemm_fp8_blockscaled(qx, sx, qw, sw)


def _wgrad(X, dY):
    qx, sx = fb.quantize_128x1(X)
    qd, sd = fb.quantize_128x1(dY)
    return fb.gemm_fp8_blockscaled(qx, sx, qd, sd, opB=fb.OP_T, bscale_mode=fb.BSCALE_ROW128)


def test_two_streams_equal_sequential():
    X = _bf16((4096, 7168), 1.0, 1, outliers=3)
    W = _bf16((7168, 4096), 0.006, 2)
    Xw = _bf16((4096, 7168), 1.0, 3)
    dY = _bf16((4096, 2048), 1.0, 4)
    torch.cuda.synchronize()
    print("[streams] sequential", flush=True)
    ref_f = _fprop(X, W)
    ref_w = _wgrad(Xw, dY)
    torch.cuda.synchronize()
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    s1.wait_stream(torch.cuda.current_stream())
    s2.wait_stream(torch.cuda.current_stream())
    print("[streams] concurrent", flush=True)
    for _ in range(3):
        with torch.cuda.stream(s1):
            out_f = _fprop(X, W)
        with torch.cuda.stream(s2):
            out_w = _wgrad(Xw, dY)
        torch.cuda.synchronize()
        assert np.array_equal(_bits(out_f), _bits(ref_f))
        assert np.array_equal(_bits(out_w), _bits(ref_w))


def test_graph_capture_replays_equal_eager():
    M, N, K = 4096, 2048, 1024     # Fprop on 256x256 tiles (128 of them)
    Ms, Ns, Ks = 1024, 1024, 4096  # split over K (16 tiles of 256x256 would not fill the GPU)
    Mn, Nn, Kn = 1024, 768, 2048   # allocation-free GEMM, also split
    assert fb.workspace_bytes(Ms, Ns, Ks) > 0 and fb.workspace_bytes(Mn, Nn, Kn) > 0
    A = _bf16((M, K), 1.0, 11, outliers=3)
    W = _bf16((K, N), 0.02, 12)
    As, Bs = _bf16((Ms, Ks), 1.0, 13), _bf16((Ks, Ns), 0.02, 14)
    An, Bn = _bf16((Mn, Kn), 1.0, 15), _bf16((Kn, Nn), 0.02, 16)
    # static buffers the captured calls read and write
    qA = fb.empty_pitched(M, K, torch.uint8); sA = torch.empty(K // 128, M, device="cuda")
    qW = fb.empty_pitched(K, N, torch.uint8); sW = torch.empty(K // 128, N // 128, device="cuda")
    C = fb.empty_pitched(M, N, torch.float32)
    qs, ss = fb.quantize_1x128(As); qbs, sbs = fb.quantize_block128(Bs)
    Cs = fb.empty_pitched(Ms, Ns, torch.float32)
    ws = torch.empty((fb.workspace_bytes(Ms, Ns, Ks) + 3) // 4, dtype=torch.float32, device="cuda")
    qn, sn = fb.quantize_1x128(An); qbn, sbn = fb.quantize_block128(Bn)
    Cn = fb.empty_pitched(Mn, Nn, torch.float32)

    def run():
        fb.quantize_1x128_block128(A, W, qx=qA, sx=sA, qw=qW, sw=sW)
        fb.gemm_fp8_blockscaled(qA, sA, qW, sW, C=C)
        fb.gemm_fp8_blockscaled(qs, ss, qbs, sbs, C=Cs, workspace=ws)
        fb.gemm_fp8_blockscaled_noalloc(qn, sn, qbn, sbn, Cn)

    def eager():
        qa, sa, qw, sw = fb.quantize_1x128_block128(A, W)
        c = fb.gemm_fp8_blockscaled(qa, sa, qw, sw)
        cs = fb.gemm_fp8_blockscaled(qs, ss, qbs, sbs)
        cn = fb.gemm_fp8_blockscaled(qn, sn, qbn, sbn)
        torch.cuda.synchronize()
        return [_bits(t) for t in (qa, sa, qw, sw, c, cs, cn)], (qa, sa, qw, sw, c)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):  # warm-up outside the capture
        run()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    print("[graph] capture", flush=True)
    with torch.cuda.graph(graph):
        run()
    torch.cuda.synchronize()
    other_a, other_b = _bf16((512, 640), 1.0, 17), _bf16((640, 384), 0.02, 18)
    for rep in range(4):
        if rep in (1, 3):  # new inputs, written in place
            A.copy_(_bf16((M, K), 1.0, 100 + rep, outliers=3))
            W.copy_(_bf16((K, N), 0.02, 200 + rep))
            qs.copy_(fb.quantize_1x128(_bf16((Ms, Ks), 1.0, 300 + rep))[0])
            qbn.copy_(fb.quantize_block128(_bf16((Kn, Nn), 0.02, 400 + rep))[0])
            torch.cuda.synchronize()
        print(f"[graph] replay {rep}", flush=True)
        graph.replay()
        torch.cuda.synchronize()
        got = [_bits(t) for t in (qA, sA, qW, sW, C, Cs, Cn)]
        want, dev_ops = eager()
        for name, g_, w_ in zip(("qA", "sA", "qW", "sW", "C", "C split", "C noalloc"), got, want):
            assert np.array_equal(g_, w_), f"replay {rep}: {name} differs from the eager call"
        if rep == 0:
            qa, sa, qw, sw, c = (t.cpu().numpy() for t in dev_ops)
            R = oracle.gemm_blockscaled(qa, sa, qw, sw)
            assert e_norm(c, R) <= 1e-3
        # unrelated eager work between replays
        qo, so = fb.quantize_1x128(other_a)
        qbo, sbo = fb.quantize_block128(other_b)
        fb.gemm_fp8_blockscaled(qo, so, qbo, sbo)
        torch.cuda.synchronize()
