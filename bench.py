"""Benchmark of the fine-grained FP8 hot path on one MI355X.

A step is one pass of the dense Fprop path on the 4096 x 7168 x 4096 workload
(DeepSeek-V3 hidden size 7168): 1x128 quantization of the activation
A [4096][7168] (BF16 -> E4M3 + FP32 scales) and 128x128 block quantization of
the weight W [7168][4096] (both in one launch of the two-operand quantizer),
and the block-scaled FP8 GEMM producing FP32 C [4096][4096], in order on one
stream.
Inputs are seeded synthetic tensors already resident in HBM; the step rotates
over several input/output sets whose total exceeds the 256 MB Infinity Cache,
so reads come from HBM.

`value` = 2*M*N*K / step time (TFLOP/s of the whole step, quantizers
included).  `roofline` reports the GEMM kernel alone (average duration from
HIP events around each launch in the timed region) against the dense FP8
MFMA peak.  `kernels` adds each kernel's time and roofline fraction (the
quantizer launch from a second pass of the same steps with events between
the launches, each quantizer also on its own; beside them `stream_us` times a
plain streaming kernel moving the same bytes over the same buffers and
`frac_stream` = stream_us / us), and `extras` times the other workloads' kernels
(backward Dgrad/Wgrad, the accumulation study, the MoE grouped GEMMs).
`cpu_baseline` times the CPU oracle on the whole step, repeated for at least 10 s.

    python bench.py [--steps K] [--warmup W] [--no-extras] [--no-cpu]
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0        # MI355X HBM3E, published
FP8_PEAK_TFLOPS = 5000.0     # MI355X dense FP8 MFMA, published (no sparsity)
QUANT_BYTES_1X128 = 2 + 1 + 4 / 128       # per element: BF16 read, code write, scale per 128
QUANT_BYTES_BLOCK = 2 + 1 + 4 / (128 * 128)

# HBM traffic of one Fprop GEMM launch (4096 x 4096 x 7168, 256 x 256 tiles),
# from rocprofv3 --pmc FETCH_SIZE and WRITE_SIZE passes over
# `bench.py --steps 3 --warmup 1 --warmup-seconds 0 --no-cpu` (64 dispatches
# of this kernel), each scaled by what the same counter reads for a plain
# 1 GiB device copy (FETCH_SIZE x2.0, WRITE_SIZE x1.0).  FETCH_SIZE counts
# what the L2s request beyond themselves: 178 MB is the compulsory minimum of
# the tile order, each of the 8 XCDs (one L2 each) reading the A and B panels
# of its 4 x 8 block of tiles once (8 x 12 x 1.84 MB); sharing across XCDs is
# left to the Infinity Cache.  Valid only for the GEMM source it was measured
# on (sha256 below); reported as null otherwise.
GEMM_TRAFFIC = {"sha256": "d7ab41e494250c7fa40bd673b214cd9b1e704c79ec03b43732dabd4a11643264",
                "fetch_bytes": 178243156, "write_bytes": 67108864}


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20,
                    help="untimed steps; the warm-up also runs for at least --warmup-seconds")
    ap.add_argument("--warmup-seconds", type=float, default=1.0)
    ap.add_argument("--sets", type=int, default=4, help="rotating input/output sets")
    ap.add_argument("--no-extras", action="store_true")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="only run a plain device copy of 1 GiB (src) -> 1 GiB (dst) a few times; "
                         "its FETCH_SIZE/WRITE_SIZE counters scale the quantizers' and GEMM's")
    return ap.parse_args()


def calibrate_copy(torch):
    """A plain copy kernel of known size: 2^30 bytes read, 2^30 written per launch."""
    src = torch.empty(1 << 28, dtype=torch.float32, device="cuda").fill_(1.0)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    t = timed_events(torch, lambda i: dst.copy_(src), 5)
    gbs = 2 * (1 << 30) / (t * 1e-3) / 1e9
    print(json.dumps({"calibration": "device copy", "bytes_read_per_launch": 1 << 30,
                      "bytes_written_per_launch": 1 << 30, "us": round(t * 1e3, 2), "GB/s": round(gbs, 1)}))


class HipEvents:
    """Timing events recorded on the current HIP stream without the
    system-scope fence that torch's events carry (timestamps only, no cache
    write-back to host scope, which costs each record several microseconds
    of GPU time)."""

    FLAGS = 0x20000000  # hipEventDisableSystemFence

    def __init__(self, torch):
        import ctypes
        self.ct = ctypes
        self.torch = torch
        self.hip = ctypes.CDLL("libamdhip64.so")
        self.hip.hipEventCreateWithFlags.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_uint]
        self.hip.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
        self.hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
        self.hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
        self.pool = []

    def record(self):
        e = self.ct.c_void_p()
        if self.hip.hipEventCreateWithFlags(self.ct.byref(e), self.FLAGS) != 0:
            raise RuntimeError("hipEventCreateWithFlags failed")
        self.pool.append(e)
        if self.hip.hipEventRecord(e, self.ct.c_void_p(self.torch.cuda.current_stream().cuda_stream)) != 0:
            raise RuntimeError("hipEventRecord failed")
        return e

    def ms(self, a, b):
        f = self.ct.c_float()
        if self.hip.hipEventElapsedTime(self.ct.byref(f), a, b) != 0:
            raise RuntimeError("hipEventElapsedTime failed")
        return f.value

    def release(self):
        for e in self.pool:
            self.hip.hipEventDestroy(e)
        self.pool = []


def progress(msg):
    """One progress line on stderr (the JSON result goes to stdout)."""
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def warm_up(torch, fn, min_seconds):
    """Run fn(i) until at least min_seconds of GPU work have passed: the GPU
    raises its clocks only after tens of milliseconds under load."""
    i = 0
    t0 = time.perf_counter()
    while True:
        fn(i)
        i += 1
        if i % 16 == 0:
            torch.cuda.synchronize()
            if time.perf_counter() - t0 >= min_seconds:
                return i


def gemm_traffic():
    """Measured HBM bytes per GEMM launch if the GEMM source is unchanged."""
    import hashlib
    src = os.path.join(ROOT, "fp8_fine_grained_quantize_amd", "csrc", "gemm.hip")
    with open(src, "rb") as f:
        if hashlib.sha256(f.read()).hexdigest() != GEMM_TRAFFIC["sha256"]:
            return None
    return GEMM_TRAFFIC["fetch_bytes"] + GEMM_TRAFFIC["write_bytes"]


def timed_events(torch, fn, reps):
    """Median duration (ms) of fn() over reps launches, HIP events (no
    system fence) on the current stream around each launch (the median keeps
    a rare host or system hiccup out of the figure).  A sleep kernel
    queued first keeps the GPU busy while the host enqueues the launches, so
    that each event pair brackets GPU work only (short kernels would
    otherwise wait on the host)."""
    fn(0)
    torch.cuda.synchronize()
    hev = HipEvents(torch)
    torch.cuda._sleep(4_000_000)
    pairs = []
    for i in range(reps):
        a = hev.record()
        fn(i)
        pairs.append((a, hev.record()))
    torch.cuda.synchronize()
    ts = sorted(hev.ms(a, b) for a, b in pairs)
    hev.release()
    return ts[len(ts) // 2]


def stream_ms(torch, fb, srcs, reps):
    """Median duration (ms) of the streaming probe (16 bytes read, 8 written
    per chunk, no tile logic) over the given BF16 inputs, each into a buffer of
    half its size: the quantizers' traffic at the same size and rotation,
    the practical ceiling their times are set against."""
    dsts = [torch.empty(x.numel(), dtype=torch.uint8, device=x.device) for x in srcs]
    n = len(srcs)
    t = timed_events(torch, lambda i: fb.stream_probe(srcs[i % n], dsts[i % n]), reps)
    del dsts
    return t


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for {args.gpus}); the multi-GPU layout is "
              "described, not built.", file=sys.stderr)
        sys.exit(2)
    import numpy as np
    import torch

    if args.calibrate_copy:
        calibrate_copy(torch)
        return

    import fp8_fine_grained_quantize_amd as fb
    import synthetic

    dev = torch.device("cuda:0")
    M, K, N = 4096, 7168, 4096
    A0, W0 = synthetic.dense_fprop()
    S = args.sets
    A = [A0.to(dev)] + [torch.roll(A0, shifts=i, dims=0).to(dev) for i in range(1, S)]
    W = [W0.to(dev)] + [torch.roll(W0, shifts=i, dims=1).to(dev) for i in range(1, S)]
    qA = [torch.empty(M, K, dtype=torch.uint8, device=dev) for _ in range(S)]
    sA = [torch.empty(K // 128, M, dtype=torch.float32, device=dev) for _ in range(S)]
    qW = [torch.empty(K, N, dtype=torch.uint8, device=dev) for _ in range(S)]
    sW = [torch.empty(K // 128, N // 128, dtype=torch.float32, device=dev) for _ in range(S)]
    C = [torch.empty(M, N, dtype=torch.float32, device=dev) for _ in range(S)]

    # Events around the GEMM only: each event record costs the step several
    # microseconds of GPU time, so the quantizers are timed in a second pass.
    ev = {k: [] for k in ("qpair", "gemm")}

    hev = HipEvents(torch)

    # Both operands are quantized by one launch (quantize_1x128_block128:
    # the two quantizers' results, bit for bit, from one grid).
    def step(i, record=False, per_kernel=False):
        j = i % S
        e0 = hev.record() if per_kernel else None
        fb.quantize_1x128_block128(A[j], W[j], qx=qA[j], sx=sA[j], qw=qW[j], sw=sW[j])
        e1 = hev.record() if record else None
        fb.gemm_fp8_blockscaled(qA[j], sA[j], qW[j], sW[j], opB=fb.OP_N, bscale_mode=fb.BSCALE_BLOCK128, C=C[j])
        if record:
            e2 = hev.record()
            ev["gemm"].append((e1, e2))
            if per_kernel:
                ev["qpair"].append((e0, e1))

    progress("warm-up")
    for i in range(args.warmup):
        step(i)
    warm_up(torch, step, args.warmup_seconds)
    torch.cuda.synchronize()

    # Timed region: exactly K steps, synchronized on both sides.
    progress(f"timed: {args.steps} steps")
    t0 = time.perf_counter()
    start = hev.record()
    for i in range(args.steps):
        step(i, record=True)
    end = hev.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_step = hev.ms(start, end) / args.steps
    flops = 2.0 * M * N * K
    value = flops / (ms_step * 1e-3) / 1e12

    def avg(k):
        return sum(hev.ms(a, b) for a, b in ev[k]) / len(ev[k])

    def pct(k):
        """10th, 50th and 90th percentile (us) of the launches recorded under k."""
        ts = sorted(hev.ms(a, b) for a, b in ev[k])
        return {f"p{q}_us": round(ts[min(len(ts) - 1, len(ts) * q // 100)] * 1e3, 2) for q in (10, 50, 90)}

    t_g = avg("gemm")
    p_g = pct("gemm")
    # Second pass, outside the timed region: the same steps with events
    # between the two launches, for the quantizer launch's duration; then
    # each quantizer on its own (separate launches back to back over the
    # same rotating sets) beside the streaming probe over the same buffers.
    for i in range(args.steps):
        step(i, record=True, per_kernel=True)
    torch.cuda.synchronize()
    t_qp = avg("qpair")
    t_q1 = timed_events(torch, lambda i: fb.quantize_1x128(A[i % S], q=qA[i % S], s=sA[i % S]), 40)
    t_qb = timed_events(torch, lambda i: fb.quantize_block128(W[i % S], q=qW[i % S], s=sW[i % S]), 40)
    st_a = stream_ms(torch, fb, A, 40)
    st_w = stream_ms(torch, fb, W, 40)
    gemm_tflops = flops / (t_g * 1e-3) / 1e12
    q1_gbs = M * K * QUANT_BYTES_1X128 / (t_q1 * 1e-3) / 1e9
    qb_gbs = K * N * QUANT_BYTES_BLOCK / (t_qb * 1e-3) / 1e9
    qp_gbs = (M * K * QUANT_BYTES_1X128 + K * N * QUANT_BYTES_BLOCK) / (t_qp * 1e-3) / 1e9
    kernels = {
        "quantize_1x128_block128": {"us": round(t_qp * 1e3, 2), "GB/s": round(qp_gbs, 1),
                                    "frac_hbm": round(qp_gbs / HBM_PEAK_GBS, 4), **pct("qpair"),
                                    "separate_launches_us": round((t_q1 + t_qb) * 1e3, 2),
                                    "stream_us": round((st_a + st_w) * 1e3, 2),
                                    "frac_stream": round((st_a + st_w) / t_qp, 3)},
        "quantize_1x128": {"us": round(t_q1 * 1e3, 2), "GB/s": round(q1_gbs, 1), "frac_hbm": round(q1_gbs / HBM_PEAK_GBS, 4),
                           "stream_us": round(st_a * 1e3, 2), "frac_stream": round(st_a / t_q1, 3)},
        "quantize_block128": {"us": round(t_qb * 1e3, 2), "GB/s": round(qb_gbs, 1), "frac_hbm": round(qb_gbs / HBM_PEAK_GBS, 4),
                              "stream_us": round(st_w * 1e3, 2), "frac_stream": round(st_w / t_qb, 3)},
        "gemm_fp8_blockscaled": {"us": round(t_g * 1e3, 2), "TFLOP/s": round(gemm_tflops, 1),
                                 "frac_mfma": round(gemm_tflops / FP8_PEAK_TFLOPS, 4), **p_g},
    }

    extras = {}
    if not args.no_extras:
        progress("extras: power-of-two step, BF16 and fused epilogues")
        # The same step with power-of-two scales (the pages' variant for some
        # activations): both quantizers in pow2 mode and the GEMM applying
        # the scales inside the matrix cores.
        ev2 = {"gemm": []}
        def step_p2(i, record=False):
            j = i % S
            fb.quantize_1x128_block128(A[j], W[j], True, True, qx=qA[j], sx=sA[j], qw=qW[j], sw=sW[j])
            e0 = hev.record() if record else None
            fb.gemm_fp8_blockscaled(qA[j], sA[j], qW[j], sW[j], C=C[j], pow2_scales=True)
            if record:
                ev2["gemm"].append((e0, hev.record()))
        for i in range(args.warmup):
            step_p2(i)
        torch.cuda.synchronize()
        s0 = hev.record()
        for i in range(args.steps):
            step_p2(i, record=True)
        s1 = hev.record()
        torch.cuda.synchronize()
        t_s2 = hev.ms(s0, s1) / args.steps
        t_g2 = sum(hev.ms(a, b) for a, b in ev2["gemm"]) / len(ev2["gemm"])
        extras["fprop_step_pow2_scales"] = {"ms_per_step": round(t_s2, 5), "TFLOP/s": round(flops / t_s2 / 1e9, 1),
                                            "gemm_us": round(t_g2 * 1e3, 2),
                                            "gemm_TFLOP/s": round(flops / t_g2 / 1e9, 1),
                                            "gemm_frac_mfma": round(flops / t_g2 / 1e9 / FP8_PEAK_TFLOPS, 4)}
        # The step's GEMM with a BF16 output (the fused BF16 epilogue), over
        # the same rotating input sets, fold and power-of-two paths.
        Cb = [torch.empty(M, N, dtype=torch.bfloat16, device=dev) for _ in range(S)]
        Qo = [torch.empty(M, N, dtype=torch.uint8, device=dev) for _ in range(S)]
        sQo = [torch.empty(N // 128, M, dtype=torch.float32, device=dev) for _ in range(S)]
        for p2 in (False, True):
            for j in range(S):
                fb.quantize_1x128(A[j], pow2=p2, q=qA[j], s=sA[j])
                fb.quantize_block128(W[j], pow2=p2, q=qW[j], s=sW[j])
            # the FP32-output GEMM timed back to back like the BF16 and fused
            # variants below (the headline figure above times it inside the step)
            t = timed_events(torch, lambda i: fb.gemm_fp8_blockscaled(qA[i % S], sA[i % S], qW[i % S], sW[i % S],
                                                                      C=C[i % S], pow2_scales=p2), 40)
            extras["fprop_gemm_fp32_out_back_to_back" + ("_pow2_scales" if p2 else "")] = {
                "us": round(t * 1e3, 2), "TFLOP/s": round(flops / t / 1e9, 1),
                "frac_mfma": round(flops / t / 1e9 / FP8_PEAK_TFLOPS, 4)}
            t = timed_events(torch, lambda i: fb.gemm_fp8_blockscaled(qA[i % S], sA[i % S], qW[i % S], sW[i % S],
                                                                      C=Cb[i % S], pow2_scales=p2), 40)
            extras["fprop_gemm_bf16_out" + ("_pow2_scales" if p2 else "")] = {
                "us": round(t * 1e3, 2), "TFLOP/s": round(flops / t / 1e9, 1),
                "frac_mfma": round(flops / t / 1e9 / FP8_PEAK_TFLOPS, 4)}
            # quantize-on-store: the next layer's FP8 input (1x128, power-of-two
            # scales) straight from the epilogue, against GEMM(BF16) + quantize_1x128
            t = timed_events(torch, lambda i: fb.gemm_fp8_blockscaled_q1x128(
                qA[i % S], sA[i % S], qW[i % S], sW[i % S], pow2_scales=p2, pow2=True, Q=Qo[i % S], sQ=sQo[i % S]), 40)
            t2 = timed_events(torch, lambda i: (fb.gemm_fp8_blockscaled(qA[i % S], sA[i % S], qW[i % S], sW[i % S],
                                                                        C=Cb[i % S], pow2_scales=p2),
                                                fb.quantize_1x128(Cb[i % S], pow2=True, q=Qo[i % S], s=sQo[i % S])), 40)
            extras["fprop_gemm_q1x128_pow2_out" + ("_pow2_scales" if p2 else "")] = {
                "us": round(t * 1e3, 2), "TFLOP/s": round(flops / t / 1e9, 1),
                "frac_mfma": round(flops / t / 1e9 / FP8_PEAK_TFLOPS, 4),
                "unfused_bf16_gemm_plus_quantize_us": round(t2 * 1e3, 2)}
        del Cb, Qo, sQo
        extras.update(run_extras(torch, fb, synthetic, dev, np))

    cpu = None
    if not args.no_cpu:
        progress("cpu baseline")
        cpu = cpu_baseline(np, synthetic, A0, W0, M, N, K)

    out = {
        "metric": "FP8 block-scaled GEMM TFLOP/s (% FP8 MFMA peak); quantize GB/s (% HBM)",
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8_e4m3 (fp32 accumulate)",
        "data": "synthetic (seeded N(0,1) activations with 1% outlier channels x30, N(0,0.006) weights)",
        "config": {"workload": "dense Fprop: q1x128(A[4096][7168]) + q128x128(W[7168][4096]) + FP8 GEMM 4096x4096x7168, FP32 out",
                   "M": M, "N": N, "K": K, "rotating_sets": S, "parallelism": "single GPU"},
        "roofline": {"bound": "mfma", "achieved": round(gemm_tflops, 1), "peak": FP8_PEAK_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(gemm_tflops / FP8_PEAK_TFLOPS, 4), "traffic": gemm_traffic(),
                     "traffic_unit": "HBM bytes per launch (rocprofv3 FETCH_SIZE + WRITE_SIZE, copy-calibrated)",
                     "kernel": "gemm_fp8_blockscaled", "algorithmic": "2*M*N*K = 240.52 GFLOP per launch"},
        "kernels": kernels,
        "extras": extras,
        "cpu_baseline": cpu,
        "wall_s_timed": round(wall, 3),
    }
    hev.release()
    print(json.dumps(out))


def n_sets(nbytes, total=640e6):
    """Input/output sets to rotate over so that a memory-bound kernel's
    launches touch more than twice the 256 MB Infinity Cache."""
    return max(2, int(-(-total // nbytes)))


class _Results(dict):
    """Extras' results; each new entry is announced on stderr."""

    def __setitem__(self, k, v):
        progress(f"extras: {k}")
        super().__setitem__(k, v)


def run_extras(torch, fb, synthetic, dev, np):
    """Per-kernel timings on the other workloads (HIP events, few reps)."""
    res = _Results()
    reps = 10
    # launch floor: the smallest launches of the library (one quantizer
    # workgroup, one 128x128x128 GEMM tile), beside which the small workloads'
    # times can be read
    x1 = torch.ones(1, 128, dtype=torch.bfloat16, device=dev)
    q1, s1 = fb.quantize_1x128(x1)
    b1, sb1 = fb.quantize_block128(torch.ones(128, 128, dtype=torch.bfloat16, device=dev))
    a1, sa1 = fb.quantize_1x128(torch.ones(128, 128, dtype=torch.bfloat16, device=dev))
    c1 = torch.empty(128, 128, dtype=torch.float32, device=dev)
    res["launch_floor"] = {
        "quantize_1x128_1x128_us": round(timed_events(torch, lambda i: fb.quantize_1x128(x1, q=q1, s=s1), 40) * 1e3, 2),
        "gemm_128x128x128_us": round(timed_events(torch, lambda i: fb.gemm_fp8_blockscaled(a1, sa1, b1, sb1, C=c1), 40) * 1e3, 2)}
    # the single-GEMM workload (256x512x1024, FP32 out): its three kernels
    A1, B1 = synthetic.single_gemm()
    A1d, B1d = A1.to(dev), B1.to(dev)
    qa1, sa1_ = fb.quantize_1x128(A1d)
    qb1, sb1_ = fb.quantize_block128(B1d)
    c1g = torch.empty(256, 512, dtype=torch.float32, device=dev)
    t_qa = timed_events(torch, lambda i: fb.quantize_1x128(A1d, q=qa1, s=sa1_), 40)
    t_qb = timed_events(torch, lambda i: fb.quantize_block128(B1d, q=qb1, s=sb1_), 40)
    t_g1 = timed_events(torch, lambda i: fb.gemm_fp8_blockscaled(qa1, sa1_, qb1, sb1_, C=c1g), 40)
    fl1 = 2.0 * 256 * 512 * 1024
    res["single_gemm_256x512x1024"] = {
        "quantize_1x128_us": round(t_qa * 1e3, 2), "quantize_block128_us": round(t_qb * 1e3, 2),
        "gemm_us": round(t_g1 * 1e3, 2), "gemm_TFLOP/s": round(fl1 / t_g1 / 1e9, 2),
        "gemm_frac_mfma": round(fl1 / t_g1 / 1e9 / FP8_PEAK_TFLOPS, 5),
        "note": "launch-latency bound (0.27 GFLOP); compare launch_floor"}
    del A1d, B1d, qa1, sa1_, qb1, sb1_, c1g
    # backward: Dgrad dX = dY W^T (OP_T), Wgrad dW = X^T dY (128x1 operands, ROW128)
    X, W, dY = synthetic.backward()
    Xd, Wd, dYd = X.to(dev), W.to(dev), dY.to(dev)
    qdY, sdY = fb.quantize_1x128(dYd)
    qW, sW = fb.quantize_block128(Wd)
    qXT, sXT = fb.quantize_128x1(Xd)
    qdYT, sdYT = fb.quantize_128x1(dYd)
    torch.cuda.synchronize()
    Cd = torch.empty(4096, 7168, dtype=torch.float32, device=dev)
    Cw = torch.empty(7168, 2048, dtype=torch.float32, device=dev)
    fl = 2.0 * 4096 * 7168 * 2048
    t = timed_events(torch, lambda i: fb.gemm_fp8_blockscaled(qdY, sdY, qW, sW, opB=fb.OP_T, C=Cd), reps)
    res["dgrad_4096x7168x2048"] = {"us": round(t * 1e3, 2), "TFLOP/s": round(fl / t / 1e9, 1)}
    t = timed_events(torch, lambda i: fb.gemm_fp8_blockscaled(qXT, sXT, qdYT, sdYT, opB=fb.OP_T,
                                                              bscale_mode=fb.BSCALE_ROW128, C=Cw), reps)
    res["wgrad_7168x2048x4096"] = {"us": round(t * 1e3, 2), "TFLOP/s": round(fl / t / 1e9, 1)}
    # the same two GEMMs with power-of-two scales applied by the matrix cores
    p_dY, p_sdY = fb.quantize_1x128(dYd, pow2=True)
    p_W, p_sW = fb.quantize_block128(Wd, pow2=True)
    p_XT, p_sXT = fb.quantize_128x1(Xd, pow2=True)
    p_dYT, p_sdYT = fb.quantize_128x1(dYd, pow2=True)
    t = timed_events(torch, lambda i: fb.gemm_fp8_blockscaled(p_dY, p_sdY, p_W, p_sW, opB=fb.OP_T, C=Cd,
                                                              pow2_scales=True), reps)
    res["dgrad_4096x7168x2048_pow2_scales"] = {"us": round(t * 1e3, 2), "TFLOP/s": round(fl / t / 1e9, 1)}
    t = timed_events(torch, lambda i: fb.gemm_fp8_blockscaled(p_XT, p_sXT, p_dYT, p_sdYT, opB=fb.OP_T,
                                                              bscale_mode=fb.BSCALE_ROW128, C=Cw, pow2_scales=True), reps)
    res["wgrad_7168x2048x4096_pow2_scales"] = {"us": round(t * 1e3, 2), "TFLOP/s": round(fl / t / 1e9, 1)}
    del p_dY, p_W, p_XT, p_dYT
    # The quantizers rotate over enough input/output sets that their launches
    # read and write from HBM, not from the Infinity Cache.
    for name, x, fn, bpe in [("quantize_128x1_X", Xd, fb.quantize_128x1, QUANT_BYTES_1X128),
                             ("quantize_128x1_dY", dYd, fb.quantize_128x1, QUANT_BYTES_1X128),
                             ("quantize_1x128_dY", dYd, fb.quantize_1x128, QUANT_BYTES_1X128),
                             ("quantize_block128_W_7168x2048", Wd, fb.quantize_block128, QUANT_BYTES_BLOCK)]:
        ns = n_sets(x.numel() * bpe)
        sets = [(x.clone(), *fn(x)) for _ in range(ns)]
        t = timed_events(torch, lambda i: fn(sets[i % ns][0], q=sets[i % ns][1], s=sets[i % ns][2])
                         if fn is not fb.quantize_128x1 else
                         fn(sets[i % ns][0], qT=sets[i % ns][1], s=sets[i % ns][2]), max(reps, 2 * ns))
        gbs = x.numel() * bpe / (t * 1e-3) / 1e9
        ts = stream_ms(torch, fb, [st[0] for st in sets], max(reps, 2 * ns))
        res[name] = {"us": round(t * 1e3, 2), "GB/s": round(gbs, 1), "frac_hbm": round(gbs / HBM_PEAK_GBS, 4),
                     "sets": ns, "stream_us": round(ts * 1e3, 2), "frac_stream": round(ts / t, 3)}
        del sets
    # the pages' backward path: the cached 1x128 FP8 copy re-quantized to
    # 128x1, for dY and for the activations X (the cached forward input)
    qX, sX = fb.quantize_1x128(Xd)
    for name, qs, ss, n in [("requantize_128x1_from_1x128_dY", qdY, sdY, dY.numel()),
                            ("requantize_128x1_from_1x128_X", qX, sX, X.numel())]:
        ns = n_sets(n * (1 + 1 + 8 / 128))
        sets = [(qs.clone(), ss.clone(), *fb.requantize_128x1_from_1x128(qs, ss)) for _ in range(ns)]
        t = timed_events(torch, lambda i: fb.requantize_128x1_from_1x128(sets[i % ns][0], sets[i % ns][1],
                                                                          qT=sets[i % ns][2], sT=sets[i % ns][3]),
                         max(reps, 2 * ns))
        gbs = n * (1 + 1 + 8 / 128) / (t * 1e-3) / 1e9
        res[name] = {"us": round(t * 1e3, 2), "GB/s": round(gbs, 1), "frac_hbm": round(gbs / HBM_PEAK_GBS, 4),
                     "sets": ns}
        del sets
    del qX, sX
    del Xd, Wd, dYd, qXT, qdYT, Cd, Cw
    # accumulation study shapes
    for Kc in (4096, 8192, 16384):
        a, b = synthetic.accum_study(Kc)
        qa, sa = fb.quantize_1x128(a.to(dev))
        qb, sb = fb.quantize_block128(b.to(dev))
        c = torch.empty(1024, 1024, dtype=torch.float32, device=dev)
        t = timed_events(torch, lambda i: fb.gemm_fp8_blockscaled(qa, sa, qb, sb, C=c), reps)
        res[f"gemm_1024x1024x{Kc}"] = {"us": round(t * 1e3, 2), "TFLOP/s": round(2.0 * 1024 * 1024 * Kc / t / 1e9, 1)}
    torch.cuda.empty_cache()
    # MoE grouped up/gate and down projections (256 experts, top-8 of 8192 tokens)
    r = synthetic.moe_routing()
    X8 = r["X"].to(dev)
    tok = r["token_of_row"].to(dev)
    offs = r["offsets"].to(torch.int32).to(dev)
    G, Kh, Nu, Nd = 256, 7168, 4096, 7168
    qX, sX = fb.quantize_1x128(X8, pow2=True)
    ns = n_sets(X8.numel() * QUANT_BYTES_1X128)
    sets = [(X8.clone(), *fb.quantize_1x128(X8, pow2=True)) for _ in range(ns)]
    t = timed_events(torch, lambda i: fb.quantize_1x128(sets[i % ns][0], pow2=True, q=sets[i % ns][1],
                                                        s=sets[i % ns][2]), max(reps, 2 * ns))
    del sets
    gbs = X8.numel() * QUANT_BYTES_1X128 / (t * 1e-3) / 1e9
    res["quantize_1x128_pow2_moe_X"] = {"us": round(t * 1e3, 2), "GB/s": round(gbs, 1), "frac_hbm": round(gbs / HBM_PEAK_GBS, 4),
                                        "sets": ns}
    qA = qX[tok].contiguous()
    sA = sX[:, tok].contiguous()
    Mt = qA.shape[0]
    # All 256 experts' weights quantized 128x128 in one launch on the stacked
    # [256*K][N] tensor (K a multiple of 128: the same blocks as each expert's
    # own quantization, scales [256*K/128][N/128] = the per-expert tables back
    # to back), timed as its own leg.
    Wst = torch.empty(G * Kh, Nu, dtype=torch.bfloat16, device=dev)
    for e in range(G):
        Wst[e * Kh:(e + 1) * Kh] = synthetic.expert_weight("up", e, device=dev)
    qU = torch.empty(G, Kh, Nu, dtype=torch.uint8, device=dev)
    sU = torch.empty(G, Kh // 128, Nu // 128, dtype=torch.float32, device=dev)
    qU2, sU2 = qU.view(G * Kh, Nu), sU.view(G * Kh // 128, Nu // 128)
    t = timed_events(torch, lambda i: fb.quantize_block128(Wst, q=qU2, s=sU2), 3)
    byts = G * Kh * Nu * QUANT_BYTES_BLOCK
    res["quantize_block128_moe_up_weights_256x7168x4096"] = {
        "us": round(t * 1e3, 1), "GB/s": round(byts / t / 1e6, 1), "frac_hbm": round(byts / t / 1e6 / HBM_PEAK_GBS, 4),
        "blocks": G * (Kh // 128) * (Nu // 128)}
    Cu = torch.empty(Mt, Nu, dtype=torch.float32, device=dev)
    t = timed_events(torch, lambda i: fb.grouped_gemm_fp8_blockscaled(offs, qA, sA, qU, sU, C=Cu), 3)
    fl = 2.0 * Mt * Nu * Kh
    byts = G * Kh * Nu + Mt * Kh + Mt * Nu * 4
    res["grouped_up_gate_65536x4096x7168_E256"] = {"us": round(t * 1e3, 1), "TFLOP/s": round(fl / t / 1e9, 1),
                                                    "GB/s": round(byts / t / 1e6, 1),
                                                    "frac_mfma": round(fl / t / 1e9 / FP8_PEAK_TFLOPS, 4),
                                                    "frac_hbm": round(byts / t / 1e6 / HBM_PEAK_GBS, 4)}
    # The up projection with power-of-two weight scales too (its input is the
    # pages' power-of-two activation), the scales then applied by the MFMA.
    Cu2 = torch.empty(Mt, Nu, dtype=torch.float32, device=dev)
    fb.quantize_block128(Wst, pow2=True, q=qU2, s=sU2)
    del Wst
    t = timed_events(torch, lambda i: fb.grouped_gemm_fp8_blockscaled(offs, qA, sA, qU, sU, C=Cu2, pow2_scales=True), 3)
    res["grouped_up_gate_65536x4096x7168_E256_pow2_scales"] = {"us": round(t * 1e3, 1),
                                                               "TFLOP/s": round(fl / t / 1e9, 1),
                                                               "frac_mfma": round(fl / t / 1e9 / FP8_PEAK_TFLOPS, 4)}
    del qU, sU, Cu2
    torch.cuda.empty_cache()
    H = (torch.nn.functional.silu(Cu[:, :2048]) * Cu[:, 2048:]).to(torch.bfloat16)
    del Cu
    qH, sH = fb.quantize_1x128(H)
    ns = n_sets(H.numel() * QUANT_BYTES_1X128)
    sets = [(H, qH, sH)] + [(H.clone(), *fb.quantize_1x128(H)) for _ in range(ns - 1)]
    t = timed_events(torch, lambda i: fb.quantize_1x128(sets[i % ns][0], q=sets[i % ns][1], s=sets[i % ns][2]),
                     max(reps, 2 * ns))
    del sets
    byts = H.numel() * QUANT_BYTES_1X128
    res["quantize_1x128_moe_H_65536x2048"] = {"us": round(t * 1e3, 2), "GB/s": round(byts / t / 1e6, 1),
                                              "frac_hbm": round(byts / t / 1e6 / HBM_PEAK_GBS, 4), "sets": ns}
    Wst = torch.empty(G * 2048, Nd, dtype=torch.bfloat16, device=dev)
    for e in range(G):
        Wst[e * 2048:(e + 1) * 2048] = synthetic.expert_weight("down", e, device=dev)
    qD = torch.empty(G, 2048, Nd, dtype=torch.uint8, device=dev)
    sD = torch.empty(G, 2048 // 128, Nd // 128, dtype=torch.float32, device=dev)
    qD2, sD2 = qD.view(G * 2048, Nd), sD.view(G * 2048 // 128, Nd // 128)
    t = timed_events(torch, lambda i: fb.quantize_block128(Wst, q=qD2, s=sD2), 3)
    byts = G * 2048 * Nd * QUANT_BYTES_BLOCK
    res["quantize_block128_moe_down_weights_256x2048x7168"] = {
        "us": round(t * 1e3, 1), "GB/s": round(byts / t / 1e6, 1), "frac_hbm": round(byts / t / 1e6 / HBM_PEAK_GBS, 4),
        "blocks": G * (2048 // 128) * (Nd // 128)}
    del Wst
    Cdn = torch.empty(Mt, Nd, dtype=torch.float32, device=dev)
    t = timed_events(torch, lambda i: fb.grouped_gemm_fp8_blockscaled(offs, qH, sH, qD, sD, C=Cdn), 3)
    fl = 2.0 * Mt * Nd * 2048
    byts = G * 2048 * Nd + Mt * 2048 + Mt * Nd * 4
    res["grouped_down_65536x7168x2048_E256"] = {"us": round(t * 1e3, 1), "TFLOP/s": round(fl / t / 1e9, 1),
                                                 "GB/s": round(byts / t / 1e6, 1),
                                                 "frac_mfma": round(fl / t / 1e9 / FP8_PEAK_TFLOPS, 4),
                                                 "frac_hbm": round(byts / t / 1e6 / HBM_PEAK_GBS, 4)}
    del qH, sH, Cdn
    torch.cuda.empty_cache()
    # MoE backward of the down projection.  Dgrad: dH_e = dOut_e W_down[e]^T
    # (the stored expert weights read transposed); Wgrad: dW_down[e] =
    # H_e^T dOut_e with both operands quantized 128x1 along tokens inside each
    # expert (ragged token groups).
    dO = synthetic.moe_grad("dout", Mt, device=dev)
    qdO, sdO = fb.quantize_1x128(dO)
    CdH = torch.empty(Mt, 2048, dtype=torch.float32, device=dev)
    t = timed_events(torch, lambda i: fb.grouped_gemm_fp8_blockscaled(offs, qdO, sdO, qD, sD, opB=fb.OP_T, C=CdH), 3)
    fl = 2.0 * Mt * 2048 * Nd
    byts = G * 2048 * Nd + Mt * Nd + Mt * 2048 * 4
    res["grouped_dgrad_down_65536x2048x7168_E256"] = {"us": round(t * 1e3, 1), "TFLOP/s": round(fl / t / 1e9, 1),
                                                       "GB/s": round(byts / t / 1e6, 1),
                                                       "frac_mfma": round(fl / t / 1e9 / FP8_PEAK_TFLOPS, 4),
                                                       "frac_hbm": round(byts / t / 1e6 / HBM_PEAK_GBS, 4)}
    del CdH, qD, sD, qdO, sdO
    torch.cuda.empty_cache()
    counts = (r["offsets"][1:] - r["offsets"][:-1]).tolist()
    groups = sum((c + 127) // 128 for c in counts)          # ragged 128-token groups over all experts
    AT, sAT = fb.quantize_128x1_grouped(H, offs)
    BT, sBT = fb.quantize_128x1_grouped(dO, offs)
    for name, src, qT_, s_ in (("H", H, AT, sAT), ("dOut", dO, BT, sBT)):
        cols = src.shape[1]
        byts = cols * (2 * Mt + 128 * groups) + 4 * groups * cols
        ns = n_sets(byts)
        sets = [(src, qT_, s_)] + [(src.clone(), *fb.quantize_128x1_grouped(src, offs)) for _ in range(ns - 1)]
        t = timed_events(torch, lambda i: fb.quantize_128x1_grouped(sets[i % ns][0], offs, qT=sets[i % ns][1],
                                                                    s=sets[i % ns][2]), max(reps, 2 * ns))
        del sets
        res[f"quantize_128x1_grouped_{name}_{Mt}x{cols}_E256"] = {"us": round(t * 1e3, 2),
                                                                  "GB/s": round(byts / t / 1e6, 1),
                                                                  "frac_hbm": round(byts / t / 1e6 / HBM_PEAK_GBS, 4)}
    Wd = torch.empty(G, 2048, Nd, dtype=torch.float32, device=dev)
    t = timed_events(torch, lambda i: fb.grouped_wgrad_fp8_blockscaled(offs, Mt, AT, sAT, BT, sBT, C=Wd), 3)
    fl = 2.0 * Mt * 2048 * Nd
    byts = G * 2048 * Nd * 4 + (2048 + Nd) * 128 * groups + 4 * groups * (2048 + Nd)
    res["grouped_wgrad_down_2048x7168_T65536_E256"] = {"us": round(t * 1e3, 1), "TFLOP/s": round(fl / t / 1e9, 1),
                                                        "GB/s": round(byts / t / 1e6, 1),
                                                        "frac_mfma": round(fl / t / 1e9 / FP8_PEAK_TFLOPS, 4),
                                                        "frac_hbm": round(byts / t / 1e6 / HBM_PEAK_GBS, 4)}
    del Wd
    torch.cuda.empty_cache()
    Wb = torch.empty(G, 2048, Nd, dtype=torch.bfloat16, device=dev)
    t = timed_events(torch, lambda i: fb.grouped_wgrad_fp8_blockscaled(offs, Mt, AT, sAT, BT, sBT, C=Wb), 3)
    byts = G * 2048 * Nd * 2 + (2048 + Nd) * 128 * groups + 4 * groups * (2048 + Nd)
    res["grouped_wgrad_down_2048x7168_T65536_E256_bf16_out"] = {
        "us": round(t * 1e3, 1), "TFLOP/s": round(fl / t / 1e9, 1), "GB/s": round(byts / t / 1e6, 1),
        "frac_mfma": round(fl / t / 1e9 / FP8_PEAK_TFLOPS, 4), "frac_hbm": round(byts / t / 1e6 / HBM_PEAK_GBS, 4)}
    del Wb, AT, BT, sAT, sBT, dO, H
    torch.cuda.empty_cache()
    return dict(res)


def cpu_baseline(np, synthetic, A0, W0, M, N, K):
    """The oracle as it stands, on the host cores, on the step itself: 1x128
    quantization of A, block quantization of W and the GEMM, repeated until
    at least 10 s of host time have passed (at most 8 passes; one pass takes
    roughly 5 s on 16 host threads).  Scaled to TFLOP/s of the GEMM FLOPs of
    the passes run."""
    import oracle
    try:
        from threadpoolctl import threadpool_info
        blas_threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        blas_threads = None
    a_bits = synthetic.bf16_bits(A0)
    w_bits = synthetic.bf16_bits(W0)
    passes = 0
    t0 = time.perf_counter()
    while passes < 8 and (passes == 0 or time.perf_counter() - t0 < 10.0):
        qa, sa = oracle.quantize_1x128(a_bits)
        qw, sw = oracle.quantize_block128(w_bits)
        oracle.gemm_blockscaled(qa, sa, qw, sw)
        passes += 1
    dt = time.perf_counter() - t0
    flops = 2.0 * M * N * K * passes
    return {"value": round(flops / dt / 1e12, 6), "unit": "TFLOP/s", "cores": blas_threads or os.cpu_count(),
            "kind": "oracle",
            "sample": f"{passes} pass(es) of the whole step: q1x128 of A[{M}][{K}] + q128x128 of W[{K}][{N}] + "
                      f"exact-partial FP64 GEMM {M}x{N}x{K}; {dt:.2f} s",
            "host_cpus_affinity": len(os.sched_getaffinity(0))}


if __name__ == "__main__":
    main()
