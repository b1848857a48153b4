"""Seeded synthetic inputs shaped like DeepSeek-V3 layers.

This module only draws random tensors (and the MoE routing that decides the
expert row layout); it holds none of the quantization or GEMM arithmetic.  Both
the oracle-side tests and the GPU-side tests and benchmark take their inputs
from here.

Recipe (all draws from one CPU ``torch.Generator`` seeded per workload, in the
order written; FP32 ``randn`` scaled by the stated standard deviation, outlier
columns multiplied by their factor, then rounded to BF16 with torch's RNE
cast):

* ``single_gemm``  A [256][1024] ~N(0,1), 4 outlier columns x50;
                   B [1024][512] ~N(0,0.02).                         seed 0
* ``dense_fprop``  A [4096][7168] ~N(0,1), round(1% of 7168) = 72 outlier
                   columns x30; W [7168][4096] ~N(0,0.006).          seed 0
* ``accum_study``  A [1024][K], B [K][1024] ~N(0,1), K in {4096, 8192, 16384}.
                                                                      seed K
* ``moe_routing``  logits [8192][256] ~N(0,1), bias [256] ~N(0,0.5); each token
                   picks the top 8 of sigmoid(logits + bias); (expert, token)
                   pairs are stably sorted by expert.  X [8192][7168] ~N(0,1).
                   Expert weights W_up[e] [7168][4096] and W_down[e] [2048][7168]
                   ~N(0,0.006) come from ``expert_weight``: a generator seeded
                   1000+e (up) or 2000+e (down) on the requested device.  seed 0
* ``backward``     X [4096][7168] ~N(0,1); W [7168][2048] ~N(0,0.006);
                   dY [4096][2048] ~N(0,1e-3).                        seed 0
* ``moe_grad``     MoE backward tensors over the expert-ordered rows of
                   ``moe_routing``: "h" [rows][2048] ~N(0,1) (the down
                   projection's input), "dout" [rows][7168] ~N(0,1e-3) (the
                   gradient of its output), "dh" [rows][4096] ~N(0,1e-3) (the
                   gradient of the up projection's output); each from its own
                   generator seeded 3000/3001/3002 on the requested device.
* ``large_bf16``   tensors past 2^31 elements for the index-range tests:
                   BF16 ~N(0,1) drawn directly in BF16 by a device generator
                   seeded by the caller, every 97th row scaled by 2^20 and
                   every 89th by 2^-20 (the scale range).
* ``random_codes`` / ``random_scales``  GEMM operands drawn directly: E4M3
                   codes uniform over all 256 byte values with the two NaN
                   codes replaced by 0x7E / 0xFE, and FP32 scales 2^u with u
                   uniform in (-12, 0]; device generator seeded by the caller.

The hidden size 7168, the expert count 256 with top-8 routing and the expert
width 2048 follow the DeepSeek-V3 description (inprokorea.com wr_id 890463,
third paragraph: one shared and 256 routed experts of intermediate size 2048,
8 active per token); 7168 itself is not printed on the pages.
"""
from __future__ import annotations

import numpy as np
import torch

__all__ = [
    "bf16_bits", "randn_bf16", "single_gemm", "dense_fprop", "accum_study",
    "moe_routing", "expert_weight", "backward", "edge_tensor", "moe_grad",
    "large_bf16", "random_codes", "random_scales",
]


def bf16_bits(t: torch.Tensor) -> np.ndarray:
    """BF16 tensor -> numpy uint16 bit patterns (no arithmetic)."""
    assert t.dtype == torch.bfloat16
    return t.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)


def randn_bf16(shape, std: float, gen: torch.Generator, outlier_cols: int = 0,
               outlier_factor: float = 1.0) -> torch.Tensor:
    x = torch.randn(*shape, generator=gen, dtype=torch.float32) * std
    if outlier_cols:
        idx = torch.randperm(shape[-1], generator=gen)[:outlier_cols]
        x[:, idx] *= outlier_factor
    return x.to(torch.bfloat16)


def single_gemm():
    g = torch.Generator().manual_seed(0)
    A = randn_bf16((256, 1024), 1.0, g, outlier_cols=4, outlier_factor=50.0)
    B = randn_bf16((1024, 512), 0.02, g)
    return A, B


def dense_fprop():
    g = torch.Generator().manual_seed(0)
    A = randn_bf16((4096, 7168), 1.0, g, outlier_cols=72, outlier_factor=30.0)
    W = randn_bf16((7168, 4096), 0.006, g)
    return A, W


def accum_study(K: int):
    g = torch.Generator().manual_seed(K)
    A = randn_bf16((1024, K), 1.0, g)
    B = randn_bf16((K, 1024), 1.0, g)
    return A, B


def moe_routing(tokens: int = 8192, experts: int = 256, topk: int = 8,
                hidden: int = 7168, with_x: bool = True):
    """Returns dict with X [tokens][hidden] bf16 (CPU), token_of_row (int64,
    the source token of each expert-ordered row), offsets (int64 [experts+1])."""
    g = torch.Generator().manual_seed(0)
    logits = torch.randn(tokens, experts, generator=g)
    bias = torch.randn(experts, generator=g) * 0.5
    X = randn_bf16((tokens, hidden), 1.0, g) if with_x else None
    affinity = torch.sigmoid(logits + bias)
    top = torch.topk(affinity, topk, dim=1).indices  # [tokens][topk]
    expert_of = top.reshape(-1)
    token_of = torch.arange(tokens).repeat_interleave(topk)
    order = torch.argsort(expert_of, stable=True)
    expert_sorted = expert_of[order]
    token_of_row = token_of[order]
    counts = torch.bincount(expert_sorted, minlength=experts)
    offsets = torch.zeros(experts + 1, dtype=torch.int64)
    offsets[1:] = torch.cumsum(counts, 0)
    return {"X": X, "token_of_row": token_of_row, "offsets": offsets, "counts": counts}


def expert_weight(kind: str, e: int, device="cpu", K: int | None = None, N: int | None = None,
                  std: float = 0.006) -> torch.Tensor:
    """Expert weight [K][N] bf16 drawn on ``device`` from its own seed."""
    if kind == "up":
        seed, K, N = 1000 + e, K or 7168, N or 4096
    elif kind == "down":
        seed, K, N = 2000 + e, K or 2048, N or 7168
    else:
        raise ValueError(kind)
    g = torch.Generator(device=device).manual_seed(seed)
    return (torch.randn(K, N, generator=g, device=device, dtype=torch.float32) * std).to(torch.bfloat16)


def moe_grad(kind: str, rows: int, device="cpu") -> torch.Tensor:
    """MoE backward tensor ``kind`` ("h", "dout" or "dh") with ``rows``
    expert-ordered rows, bf16, drawn on ``device``."""
    seed, cols, std = {"h": (3000, 2048, 1.0), "dout": (3001, 7168, 1e-3), "dh": (3002, 4096, 1e-3)}[kind]
    g = torch.Generator(device=device).manual_seed(seed)
    return (torch.randn(rows, cols, generator=g, device=device, dtype=torch.float32) * std).to(torch.bfloat16)


def backward():
    g = torch.Generator().manual_seed(0)
    X = randn_bf16((4096, 7168), 1.0, g)
    W = randn_bf16((7168, 2048), 0.006, g)
    dY = randn_bf16((4096, 2048), 1e-3, g)
    return X, W, dY


def edge_tensor(shape, seed: int, zero_tile_every: int = 7) -> torch.Tensor:
    """BF16 tensor mixing magnitudes over the whole BF16 range: normal values,
    subnormals, exact zeros and negative zeros, whole zero rows, and huge
    values; used for edge-case parity."""
    g = torch.Generator().manual_seed(seed)
    n = int(np.prod(shape))
    mant = torch.randn(n, generator=g, dtype=torch.float32)
    expo = torch.randint(-140, 120, (n,), generator=g).to(torch.float32)
    x = mant * torch.exp2(expo)
    bits = x.to(torch.bfloat16).view(torch.int16).clone()
    pick = torch.randint(0, 16, (n,), generator=g)
    bits[pick == 0] = 0
    bits[pick == 1] = -32768  # 0x8000, negative zero
    t = bits.view(torch.bfloat16).reshape(shape).clone()
    if len(shape) == 2 and zero_tile_every:
        t[::zero_tile_every, :] = 0
    return t


def large_bf16(shape, seed: int, device="cuda") -> torch.Tensor:
    g = torch.Generator(device=device).manual_seed(seed)
    x = torch.randn(shape, generator=g, device=device, dtype=torch.bfloat16)
    x[::97] *= 2.0 ** 20
    x[::89] *= 2.0 ** -20
    return x


def random_codes(shape, seed: int, device="cuda") -> torch.Tensor:
    g = torch.Generator(device=device).manual_seed(seed)
    c = torch.randint(0, 256, shape, generator=g, device=device, dtype=torch.uint8)
    nan = (c & 0x7F) == 0x7F
    c[nan] -= 1
    return c


def random_scales(shape, seed: int, device="cuda") -> torch.Tensor:
    g = torch.Generator(device=device).manual_seed(seed)
    return torch.exp2(torch.rand(shape, generator=g, device=device) * -12.0)
