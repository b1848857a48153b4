"""Accumulation study on the CPU (context only, not a parity check): the
maximum relative error E_norm = max|C - R| / max|R| of an FP8 GEMM whose
products are accumulated with the limited precision the pages report for the
H800 (``limited_dot``: terms aligned to the largest exponent, 14 bits kept,
32 products per step), against R = the exact FP64 sum of the same quantized
inputs, for

  * tensor-wise scales with the whole K accumulated in the limited format
    (the setting of the pages' "nearly 2 %" at K = 4096), and
  * the pages' method: 1x128 / 128x128 scales, each 128-deep group
    accumulated in the limited format, then promoted to FP32 with its scales.

Inputs: the accumulation-study operands A [1024][K], B [K][1024] ~ N(0, 1)
(zero mean), and their absolute values (all products positive, so the
truncation errors add up instead of cancelling); the first 64 rows and 64
columns.  Run: python -m oracle.limited_accumulation_study
"""
import numpy as np

from . import fp8_oracle as o


def study(K: int, positive: bool, rows: int = 64, cols: int = 64):
    import synthetic
    A, B = synthetic.accum_study(K)
    if positive:
        A, B = A.abs(), B.abs()
    a, b = synthetic.bf16_bits(A[:rows]), synthetic.bf16_bits(B[:, :cols])
    qa, sa = o.quantize_per_tensor(a)
    qb, sb = o.quantize_per_tensor(b)
    ref_t = (o.e4m3_decode(qa) @ o.e4m3_decode(qb)) * (np.float64(sa) * np.float64(sb))
    whole = o.gemm_limited_per_tensor(qa, sa, qb, sb)
    qa1, sa1 = o.quantize_1x128(a)
    qb1, sb1 = o.quantize_block128(b)
    ref_g = o.gemm_blockscaled(qa1, sa1, qb1, sb1)
    grouped = o.gemm_blockscaled_limited(qa1, sa1, qb1, sb1)
    en = lambda c, r: float(np.max(np.abs(c - r)) / np.max(np.abs(r)))
    return en(whole, ref_t), en(grouped, ref_g)


if __name__ == "__main__":
    print("| K | inputs | whole K, tensor-wise scales | per-128 promotion, 1x128/128x128 scales |")
    print("|---|---|---|---|")
    for K in (4096, 8192, 16384):
        for positive in (False, True):
            w, g = study(K, positive)
            print(f"| {K} | {'|N(0,1)|' if positive else 'N(0,1)'} | {w:.3%} | {g:.2e} |", flush=True)
