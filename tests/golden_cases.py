"""Loader for the hand-derived quantizer fixtures in tests/golden/."""
import json
import os

import numpy as np

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "quant_cases.json")


def _bf16_bits_of(v):
    if v == "-0":
        return 0x8000
    f = np.float32(v)
    b = int(f.view(np.uint32))
    assert b & 0xFFFF == 0, f"{v} is not exact in BF16"
    return b >> 16


def load_cases():
    with open(GOLDEN) as fh:
        data = json.load(fh)
    out = []
    for c in data["cases"]:
        R, C = c["shape"]
        x = np.zeros((R, C), np.uint16)
        for r, col, v in c["entries"]:
            x[r, col] = _bf16_bits_of(v)
        scales = np.array([[int(h, 16) for h in row] for row in c["scales"]], np.uint32)
        codes = [(r, col, int(h, 16)) for r, col, h in c.get("codes", c.get("codes_T", []))]
        out.append(dict(name=c["name"], kind=c["kind"], pow2=c["pow2"], x=x, scale_bits=scales,
                        codes=codes, transposed="codes_T" in c))
    return out
