"""The streaming probe (the quantizers' comparison kernel) reads every chunk
and writes the documented fold of it, including a count that leaves a
partial last pass of the grid."""
import numpy as np
import pytest
import torch

import fp8_fine_grained_quantize_amd as fb

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("chunks", [1, 511, 512, 100003, 3 * 1024 * 1024 + 7])
def test_stream_probe_output(chunks):
    rng = np.random.default_rng(chunks)
    w = rng.integers(0, 2 ** 32, (chunks, 4), dtype=np.uint32)
    src = torch.from_numpy(w.view(np.uint8).reshape(-1)).cuda()
    dst = torch.zeros(chunks * 8, dtype=torch.uint8, device="cuda")
    print(f"[stream] chunks={chunks}", flush=True)
    fb.stream_probe(src, dst)
    torch.cuda.synchronize()
    got = dst.cpu().numpy().view(np.uint32).reshape(chunks, 2)
    want = np.stack([w[:, 0] ^ w[:, 1], w[:, 2] ^ w[:, 3]], axis=1)
    assert np.array_equal(got, want)
