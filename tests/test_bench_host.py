"""Host-side checks of bench.py (no GPU): the one-GPU rule of its command
line and the guard that keeps the committed HBM traffic figure tied to the
GEMM source it was measured on."""
import importlib.util
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _bench():
    spec = importlib.util.spec_from_file_location("bench_under_test", os.path.join(ROOT, "bench.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def test_more_than_one_gpu_is_refused_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU only" in r.stderr
    assert r.stdout == ""


def test_traffic_figure_follows_the_gemm_source():
    b = _bench()
    t = b.gemm_traffic()
    algorithmic = 2 * 4096 * 7168 + (7168 // 128) * 4096 * 4 + (7168 // 128) * (4096 // 128) * 4 + 4096 * 4096 * 4
    if t is not None:  # measured on this very source: at least the compulsory bytes, and no wild re-reads
        assert algorithmic <= t <= 4 * algorithmic
    b.GEMM_TRAFFIC = dict(b.GEMM_TRAFFIC, sha256="0" * 64)
    assert b.gemm_traffic() is None  # any other source: no figure
