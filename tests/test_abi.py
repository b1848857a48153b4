"""The C-ABI library loads, exports every symbol the public header declares,
and rejects invalid arguments on the host before anything is enqueued.

CPU only: every call here either fails validation or has an empty shape, so
no HIP runtime call is made.
"""
import ctypes
import os
import re

import pytest

import fp8_fine_grained_quantize_amd as fb

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include", "libfp8blk.h")

INVALID, OK, UNSUPPORTED = 1, 0, 2


def _declared():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"\b(fp8blk_[a-z0-9_]+)\s*\(", text)))


def test_library_is_built():
    assert os.path.exists(fb.library_path), "run python -m fp8_fine_grained_quantize_amd.build"


def test_exports_every_declared_symbol():
    L = fb.lib()
    declared = _declared()
    assert len(declared) >= 9
    for name in declared:
        assert hasattr(L, name), name
    assert sorted(fb.EXPORTED_SYMBOLS) == declared


def test_version_and_status_strings():
    assert fb.abi_version() == 6
    assert fb.token_group_slots(65536, 256) == 512 + 256
    assert fb.token_group_slots(100, 3) == 3 and fb.token_group_slots(-1, 3) == 0
    assert fb.status_string(0) == "FP8BLK_OK"
    assert fb.status_string(1) == "FP8BLK_ERR_INVALID_ARG"
    assert fb.status_string(2) == "FP8BLK_ERR_UNSUPPORTED"
    assert fb.status_string(3) == "FP8BLK_ERR_LAUNCH"
    assert fb.workspace_bytes(4096, 4096, 7168, 1) == 0      # tiles fill the GPU: no split
    ws = fb.workspace_bytes(1024, 1024, 4096, 1)              # 64 tiles: K is split
    assert ws > 0 and ws % (1024 * 1024 * 4) == 0 and 2 <= ws // (1024 * 1024 * 4) <= 16
    assert fb.workspace_bytes(1024, 1024, 4096, 8) == 0       # grouped: none
    assert fb.workspace_bytes(1024, 1024, 256, 1) == 0        # two K groups: no split


P = ctypes.c_void_p
FAKE = P(0x100000)     # never dereferenced: every call below fails validation
MIS = P(0x100004)      # misaligned for 16-byte matrices
NULL = P(0)


@pytest.mark.parametrize("fn", ["fp8blk_quantize_1x128", "fp8blk_quantize_128x1", "fp8blk_quantize_block128"])
def test_quantizer_validation(fn):
    f = getattr(fb.lib(), fn)
    # null input
    assert f(NULL, 4, 128, 128, FAKE, 128, FAKE, 0, NULL) == INVALID
    # null output / scales
    assert f(FAKE, 4, 128, 128, NULL, 128, FAKE, 0, NULL) == INVALID
    assert f(FAKE, 4, 128, 128, FAKE, 128, NULL, 0, NULL) == INVALID
    # negative sizes
    assert f(FAKE, -1, 128, 128, FAKE, 128, FAKE, 0, NULL) == INVALID
    assert f(FAKE, 4, -128, 128, FAKE, 128, FAKE, 0, NULL) == INVALID
    # unknown flag
    assert f(FAKE, 4, 128, 128, FAKE, 128, FAKE, 0x2, NULL) == INVALID
    # pitch below the row length, or not a multiple of 16 bytes
    if fn == "fp8blk_quantize_128x1":
        assert f(FAKE, 4, 128, 120, FAKE, 16, FAKE, 0, NULL) == INVALID  # ldx < C
        assert f(FAKE, 4, 128, 128, FAKE, 4, FAKE, 0, NULL) == INVALID   # ldqT not 16-byte multiple
        assert f(FAKE, 40, 128, 128, FAKE, 32, FAKE, 0, NULL) == INVALID  # ldqT < T
    else:
        assert f(FAKE, 4, 128, 120, FAKE, 128, FAKE, 0, NULL) == INVALID
        assert f(FAKE, 4, 128, 132, FAKE, 132, FAKE, 0, NULL) == INVALID
        assert f(FAKE, 4, 128, 128, FAKE, 112, FAKE, 0, NULL) == INVALID
    # misaligned matrix pointer
    assert f(MIS, 4, 128, 128, FAKE, 128, FAKE, 0, NULL) == INVALID
    # empty shapes are valid no-ops (nothing enqueued)
    assert f(NULL, 0, 128, 128, NULL, 128, NULL, 0, NULL) == OK
    assert f(NULL, 4, 0, 128, NULL, 128, NULL, 0, NULL) == OK


def test_two_operand_quantizer_validation():
    f = fb.lib().fp8blk_quantize_1x128_block128
    good = (FAKE, 4, 128, 128, FAKE, 128, FAKE, 0)  # valid on its own; never passed with a valid partner
    # each side's arguments are checked as by its own entry point
    assert f(NULL, 4, 128, 128, FAKE, 128, FAKE, 0, *good, NULL) == INVALID
    assert f(*good, FAKE, 4, 128, 128, FAKE, 128, NULL, 0, NULL) == INVALID
    assert f(FAKE, 4, 128, 120, FAKE, 128, FAKE, 0, *good, NULL) == INVALID
    assert f(*good, FAKE, 4, 128, 128, FAKE, 112, FAKE, 0, NULL) == INVALID
    assert f(FAKE, 4, 128, 128, FAKE, 128, FAKE, 0x2, *good, NULL) == INVALID
    assert f(*good, FAKE, 4, 128, 128, FAKE, 128, FAKE, 0x4, NULL) == INVALID
    assert f(MIS, 4, 128, 128, FAKE, 128, FAKE, 0, *good, NULL) == INVALID
    # both empty: a valid no-op
    assert f(NULL, 0, 128, 128, NULL, 128, NULL, 0, NULL, 4, 0, 128, NULL, 128, NULL, 0, NULL) == OK


def test_requantize_validation():
    f = fb.lib().fp8blk_requantize_128x1_from_1x128
    assert f(NULL, FAKE, 256, 128, 128, FAKE, 256, FAKE, 0, NULL) == INVALID
    assert f(FAKE, NULL, 256, 128, 128, FAKE, 256, FAKE, 0, NULL) == INVALID
    assert f(FAKE, FAKE, 256, 128, 128, FAKE, 256, FAKE, 4, NULL) == INVALID
    assert f(FAKE, FAKE, 256, 128, 100, FAKE, 256, FAKE, 0, NULL) == INVALID
    assert f(NULL, NULL, 0, 128, 128, NULL, 16, NULL, 0, NULL) == OK


def test_probe_validation():
    """Diagnostic entry points reject bad arguments before any launch."""
    f = fb.lib().fp8blk_mfma_probe
    assert f(2, FAKE, FAKE, FAKE, NULL) == INVALID
    assert f(0, NULL, FAKE, FAKE, NULL) == INVALID
    assert f(0, MIS, FAKE, FAKE, NULL) == INVALID
    g = fb.lib().fp8blk_stream_probe
    assert g(FAKE, -1, FAKE, NULL) == INVALID
    assert g(NULL, 4, FAKE, NULL) == INVALID
    assert g(MIS, 4, FAKE, NULL) == INVALID
    assert g(FAKE, 4, P(0x100004), NULL) == INVALID
    assert g(NULL, 0, NULL, NULL) == OK


def _gemm(M=256, N=256, K=256, A=FAKE, lda=256, sA=FAKE, B=FAKE, ldb=256, opB=0, sB=FAKE, mode=0, C=FAKE,
          ldc=256):
    return fb.lib().fp8blk_gemm_fp8_blockscaled(M, N, K, A, lda, sA, B, ldb, opB, sB, mode, C, ldc, NULL, 0, NULL)


def test_gemm_validation():
    assert _gemm(K=200) == INVALID            # K % 128
    assert _gemm(K=0) == INVALID
    assert _gemm(M=-1) == INVALID
    assert _gemm(opB=2) == INVALID
    assert _gemm(mode=5) == INVALID
    assert _gemm(A=NULL) == INVALID
    assert _gemm(B=NULL) == INVALID
    assert _gemm(C=NULL) == INVALID
    assert _gemm(sA=NULL) == INVALID
    assert _gemm(sB=NULL) == INVALID
    assert _gemm(lda=128) == INVALID           # lda < K
    assert _gemm(ldb=100) == INVALID           # not a 16-byte multiple
    assert _gemm(ldc=255) == INVALID           # < N
    assert _gemm(opB=1, ldb=128) == INVALID    # [N][K] needs ldb >= K
    assert _gemm(A=MIS) == INVALID
    assert _gemm(M=0) == OK and _gemm(N=0) == OK
    assert _gemm(opB=0x200, ldc=260) == INVALID    # BF16 C: pitch must be a multiple of 8 elements
    assert _gemm(opB=0x400) == INVALID             # unknown flag bit
    # per-lane copy offsets are 32-bit: operand pitches of 2^23 bytes or more are refused
    assert _gemm(lda=1 << 23) == UNSUPPORTED
    assert _gemm(opB=1, ldb=1 << 23) == UNSUPPORTED


def test_q1x128_validation():
    f = fb.lib().fp8blk_gemm_fp8_blockscaled_q1x128

    def call(M=256, N=256, K=256, A=FAKE, lda=256, sA=FAKE, B=FAKE, ldb=256, opB=0, sB=FAKE, Q=FAKE, ldq=256,
             sQ=FAKE, qflags=0):
        return f(M, N, K, A, lda, sA, B, ldb, opB, sB, Q, ldq, sQ, qflags, NULL)

    assert call(Q=NULL) == INVALID and call(sQ=NULL) == INVALID
    assert call(ldq=200) == INVALID             # below N
    assert call(ldq=264) == INVALID             # not a 16-byte multiple
    assert call(qflags=2) == INVALID
    assert call(K=200) == INVALID and call(opB=2) == INVALID
    assert call(M=0) == OK and call(N=0) == OK


def test_grouped_validation():
    f = fb.lib().fp8blk_grouped_gemm_fp8_blockscaled

    def call(G=4, off=FAKE, Mt=256, mgr=0, N=256, K=256, A=FAKE, lda=256, sA=FAKE, B=FAKE, ldb=256,
             strideB=65536, opB=0, sB=FAKE, ssB=4, C=FAKE, ldc=256):
        return f(G, off, Mt, mgr, N, K, A, lda, sA, B, ldb, strideB, opB, sB, ssB, C, ldc, NULL, 0, NULL)

    assert call(off=NULL) == INVALID
    assert call(K=100) == INVALID
    assert call(strideB=1000) == INVALID       # below one expert's matrix
    assert call(ssB=1) == INVALID              # below one expert's scale table
    assert call(opB=3) == INVALID
    assert call(G=-1) == INVALID
    assert call(G=0) == OK and call(Mt=0) == OK


def test_grouped_128x1_validation():
    f = fb.lib().fp8blk_quantize_128x1_grouped
    T, G = 300, 4                      # 6 group slots: qT needs 768 columns

    def call(T=T, C=256, ldx=256, G=G, off=FAKE, qT=FAKE, ldqT=768, s=FAKE, flags=0):
        return f(FAKE, T, C, ldx, G, off, qT, ldqT, s, flags, NULL)

    assert call(off=NULL) == INVALID
    assert call(ldqT=752) == INVALID            # fewer columns than 128 slots
    assert call(qT=NULL) == INVALID
    assert call(s=NULL) == INVALID
    assert call(flags=2) == INVALID
    assert call(G=-1) == INVALID and call(T=-1) == INVALID
    assert call(ldx=100) == INVALID
    assert f(NULL, 0, 256, 256, G, FAKE, NULL, 512, NULL, 0, NULL) == OK   # no tokens
    assert call(G=0, ldqT=256) == OK                                        # no experts


def test_grouped_wgrad_validation():
    f = fb.lib().fp8blk_grouped_wgrad_fp8_blockscaled
    T, G, M, N = 300, 4, 128, 256      # 6 group slots: operands need 768 columns

    def call(G=G, off=FAKE, T=T, M=M, N=N, A=FAKE, lda=768, sA=FAKE, B=FAKE, ldb=768, sB=FAKE, flags=0,
             C=FAKE, ldc=256, sC=128 * 256):
        return f(G, off, T, M, N, A, lda, sA, B, ldb, sB, flags, C, ldc, sC, NULL)

    assert call(off=NULL) == INVALID
    assert call(lda=640) == INVALID and call(ldb=640) == INVALID
    assert call(A=NULL) == INVALID and call(B=NULL) == INVALID and call(C=NULL) == INVALID
    assert call(sA=NULL) == INVALID and call(sB=NULL) == INVALID
    assert call(sC=128 * 256 - 4) == INVALID    # experts' outputs would overlap
    assert call(sC=128 * 256 + 2) == INVALID    # not 16-byte aligned per expert
    assert call(flags=1) == INVALID
    assert call(M=-1) == INVALID and call(T=-1) == INVALID
    assert call(G=0) == OK and call(M=0) == OK and call(N=0) == OK
    assert call(T=0, A=NULL, B=NULL, sA=NULL, sB=NULL, off=NULL) == INVALID   # C is still written


def test_binding_fails_loudly_without_library(monkeypatch, tmp_path):
    monkeypatch.setattr(fb, "library_path", str(tmp_path / "missing.so"))
    monkeypatch.setattr(fb, "_LIB", None)
    with pytest.raises(fb.Fp8BlkError):
        fb.lib()
