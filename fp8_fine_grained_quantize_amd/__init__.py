"""Python binding for libfp8blk (fine-grained FP8 quantization + block-scaled
FP8 GEMM on MI355X / gfx950).

Argument marshalling only: every step runs in the HIP kernels of
``libfp8blk.so``.  PyTorch supplies device memory (output tensors are
allocated with ``torch.empty``) and the current HIP stream.  The library must
have been built (``python -m fp8_fine_grained_quantize_amd.build``); there is
no fallback of any kind, and every failed call raises ``Fp8BlkError``.

Function names and argument meanings follow ``include/libfp8blk.h``.
"""
from __future__ import annotations

import ctypes
import os

import torch

__all__ = [
    "Fp8BlkError", "lib", "library_path", "OP_N", "OP_T", "BSCALE_BLOCK128", "BSCALE_ROW128",
    "SCALE_POW2", "GEMM_POW2_SCALES", "GEMM_OUT_BF16", "quantize_1x128", "quantize_128x1", "quantize_block128",
    "requantize_128x1_from_1x128", "gemm_fp8_blockscaled", "grouped_gemm_fp8_blockscaled",
    "quantize_128x1_grouped", "token_group_slots", "grouped_wgrad_fp8_blockscaled", "gemm_fp8_blockscaled_q1x128",
    "workspace_bytes", "status_string", "abi_version", "EXPORTED_SYMBOLS", "empty_pitched", "as_pitched",
    "mfma_probe", "gemm_fp8_blockscaled_noalloc",
]

OP_N, OP_T = 0, 1
BSCALE_BLOCK128, BSCALE_ROW128 = 0, 1
SCALE_POW2 = 0x1
GEMM_POW2_SCALES = 0x100   # OR into opB: every scale is a power of two
GEMM_OUT_BF16 = 0x200      # OR into opB (flags of the grouped Wgrad): C is BF16

library_path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libfp8blk.so")

_i64, _u32, _vp, _sz, _int = ctypes.c_int64, ctypes.c_uint32, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int

_SIGNATURES = {
    "fp8blk_quantize_1x128": (_int, [_vp, _i64, _i64, _i64, _vp, _i64, _vp, _u32, _vp]),
    "fp8blk_quantize_128x1": (_int, [_vp, _i64, _i64, _i64, _vp, _i64, _vp, _u32, _vp]),
    "fp8blk_quantize_block128": (_int, [_vp, _i64, _i64, _i64, _vp, _i64, _vp, _u32, _vp]),
    "fp8blk_quantize_1x128_block128": (_int, [_vp, _i64, _i64, _i64, _vp, _i64, _vp, _u32,
                                              _vp, _i64, _i64, _i64, _vp, _i64, _vp, _u32, _vp]),
    "fp8blk_requantize_128x1_from_1x128": (_int, [_vp, _vp, _i64, _i64, _i64, _vp, _i64, _vp, _u32, _vp]),
    "fp8blk_gemm_fp8_blockscaled": (_int, [_i64, _i64, _i64, _vp, _i64, _vp, _vp, _i64, _int, _vp, _int,
                                           _vp, _i64, _vp, _sz, _vp]),
    "fp8blk_gemm_fp8_blockscaled_q1x128": (_int, [_i64, _i64, _i64, _vp, _i64, _vp, _vp, _i64, _int, _vp, _vp, _i64,
                                                  _vp, _u32, _vp]),
    "fp8blk_grouped_gemm_fp8_blockscaled": (_int, [_i64, _vp, _i64, _i64, _i64, _i64, _vp, _i64, _vp, _vp,
                                                   _i64, _i64, _int, _vp, _i64, _vp, _i64, _vp, _sz, _vp]),
    "fp8blk_quantize_128x1_grouped": (_int, [_vp, _i64, _i64, _i64, _i64, _vp, _vp, _i64, _vp, _u32, _vp]),
    "fp8blk_token_group_slots": (_i64, [_i64, _i64]),
    "fp8blk_grouped_wgrad_fp8_blockscaled": (_int, [_i64, _vp, _i64, _i64, _i64, _vp, _i64, _vp, _vp, _i64,
                                                    _vp, _u32, _vp, _i64, _i64, _vp]),
    "fp8blk_workspace_bytes": (_sz, [_i64, _i64, _i64, _i64]),
    "fp8blk_mfma_probe": (_int, [_int, _vp, _vp, _vp, _vp]),
    "fp8blk_stream_probe": (_int, [_vp, _i64, _vp, _vp]),
    "fp8blk_gemm_fp8_blockscaled_noalloc": (_int, [_i64, _i64, _i64, _vp, _i64, _vp, _vp, _i64, _int, _vp, _int,
                                                   _vp, _i64, _vp]),
    "fp8blk_status_string": (ctypes.c_char_p, [_int]),
    "fp8blk_abi_version": (_int, []),
}
EXPORTED_SYMBOLS = tuple(_SIGNATURES)


class Fp8BlkError(RuntimeError):
    pass


_LIB = None


def lib() -> ctypes.CDLL:
    """Load libfp8blk.so (after torch, so that both use the same HIP runtime)."""
    global _LIB
    if _LIB is None:
        if not os.path.exists(library_path):
            raise Fp8BlkError(f"{library_path} is missing: build it with "
                              "`python -m fp8_fine_grained_quantize_amd.build`")
        L = ctypes.CDLL(library_path)
        for name, (res, args) in _SIGNATURES.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _LIB = L
    return _LIB


def status_string(code: int) -> str:
    return lib().fp8blk_status_string(code).decode()


def abi_version() -> int:
    return lib().fp8blk_abi_version()


def workspace_bytes(M: int, N: int, K: int, G: int = 1) -> int:
    return lib().fp8blk_workspace_bytes(M, N, K, G)


def mfma_probe(A: torch.Tensor, B: torch.Tensor, instr: int = 0) -> torch.Tensor:
    """One 16x16 tile product over 128 E4M3 k by matrix-core instruction
    `instr` (see fp8blk_mfma_probe); A, B uint8 [16][128] on the device."""
    assert A.dtype == torch.uint8 and B.dtype == torch.uint8
    assert tuple(A.shape) == (16, 128) and tuple(B.shape) == (16, 128)
    A, B = A.contiguous(), B.contiguous()
    C = torch.empty(16, 16, dtype=torch.float32, device=A.device)
    _check(lib().fp8blk_mfma_probe(instr, _ptr(A), _ptr(B), _ptr(C), _stream()), "mfma_probe")
    return C


def stream_probe(src: torch.Tensor, dst: torch.Tensor) -> torch.Tensor:
    """Plain streaming kernel with the quantizers' traffic (see
    fp8blk_stream_probe): reads src (a multiple of 16 bytes), writes half as
    many bytes into dst; both contiguous on the device."""
    nb = src.numel() * src.element_size()
    assert src.is_contiguous() and dst.is_contiguous() and nb % 16 == 0
    assert dst.numel() * dst.element_size() >= nb // 2
    _check(lib().fp8blk_stream_probe(_ptr(src), nb // 16, _ptr(dst), _stream()), "stream_probe")
    return dst


def _check(code: int, what: str):
    if code != 0:
        raise Fp8BlkError(f"{what} failed: {status_string(code)}")


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None and t.numel() else ctypes.c_void_p(0)


def _pitch(t: torch.Tensor) -> int:
    """Row pitch (elements) of a row-major 2-D view."""
    assert t.dim() == 2, "expected a 2-D tensor"
    if t.numel() == 0:
        return _pad16(t.shape[1], t.element_size())
    assert t.stride(1) == 1 or t.shape[1] == 1, "expected a row-major 2-D tensor (unit column stride)"
    return t.stride(0) if t.stride(0) >= t.shape[1] else t.shape[1]


def _bf16_bits(x: torch.Tensor) -> torch.Tensor:
    if x.dtype == torch.bfloat16:
        return x
    if x.dtype in (torch.int16, torch.uint16):
        return x
    raise TypeError(f"expected a bfloat16 tensor, got {x.dtype}")


def _pad16(n: int, elem: int) -> int:
    q = 16 // elem
    return (n + q - 1) // q * q


def _empty_pitched(rows: int, cols: int, dtype, device, elem: int):
    """[rows][cols] view into storage whose row pitch is a multiple of 16 bytes."""
    pitch = _pad16(cols, elem)
    if pitch == cols:
        return torch.empty(rows, cols, dtype=dtype, device=device)
    return torch.empty(rows, pitch, dtype=dtype, device=device)[:, :cols]


def empty_pitched(rows: int, cols: int, dtype, device="cuda"):
    """Allocate a [rows][cols] matrix whose row pitch is a multiple of 16 bytes
    (the layout every entry point requires)."""
    return _empty_pitched(rows, cols, dtype, device, torch.empty(0, dtype=dtype).element_size())


def as_pitched(t: torch.Tensor) -> torch.Tensor:
    """Return `t` itself if its rows already sit at a 16-byte pitch, else a
    copy in a freshly allocated 16-byte-pitched matrix."""
    if t.dim() == 2 and t.stride(1) == 1 and (t.stride(0) * t.element_size()) % 16 == 0 \
            and t.data_ptr() % 16 == 0:
        return t
    out = empty_pitched(t.shape[0], t.shape[1], t.dtype, t.device)
    out.copy_(t)
    return out


def quantize_1x128(x: torch.Tensor, pow2: bool = False, q=None, s=None):
    """x [M][K] bf16 (device) -> (q uint8 [M][K], s float32 [ceil(K/128)][M])."""
    x = _bf16_bits(x)
    M, K = x.shape
    G = (K + 127) // 128
    q = _empty_pitched(M, K, torch.uint8, x.device, 1) if q is None else q
    s = torch.empty(G, M, dtype=torch.float32, device=x.device) if s is None else s
    _check(lib().fp8blk_quantize_1x128(_ptr(x), M, K, _pitch(x), _ptr(q), _pitch(q), _ptr(s),
                                       SCALE_POW2 if pow2 else 0, _stream()), "quantize_1x128")
    return q, s


def quantize_128x1(x: torch.Tensor, pow2: bool = False, qT=None, s=None):
    """x [T][C] bf16 -> (qT uint8 [C][T], s float32 [ceil(T/128)][C])."""
    x = _bf16_bits(x)
    T, C = x.shape
    G = (T + 127) // 128
    qT = _empty_pitched(C, T, torch.uint8, x.device, 1) if qT is None else qT
    s = torch.empty(G, C, dtype=torch.float32, device=x.device) if s is None else s
    _check(lib().fp8blk_quantize_128x1(_ptr(x), T, C, _pitch(x), _ptr(qT), _pitch(qT), _ptr(s),
                                       SCALE_POW2 if pow2 else 0, _stream()), "quantize_128x1")
    return qT, s


def quantize_block128(w: torch.Tensor, pow2: bool = False, q=None, s=None):
    """w [R][C] bf16 -> (q uint8 [R][C], s float32 [ceil(R/128)][ceil(C/128)])."""
    w = _bf16_bits(w)
    R, C = w.shape
    q = _empty_pitched(R, C, torch.uint8, w.device, 1) if q is None else q
    s = torch.empty((R + 127) // 128, (C + 127) // 128, dtype=torch.float32, device=w.device) if s is None else s
    _check(lib().fp8blk_quantize_block128(_ptr(w), R, C, _pitch(w), _ptr(q), _pitch(q), _ptr(s),
                                          SCALE_POW2 if pow2 else 0, _stream()), "quantize_block128")
    return q, s


def quantize_1x128_block128(x: torch.Tensor, w: torch.Tensor, pow2_x: bool = False, pow2_w: bool = False,
                            qx=None, sx=None, qw=None, sw=None):
    """quantize_1x128(x) and quantize_block128(w) in one launch (the two
    operands of an Fprop GEMM); returns (qx, sx, qw, sw) as the two calls do."""
    x, w = _bf16_bits(x), _bf16_bits(w)
    M, K = x.shape
    R, C = w.shape
    qx = _empty_pitched(M, K, torch.uint8, x.device, 1) if qx is None else qx
    sx = torch.empty((K + 127) // 128, M, dtype=torch.float32, device=x.device) if sx is None else sx
    qw = _empty_pitched(R, C, torch.uint8, w.device, 1) if qw is None else qw
    sw = torch.empty((R + 127) // 128, (C + 127) // 128, dtype=torch.float32, device=w.device) if sw is None else sw
    _check(lib().fp8blk_quantize_1x128_block128(_ptr(x), M, K, _pitch(x), _ptr(qx), _pitch(qx), _ptr(sx),
                                                SCALE_POW2 if pow2_x else 0, _ptr(w), R, C, _pitch(w), _ptr(qw),
                                                _pitch(qw), _ptr(sw), SCALE_POW2 if pow2_w else 0, _stream()),
           "quantize_1x128_block128")
    return qx, sx, qw, sw


def requantize_128x1_from_1x128(q: torch.Tensor, sq: torch.Tensor, pow2: bool = False, qT=None, sT=None):
    """Cached 1x128 codes q [T][C] + scales sq [ceil(C/128)][T] ->
    (qT uint8 [C][T], sT float32 [ceil(T/128)][C])."""
    T, C = q.shape
    qT = _empty_pitched(C, T, torch.uint8, q.device, 1) if qT is None else qT
    sT = torch.empty((T + 127) // 128, C, dtype=torch.float32, device=q.device) if sT is None else sT
    _check(lib().fp8blk_requantize_128x1_from_1x128(_ptr(q), _ptr(sq), T, C, _pitch(q), _ptr(qT), _pitch(qT),
                                                    _ptr(sT), SCALE_POW2 if pow2 else 0, _stream()),
           "requantize_128x1_from_1x128")
    return qT, sT


def _out_flag(C, out_dtype):
    dt = C.dtype if C is not None else out_dtype
    if dt == torch.bfloat16:
        return GEMM_OUT_BF16, torch.bfloat16, 2
    if dt == torch.float32:
        return 0, torch.float32, 4
    raise TypeError(f"output must be float32 or bfloat16, got {dt}")


def gemm_fp8_blockscaled(A, sA, B, sB, opB: int = OP_N, bscale_mode: int = BSCALE_BLOCK128, C=None,
                         split_k: bool = True, workspace=None, pow2_scales: bool = False,
                         out_dtype=torch.float32):
    """C[M][N] float32 = block-scaled product of E4M3 codes A [M][K] and B
    ([K][N] for OP_N, [N][K] for OP_T); see the header for scale layouts.
    With split_k, a workspace of workspace_bytes(M, N, K) bytes is passed
    (allocated here unless given), which lets the library split K on shapes
    whose tiles cannot fill the GPU.  pow2_scales asserts that every scale is
    a power of two (GEMM_POW2_SCALES).  out_dtype (or C's dtype) float32 or
    bfloat16 (GEMM_OUT_BF16: the FP32 result rounded to nearest even)."""
    M, K = A.shape
    N = B.shape[1] if opB == OP_N else B.shape[0]
    ob, odt, oel = _out_flag(C, out_dtype)
    C = _empty_pitched(M, N, odt, A.device, oel) if C is None else C
    ws_ptr, ws_bytes = None, 0
    if split_k and M and N and K:
        need = workspace_bytes(M, N, K, 1)
        if need:
            if workspace is None:
                workspace = torch.empty((need + 3) // 4, dtype=torch.float32, device=A.device)
            ws_ptr, ws_bytes = _ptr(workspace), workspace.numel() * workspace.element_size()
    _check(lib().fp8blk_gemm_fp8_blockscaled(M, N, K, _ptr(A), _pitch(A), _ptr(sA), _ptr(B), _pitch(B),
                                             opB | (GEMM_POW2_SCALES if pow2_scales else 0) | ob, _ptr(sB), bscale_mode,
                                             _ptr(C), _pitch(C), ws_ptr, ws_bytes, _stream()),
           "gemm_fp8_blockscaled")
    return C


def gemm_fp8_blockscaled_noalloc(A, sA, B, sB, C, opB: int = OP_N, bscale_mode: int = BSCALE_BLOCK128,
                                 pow2_scales: bool = False):
    """The dense GEMM through fp8blk_gemm_fp8_blockscaled_noalloc: C (float32
    or bfloat16) given by the caller; split-K partials in the library's own
    per-device scratch array, so the call allocates nothing."""
    M, K = A.shape
    N = B.shape[1] if opB == OP_N else B.shape[0]
    ob, _, _ = _out_flag(C, C.dtype)
    _check(lib().fp8blk_gemm_fp8_blockscaled_noalloc(M, N, K, _ptr(A), _pitch(A), _ptr(sA), _ptr(B), _pitch(B),
                                                     opB | (GEMM_POW2_SCALES if pow2_scales else 0) | ob, _ptr(sB),
                                                     bscale_mode, _ptr(C), _pitch(C), _stream()),
           "gemm_fp8_blockscaled_noalloc")
    return C


def gemm_fp8_blockscaled_q1x128(A, sA, B, sB, opB: int = OP_N, pow2_scales: bool = False, pow2: bool = False,
                                Q=None, sQ=None):
    """Block-scaled GEMM (block-scaled B) whose output is quantized on store:
    returns (Q uint8 [M][N], sQ float32 [ceil(N/128)][M]) = quantize_1x128 of
    the BF16-rounded product, with power-of-two scales when pow2."""
    M, K = A.shape
    N = B.shape[1] if opB == OP_N else B.shape[0]
    Q = _empty_pitched(M, N, torch.uint8, A.device, 1) if Q is None else Q
    sQ = torch.empty((N + 127) // 128, M, dtype=torch.float32, device=A.device) if sQ is None else sQ
    _check(lib().fp8blk_gemm_fp8_blockscaled_q1x128(
        M, N, K, _ptr(A), _pitch(A), _ptr(sA), _ptr(B), _pitch(B), opB | (GEMM_POW2_SCALES if pow2_scales else 0),
        _ptr(sB), _ptr(Q), _pitch(Q), _ptr(sQ), SCALE_POW2 if pow2 else 0, _stream()), "gemm_fp8_blockscaled_q1x128")
    return Q, sQ


def grouped_gemm_fp8_blockscaled(offsets, A, sA, B, sB, opB: int = OP_N, max_group_rows=None, C=None,
                                 pow2_scales: bool = False, out_dtype=torch.float32):
    """Per-expert GEMM.  offsets: device int32 [G+1]; A [M_total][K];
    B [G][K][N] (OP_N) or [G][N][K] (OP_T) contiguous per expert; sB [G][...]."""
    G = offsets.numel() - 1
    M, K = A.shape
    N = B.shape[2] if opB == OP_N else B.shape[1]
    assert offsets.dtype == torch.int32 and offsets.is_cuda
    assert B.dim() == 3 and B.stride(2) == 1
    ob, odt, oel = _out_flag(C, out_dtype)
    C = _empty_pitched(M, N, odt, A.device, oel) if C is None else C
    mgr = M if max_group_rows is None else int(max_group_rows)
    _check(lib().fp8blk_grouped_gemm_fp8_blockscaled(
        G, _ptr(offsets), M, mgr, N, K, _ptr(A), _pitch(A), _ptr(sA), _ptr(B), B.stride(1), B.stride(0),
        opB | (GEMM_POW2_SCALES if pow2_scales else 0) | ob,
        _ptr(sB), sB.stride(0), _ptr(C), _pitch(C), None, 0, _stream()), "grouped_gemm_fp8_blockscaled")
    return C


def token_group_slots(T: int, G: int) -> int:
    """Group slots to allocate for T tokens split into G experts (T//128 + G)."""
    return lib().fp8blk_token_group_slots(T, G)


def quantize_128x1_grouped(x: torch.Tensor, offsets: torch.Tensor, pow2: bool = False, qT=None, s=None):
    """MoE Wgrad operand: x [T][C] bf16 (tokens in expert order), offsets
    device int32 [G+1] -> (qT uint8 [C][128*S], s float32 [S][C]) with
    S = token_group_slots(T, G); expert e's token j is column 128*PG[e] + j,
    PG[e] = sum of ceil(M_e'/128) over e' < e (see the header)."""
    x = _bf16_bits(x)
    T, C = x.shape
    G = offsets.numel() - 1
    assert offsets.dtype == torch.int32 and offsets.is_cuda
    S = token_group_slots(T, G)
    qT = _empty_pitched(C, 128 * S, torch.uint8, x.device, 1) if qT is None else qT
    s = torch.empty(S, C, dtype=torch.float32, device=x.device) if s is None else s
    _check(lib().fp8blk_quantize_128x1_grouped(_ptr(x), T, C, _pitch(x), G, _ptr(offsets), _ptr(qT), _pitch(qT),
                                               _ptr(s), SCALE_POW2 if pow2 else 0, _stream()),
           "quantize_128x1_grouped")
    return qT, s


def grouped_wgrad_fp8_blockscaled(offsets: torch.Tensor, T: int, AT, sA, BT, sB, C=None, pow2_scales: bool = False,
                                  out_dtype=torch.float32):
    """MoE grouped Wgrad: dW_e = X_e^T dY_e for every expert from the outputs
    of quantize_128x1_grouped of X (AT [M][128*S], sA) and of dY (BT
    [N][128*S], sB) with the same offsets and T.  Returns C float32 [G][M][N]."""
    G = offsets.numel() - 1
    assert offsets.dtype == torch.int32 and offsets.is_cuda
    M, N = AT.shape[0], BT.shape[0]
    ob, odt, oel = _out_flag(C, out_dtype)
    if C is None:
        C = torch.empty(G, M, _pad16(N, oel), dtype=odt, device=AT.device)[:, :, :N]
    assert C.dim() == 3 and C.stride(2) == 1
    _check(lib().fp8blk_grouped_wgrad_fp8_blockscaled(
        G, _ptr(offsets), T, M, N, _ptr(AT), _pitch(AT), _ptr(sA), _ptr(BT), _pitch(BT), _ptr(sB),
        (GEMM_POW2_SCALES if pow2_scales else 0) | ob, _ptr(C), C.stride(1), C.stride(0), _stream()),
        "grouped_wgrad_fp8_blockscaled")
    return C
