"""Thin ctypes binding of libdg (include/dg.h), with the same call names.

Argument marshalling only: tensors are checked for dtype, shape, device and
contiguity, their device pointers and the current HIP stream are passed through, and a
non-zero status raises ``DGError``.  All arithmetic runs in libdg's HIP kernels; there
is no fallback, and a missing library raises at load time.
"""
from __future__ import annotations

import ctypes
import os
import threading

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libdg.so")

DG_DENSE, DG_CONTIGUOUS, DG_MASKED = 0, 1, 2
DG_FP8_E4M3, DG_FP8_E5M2 = 0, 1
_FORMATS = {"e4m3": DG_FP8_E4M3, "e5m2": DG_FP8_E5M2}
_FP8_DTYPES = {torch.float8_e4m3fn: DG_FP8_E4M3, torch.float8_e5m2: DG_FP8_E5M2}
_lib = None
_lock = threading.Lock()
_workspaces: dict = {}


class DGError(RuntimeError):
    def __init__(self, status: int, call: str):
        self.status = status
        super().__init__(f"{call} failed: {dg_status_string(status)} ({status})")


def load_library():
    """Load libdg.so from the package directory (raises if it was not built)."""
    global _lib
    if _lib is not None:
        return _lib
    with _lock:
        if _lib is not None:
            return _lib
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -m moe_grouped_gemm_lhs_amd.build`")
        lib = ctypes.CDLL(LIB_PATH)
        P, I64, SZ, I = ctypes.c_void_p, ctypes.c_int64, ctypes.c_size_t, ctypes.c_int
        lib.dg_get_m_alignment_for_contiguous_layout.restype = I
        lib.dg_get_m_alignment_for_contiguous_layout.argtypes = []
        lib.dg_status_string.restype = ctypes.c_char_p
        lib.dg_status_string.argtypes = [I]
        lib.dg_workspace_bytes.restype = SZ
        lib.dg_workspace_bytes.argtypes = [I, I64, I64, I64, I64]
        lib.dg_instance_name.restype = ctypes.c_char_p
        lib.dg_instance_name.argtypes = [I, I64, I64, I64, I64]
        lib.dg_gemm_fp8_nt.restype = I
        lib.dg_gemm_fp8_nt.argtypes = [P, P, P, P, P, I64, I64, I64, P, SZ, P]
        lib.dg_grouped_gemm_fp8_contiguous.restype = I
        lib.dg_grouped_gemm_fp8_contiguous.argtypes = [P, P, P, P, P, P, I64, I64, I64, I64,
                                                       P, SZ, P]
        lib.dg_grouped_gemm_fp8_masked.restype = I
        lib.dg_grouped_gemm_fp8_masked.argtypes = [P, P, P, P, P, P, I64, I64, I64, I64,
                                                   P, SZ, P]
        lib.dg_gemm_fp8_nt_noalloc.restype = I
        lib.dg_gemm_fp8_nt_noalloc.argtypes = [P, P, P, P, P, I64, I64, I64, P]
        lib.dg_gemm_fp8_nt_ex.restype = I
        lib.dg_gemm_fp8_nt_ex.argtypes = [P, I, P, P, I, P, P, I64, I64, I64, P, SZ, P]
        lib.dg_grouped_gemm_fp8_contiguous_ex.restype = I
        lib.dg_grouped_gemm_fp8_contiguous_ex.argtypes = [P, I, P, P, I, P, P, P, I64, I64, I64,
                                                          I64, P, SZ, P]
        lib.dg_quantize_fp8_1x128.restype = I
        lib.dg_quantize_fp8_1x128.argtypes = [P, I, P, P, I64, I64, I, P]
        lib.dg_quantize_fp8_128x128.restype = I
        lib.dg_quantize_fp8_128x128.argtypes = [P, I, P, P, I64, I64, I, P]
        lib.dg_transpose_fp8.restype = I
        lib.dg_transpose_fp8.argtypes = [P, P, I64, I64, P]
        lib.dg_grouped_gemm_fp8_masked_ex.restype = I
        lib.dg_grouped_gemm_fp8_masked_ex.argtypes = [P, I, P, P, I, P, P, P, I64, I64, I64,
                                                      I64, P, SZ, P]
        _lib = lib
    return _lib


def dg_get_m_alignment_for_contiguous_layout() -> int:
    return int(load_library().dg_get_m_alignment_for_contiguous_layout())


def dg_status_string(status: int) -> str:
    return load_library().dg_status_string(int(status)).decode()


def dg_workspace_bytes(kind: int, rows_or_cap: int, N: int, K: int, G: int = 1) -> int:
    return int(load_library().dg_workspace_bytes(kind, rows_or_cap, N, K, G))


def dg_instance_name(kind: int, rows_or_cap: int, N: int, K: int, G: int = 1) -> str:
    return load_library().dg_instance_name(kind, rows_or_cap, N, K, G).decode()


# ------------------------------------------------------------------------ marshalling
def _bytes_view(t: torch.Tensor, name: str, fmt=None):
    """The operand as uint8 bytes and its format code: float8_e4m3fn / float8_e5m2
    tensors carry their format; uint8 bytes are E4M3 unless `fmt` ('e4m3' / 'e5m2')
    says otherwise."""
    if fmt is not None and fmt not in _FORMATS:
        raise ValueError(f"{name}: unknown operand format {fmt!r}")
    if t.dtype in _FP8_DTYPES:
        code = _FP8_DTYPES[t.dtype]
        if fmt is not None and _FORMATS[fmt] != code:
            raise ValueError(f"{name}: format {fmt!r} contradicts dtype {t.dtype}")
        return t.view(torch.uint8), code
    if t.dtype != torch.uint8:
        raise TypeError(f"{name} must be uint8, float8_e4m3fn or float8_e5m2, got {t.dtype}")
    return t, _FORMATS[fmt or "e4m3"]


def _check(t: torch.Tensor, name: str, dtype, shape, device):
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if t.device != device:
        raise ValueError(f"{name} must be on {device}, got {t.device}")


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else None


def _stream(device, stream):
    """The launch stream as the hipStream_t handle the C calls take."""
    return ctypes.c_void_p(_launch_stream(device, stream).cuda_stream)


def _launch_stream(device, stream):
    """The stream the call runs on: the one given, else the device's current stream."""
    return stream if stream is not None else torch.cuda.current_stream(device)


def _workspace(kind, rows, N, K, G, device, workspace, stream):
    """The caller's workspace, or one kept per (device, launch stream): allocated and
    zero filled on the launch stream, so the fill is ordered before the call and calls
    on different streams never share one (every call leaves it zero filled again).
    Under graph capture each call gets a fresh one from the graph's memory, zero filled
    by a kernel inside the graph."""
    need = dg_workspace_bytes(kind, rows, N, K, G)
    if workspace is not None:
        return workspace, workspace.numel() * workspace.element_size()
    if need == 0:
        return None, 0
    with torch.cuda.stream(stream):
        if torch.cuda.is_current_stream_capturing():
            ws = torch.zeros(need, dtype=torch.uint8, device=device)
            return ws, ws.numel()
        key = (device.index, stream.cuda_stream)
        with _lock:
            ws = _workspaces.get(key)
            if ws is None or ws.numel() < need:
                # the previous one was used on this stream only, so the allocator may
                # hand its memory out again in this stream's order
                ws = torch.zeros(need, dtype=torch.uint8, device=device)
                _workspaces[key] = ws
    return ws, ws.numel()


def dg_gemm_fp8_nt(A, sA, B, sB, C=None, *, a_format=None, b_format=None, workspace=None,
                   stream=None):
    """Dense C (M x N bf16) = A (M x K fp8) x B (N x K fp8)^T with block scales.  The
    operand formats come from float8 dtypes, or a_format / b_format ('e4m3', 'e5m2')
    for uint8 bytes (default E4M3); any non-E4M3 operand goes through the _ex call."""
    (A, fa), (B, fb) = _bytes_view(A, "A", a_format), _bytes_view(B, "B", b_format)
    M, K = A.shape
    N = B.shape[0]
    dev = A.device
    nkb, nnb = -(-K // 128), -(-N // 128)
    _check(A, "A", torch.uint8, (M, K), dev)
    _check(B, "B", torch.uint8, (N, K), dev)
    _check(sA, "sA", torch.float32, (M, nkb), dev)
    _check(sB, "sB", torch.float32, (nnb, nkb), dev)
    if C is None:
        C = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
    _check(C, "C", torch.bfloat16, (M, N), dev)
    st_ = _launch_stream(dev, stream)
    ws, wsb = _workspace(DG_DENSE, M, N, K, 1, dev, workspace, st_)
    lib = load_library()
    if fa == DG_FP8_E4M3 and fb == DG_FP8_E4M3:
        st = lib.dg_gemm_fp8_nt(_ptr(A), _ptr(sA), _ptr(B), _ptr(sB), _ptr(C), M, N, K,
                                _ptr(ws), wsb, ctypes.c_void_p(st_.cuda_stream))
    else:
        st = lib.dg_gemm_fp8_nt_ex(_ptr(A), fa, _ptr(sA), _ptr(B), fb, _ptr(sB), _ptr(C), M, N,
                                   K, _ptr(ws), wsb, ctypes.c_void_p(st_.cuda_stream))
    if st != 0:
        raise DGError(st, "dg_gemm_fp8_nt")
    return C


def dg_gemm_fp8_nt_noalloc(A, sA, B, sB, C=None, *, stream=None):
    """dg_gemm_fp8_nt without a workspace argument: split-K calls use the library's
    static per-GPU workspace (calls that overlap on one GPU race).  E4M3 operands."""
    (A, fa), (B, fb) = _bytes_view(A, "A"), _bytes_view(B, "B")
    if fa != DG_FP8_E4M3 or fb != DG_FP8_E4M3:
        raise ValueError("dg_gemm_fp8_nt_noalloc takes E4M3 operands")
    M, K = A.shape
    N = B.shape[0]
    dev = A.device
    nkb, nnb = -(-K // 128), -(-N // 128)
    _check(A, "A", torch.uint8, (M, K), dev)
    _check(B, "B", torch.uint8, (N, K), dev)
    _check(sA, "sA", torch.float32, (M, nkb), dev)
    _check(sB, "sB", torch.float32, (nnb, nkb), dev)
    if C is None:
        C = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
    _check(C, "C", torch.bfloat16, (M, N), dev)
    st = load_library().dg_gemm_fp8_nt_noalloc(_ptr(A), _ptr(sA), _ptr(B), _ptr(sB), _ptr(C),
                                               M, N, K, _stream(dev, stream))
    if st != 0:
        raise DGError(st, "dg_gemm_fp8_nt_noalloc")
    return C


def dg_grouped_gemm_fp8_contiguous(A, sA, B, sB, group_idx, C=None, *, a_format=None,
                                   b_format=None, workspace=None, stream=None):
    """Contiguous grouped GEMM: A (M_total x K), B (G x N x K), group_idx (M_total int32);
    operand formats as for dg_gemm_fp8_nt."""
    (A, fa), (B, fb) = _bytes_view(A, "A", a_format), _bytes_view(B, "B", b_format)
    M, K = A.shape
    G, N = B.shape[0], B.shape[1]
    dev = A.device
    nkb, nnb = -(-K // 128), -(-N // 128)
    _check(A, "A", torch.uint8, (M, K), dev)
    _check(B, "B", torch.uint8, (G, N, K), dev)
    _check(sA, "sA", torch.float32, (M, nkb), dev)
    _check(sB, "sB", torch.float32, (G, nnb, nkb), dev)
    _check(group_idx, "group_idx", torch.int32, (M,), dev)
    if C is None:
        C = torch.zeros((M, N), dtype=torch.bfloat16, device=dev)
    _check(C, "C", torch.bfloat16, (M, N), dev)
    st_ = _launch_stream(dev, stream)
    ws, wsb = _workspace(DG_CONTIGUOUS, M, N, K, G, dev, workspace, st_)
    lib = load_library()
    if fa == DG_FP8_E4M3 and fb == DG_FP8_E4M3:
        st = lib.dg_grouped_gemm_fp8_contiguous(
            _ptr(A), _ptr(sA), _ptr(B), _ptr(sB), _ptr(group_idx), _ptr(C), M, N, K, G,
            _ptr(ws), wsb, ctypes.c_void_p(st_.cuda_stream))
    else:
        st = lib.dg_grouped_gemm_fp8_contiguous_ex(
            _ptr(A), fa, _ptr(sA), _ptr(B), fb, _ptr(sB), _ptr(group_idx), _ptr(C), M, N, K, G,
            _ptr(ws), wsb, ctypes.c_void_p(st_.cuda_stream))
    if st != 0:
        raise DGError(st, "dg_grouped_gemm_fp8_contiguous")
    return C


def dg_grouped_gemm_fp8_masked(A, sA, B, sB, masked_m, C=None, *, a_format=None,
                               b_format=None, workspace=None, stream=None):
    """Masked grouped GEMM: A (G x cap x K), B (G x N x K), masked_m (G int32); operand
    formats as for dg_gemm_fp8_nt."""
    (A, fa), (B, fb) = _bytes_view(A, "A", a_format), _bytes_view(B, "B", b_format)
    G, cap, K = A.shape
    N = B.shape[1]
    dev = A.device
    nkb, nnb = -(-K // 128), -(-N // 128)
    _check(A, "A", torch.uint8, (G, cap, K), dev)
    _check(B, "B", torch.uint8, (G, N, K), dev)
    _check(sA, "sA", torch.float32, (G, cap, nkb), dev)
    _check(sB, "sB", torch.float32, (G, nnb, nkb), dev)
    _check(masked_m, "masked_m", torch.int32, (G,), dev)
    if C is None:
        C = torch.zeros((G, cap, N), dtype=torch.bfloat16, device=dev)
    _check(C, "C", torch.bfloat16, (G, cap, N), dev)
    st_ = _launch_stream(dev, stream)
    ws, wsb = _workspace(DG_MASKED, cap, N, K, G, dev, workspace, st_)
    lib = load_library()
    if fa == DG_FP8_E4M3 and fb == DG_FP8_E4M3:
        st = lib.dg_grouped_gemm_fp8_masked(
            _ptr(A), _ptr(sA), _ptr(B), _ptr(sB), _ptr(masked_m), _ptr(C), G, cap, N, K,
            _ptr(ws), wsb, ctypes.c_void_p(st_.cuda_stream))
    else:
        st = lib.dg_grouped_gemm_fp8_masked_ex(
            _ptr(A), fa, _ptr(sA), _ptr(B), fb, _ptr(sB), _ptr(masked_m), _ptr(C), G, cap, N,
            K, _ptr(ws), wsb, ctypes.c_void_p(st_.cuda_stream))
    if st != 0:
        raise DGError(st, "dg_grouped_gemm_fp8_masked")
    return C


DG_IN_F32, DG_IN_BF16 = 0, 1
_IN_DTYPES = {torch.float32: DG_IN_F32, torch.bfloat16: DG_IN_BF16}
_FP8_OF = {"e4m3": torch.float8_e4m3fn, "e5m2": torch.float8_e5m2}


def _quantize(call, X, fmt, scale_rows, Q, S, stream):
    if fmt not in _FORMATS:
        raise ValueError(f"unknown fp8 format {fmt!r}")
    if X.dtype not in _IN_DTYPES:
        raise TypeError(f"X must be float32 or bfloat16, got {X.dtype}")
    if X.dim() != 2:
        raise ValueError("X must be 2-D (rows x K)")
    rows, K = X.shape
    dev = X.device
    if not X.is_contiguous():
        raise ValueError("X must be contiguous")
    if Q is None:
        Q = torch.empty((rows, K), dtype=torch.uint8, device=dev)
    Qb = Q.view(torch.uint8) if Q.dtype in _FP8_DTYPES else Q
    _check(Qb, "Q", torch.uint8, (rows, K), dev)
    if S is None:
        S = torch.empty((scale_rows, K // 128), dtype=torch.float32, device=dev)
    _check(S, "S", torch.float32, (scale_rows, K // 128), dev)
    st = getattr(load_library(), call)(_ptr(X), _IN_DTYPES[X.dtype], _ptr(Qb), _ptr(S), rows,
                                       K, _FORMATS[fmt], _stream(dev, stream))
    if st != 0:
        raise DGError(st, call)
    return Qb.view(_FP8_OF[fmt]), S


def dg_quantize_fp8_1x128(X, fmt="e4m3", Q=None, S=None, *, stream=None):
    """Per-row 1x128 quantisation of X (rows x K, float32 or bfloat16) to fp8 ('e4m3' or
    'e5m2').  Returns (Q rows x K as a float8 tensor, S rows x K/128 float32)."""
    return _quantize("dg_quantize_fp8_1x128", X, fmt, X.shape[0], Q, S, stream)


def dg_quantize_fp8_128x128(X, fmt="e4m3", Q=None, S=None, *, stream=None):
    """128x128-block quantisation of X (rows x K, float32 or bfloat16) to fp8.  Returns
    (Q rows x K as a float8 tensor, S ceil(rows/128) x K/128 float32)."""
    return _quantize("dg_quantize_fp8_128x128", X, fmt, -(-X.shape[0] // 128), Q, S, stream)


def dg_transpose_fp8(X, Y=None, *, stream=None):
    """Y (cols x rows) = X (rows x cols)^T for a byte / fp8 matrix on the GPU (rows and
    cols multiples of 16).  Y keeps X's dtype."""
    if X.dim() != 2:
        raise ValueError("X must be 2-D")
    Xb = X.view(torch.uint8) if X.dtype in _FP8_DTYPES else X
    if Xb.dtype != torch.uint8:
        raise TypeError(f"X must be uint8 or float8, got {X.dtype}")
    rows, cols = Xb.shape
    dev = Xb.device
    _check(Xb, "X", torch.uint8, (rows, cols), dev)
    if Y is None:
        Y = torch.empty((cols, rows), dtype=X.dtype, device=dev)
    Yb = Y.view(torch.uint8) if Y.dtype in _FP8_DTYPES else Y
    _check(Yb, "Y", torch.uint8, (cols, rows), dev)
    st = load_library().dg_transpose_fp8(_ptr(Xb), _ptr(Yb), rows, cols, _stream(dev, stream))
    if st != 0:
        raise DGError(st, "dg_transpose_fp8")
    return Y


def group_sizes_to_idx(sizes, device=None) -> torch.Tensor:
    """Per-row int32 group index of contiguous segments of the given sizes."""
    sizes = torch.as_tensor(list(sizes), dtype=torch.int64)
    idx = torch.repeat_interleave(torch.arange(len(sizes), dtype=torch.int32), sizes)
    return idx.to(device) if device is not None else idx
