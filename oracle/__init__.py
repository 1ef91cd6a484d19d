"""CPU oracle for the FP8 block-scaled NT GEMM -- TEST INFRASTRUCTURE ONLY.

Only the tests, the smoke check and the benchmark's CPU-baseline leg may import this
package.  The GPU library never links, loads or calls it, and the two share no code.

The arithmetic lives in ``dgref.c`` (plain C, fp64, OpenMP over output rows); this
module builds it with gcc when needed and marshals NumPy arrays through ctypes.
Every function returns bf16 results as uint16 bit patterns.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "dgref.c")
_LIB = os.path.join(_HERE, "libdgref.so")
_lib = None


def build(force: bool = False) -> str:
    """Compile dgref.c into libdgref.so (gcc, -O2, OpenMP, no FP contraction)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + f".tmp{os.getpid()}"
        subprocess.check_call(["gcc", "-O2", "-fopenmp", "-ffp-contract=off", "-fno-fast-math",
                               "-fPIC", "-shared", "-std=c99", "-Wall", _SRC, "-o", tmp, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is None:
        lib = ctypes.CDLL(build())
        P = ctypes.c_void_p
        I64 = ctypes.c_int64
        lib.dgref_e4m3fn_decode.restype = ctypes.c_double
        lib.dgref_e4m3fn_decode.argtypes = [ctypes.c_uint8]
        lib.dgref_bf16_rne.restype = ctypes.c_uint16
        lib.dgref_bf16_rne.argtypes = [ctypes.c_double]
        lib.dgref_threads.restype = ctypes.c_int
        I = ctypes.c_int
        lib.dgref_gemm_fp8_nt_fmt.restype = I
        lib.dgref_gemm_fp8_nt_fmt.argtypes = [P, I, P, P, I, P, P, P, I64, I64, I64]
        lib.dgref_grouped_contiguous_fmt.restype = I
        lib.dgref_grouped_contiguous_fmt.argtypes = [P, I, P, P, I, P, P, P, P, I64, I64, I64,
                                                     I64]
        lib.dgref_grouped_masked_fmt.restype = I
        lib.dgref_grouped_masked_fmt.argtypes = [P, I, P, P, I, P, P, P, P, I64, I64, I64, I64]
        lib.dgref_bf16_rne_array.argtypes = [P, P, I64]
        lib.dgref_e4m3fn_decode_array.argtypes = [P, P, I64]
        lib.dgref_e5m2_decode_array.argtypes = [P, P, I64]
        lib.dgref_encode_fp8_array.argtypes = [P, P, I64, I]
        lib.dgref_quantize_1x128.restype = I
        lib.dgref_quantize_1x128.argtypes = [P, I64, I64, I, P, P]
        lib.dgref_quantize_128x128.restype = I
        lib.dgref_quantize_128x128.argtypes = [P, I64, I64, I, P, P]
        _lib = lib
    return _lib


def _p(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _c(a, dtype):
    a = np.ascontiguousarray(a, dtype=dtype)
    return a


def threads() -> int:
    return int(_load().dgref_threads())


def decode_e4m3fn(codes) -> np.ndarray:
    codes = _c(codes, np.uint8)
    out = np.empty(codes.shape, dtype=np.float64)
    _load().dgref_e4m3fn_decode_array(_p(codes), _p(out), codes.size)
    return out


def decode_e5m2(codes) -> np.ndarray:
    codes = _c(codes, np.uint8)
    out = np.empty(codes.shape, dtype=np.float64)
    _load().dgref_e5m2_decode_array(_p(codes), _p(out), codes.size)
    return out


FORMATS = {"e4m3": 0, "e5m2": 1}


def _fmt(f) -> int:
    """Operand format: 'e4m3' (E4M3, the default) or 'e5m2'."""
    if f not in FORMATS:
        raise ValueError(f"unknown operand format {f!r}")
    return FORMATS[f]


def bf16_rne(x) -> np.ndarray:
    x = _c(x, np.float64)
    out = np.empty(x.shape, dtype=np.uint16)
    _load().dgref_bf16_rne_array(_p(x), _p(out), x.size)
    return out


def _prep_out(C, shape, want_acc):
    if C is None:
        C = np.zeros(shape, dtype=np.uint16)
    else:
        assert C.dtype == np.uint16 and C.flags.c_contiguous and C.shape == tuple(shape)
    acc = np.full(shape, np.nan, dtype=np.float64) if want_acc else None
    return C, acc


def gemm_fp8_nt(A, sA, B, sB, C=None, want_acc=False, a_fmt="e4m3", b_fmt="e4m3"):
    """Dense NT GEMM.  A: M x K uint8, sA: M x ceil(K/128) f32, B: N x K uint8,
    sB: ceil(N/128) x ceil(K/128) f32; a_fmt / b_fmt: 'e4m3' or 'e5m2' codes.
    Returns C (M x N bf16 bits)[, fp64 values]."""
    A, B = _c(A, np.uint8), _c(B, np.uint8)
    sA, sB = _c(sA, np.float32), _c(sB, np.float32)
    M, K = A.shape
    N = B.shape[0]
    nkb = -(-K // 128)
    assert B.shape[1] == K and sA.shape == (M, nkb) and sB.shape == (-(-N // 128), nkb)
    C, acc = _prep_out(C, (M, N), want_acc)
    _load().dgref_gemm_fp8_nt_fmt(_p(A), _fmt(a_fmt), _p(sA), _p(B), _fmt(b_fmt), _p(sB),
                                  _p(C), _p(acc), M, N, K)
    return (C, acc) if want_acc else C


def grouped_contiguous(A, sA, B, sB, group_idx, G, C=None, want_acc=False, a_fmt="e4m3",
                       b_fmt="e4m3"):
    """Contiguous grouped NT GEMM.  A: M_total x K, B: G*N x K (G stacked N x K),
    sB: G*ceil(N/128) x ceil(K/128), group_idx: M_total int32."""
    A, B = _c(A, np.uint8), _c(B, np.uint8)
    sA, sB = _c(sA, np.float32), _c(sB, np.float32)
    gi = _c(group_idx, np.int32)
    M, K = A.shape
    N = B.shape[0] // G
    nkb = -(-K // 128)
    assert B.shape == (G * N, K) and sA.shape == (M, nkb) and gi.shape == (M,)
    assert sB.shape == (G * -(-N // 128), nkb)
    C, acc = _prep_out(C, (M, N), want_acc)
    _load().dgref_grouped_contiguous_fmt(_p(A), _fmt(a_fmt), _p(sA), _p(B), _fmt(b_fmt), _p(sB),
                                         _p(gi), _p(C), _p(acc), M, N, K, G)
    return (C, acc) if want_acc else C


def grouped_masked(A, sA, B, sB, masked_m, G, cap, C=None, want_acc=False, a_fmt="e4m3",
                   b_fmt="e4m3"):
    """Masked grouped NT GEMM.  A: G*cap x K, B: G*N x K, masked_m: G int32.
    C: G*cap x N; rows past masked_m[g] keep whatever C held."""
    A, B = _c(A, np.uint8), _c(B, np.uint8)
    sA, sB = _c(sA, np.float32), _c(sB, np.float32)
    mm = _c(masked_m, np.int32)
    K = A.shape[1]
    N = B.shape[0] // G
    nkb = -(-K // 128)
    assert A.shape == (G * cap, K) and B.shape == (G * N, K) and mm.shape == (G,)
    assert sA.shape == (G * cap, nkb) and sB.shape == (G * -(-N // 128), nkb)
    C, acc = _prep_out(C, (G * cap, N), want_acc)
    _load().dgref_grouped_masked_fmt(_p(A), _fmt(a_fmt), _p(sA), _p(B), _fmt(b_fmt), _p(sB),
                                     _p(mm), _p(C), _p(acc), G, cap, N, K)
    return (C, acc) if want_acc else C


def encode_fp8(x, fmt: str = "e4m3") -> np.ndarray:
    """Nearest fp8 code of each (finite) value, ties to even, saturating."""
    x = _c(x, np.float64)
    out = np.empty(x.shape, dtype=np.uint8)
    _load().dgref_encode_fp8_array(_p(x), _p(out), x.size, _fmt(fmt))
    return out


def _as_f32(X):
    """fp32 values of an fp32 array, or of bf16 bit patterns (uint16), exactly."""
    X = np.asarray(X)
    if X.dtype == np.uint16:
        return np.ascontiguousarray((X.astype(np.uint32) << 16).view(np.float32))
    return _c(X, np.float32)


def quantize_1x128(X, fmt: str = "e4m3"):
    """Per-row 1x128 quantisation of rows x K values (fp32, or bf16 bits as uint16).
    Returns (codes uint8 rows x K, scales f32 rows x K/128)."""
    X = _as_f32(X)
    rows, K = X.shape
    Q = np.empty((rows, K), np.uint8)
    S = np.empty((rows, K // 128), np.float32)
    if _load().dgref_quantize_1x128(_p(X), rows, K, _fmt(fmt), _p(Q), _p(S)) != 0:
        raise ValueError("K must be a multiple of 128")
    return Q, S


def quantize_128x128(X, fmt: str = "e4m3"):
    """128x128-block quantisation of rows x K values (fp32, or bf16 bits as uint16).
    Returns (codes uint8 rows x K, scales f32 ceil(rows/128) x K/128)."""
    X = _as_f32(X)
    rows, K = X.shape
    Q = np.empty((rows, K), np.uint8)
    S = np.empty((-(-rows // 128), K // 128), np.float32)
    if _load().dgref_quantize_128x128(_p(X), rows, K, _fmt(fmt), _p(Q), _p(S)) != 0:
        raise ValueError("K must be a multiple of 128")
    return Q, S
