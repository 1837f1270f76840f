"""CPU oracle for the tiled dense GEMM -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  The GPU library never does, and this
package imports nothing from it: the two share no code.

The arithmetic lives in ``oracle.c`` (plain C, binary64, sequential k order,
one round-to-nearest-even to the output type).  This module only builds that
file with gcc, loads it with ctypes and moves numpy arrays in and out.

What each function computes and which passage of the pages it follows is
stated in ``oracle.c``.  Parity status of every function is pinned by the
``-m "not gpu"`` tests (closed forms, brute force with exact rationals,
invariants, numpy float64 cross-checks); none is "parity unpinned".
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

_lib = None


def build(verbose: bool = False) -> str:
    """Compile oracle.c into liboracle.so with gcc (no fast-math: k order is fixed)."""
    cmd = ["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c11",
           "-Wall", "-Wextra", "-o", _LIB + ".tmp", _SRC, "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(_LIB + ".tmp", _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB):
        build()
    lib = ctypes.CDLL(_LIB)
    i64, u16p, u8p, f64p, i64p = (ctypes.c_int64, ctypes.c_void_p, ctypes.c_void_p,
                                  ctypes.c_void_p, ctypes.c_void_p)
    for name in ("oracle_gemm_bf16_nt", "oracle_gemm_f16_nn"):
        getattr(lib, name).argtypes = [i64, i64, i64, u16p, u16p, u16p, f64p]
        getattr(lib, name).restype = None
    lib.oracle_gemm_mxfp8_nt.argtypes = [i64, i64, i64, u8p, u8p, u8p, u8p, u16p, f64p]
    lib.oracle_gemm_mxfp8_nt.restype = None
    for name in ("oracle_gemm_bf16_nt_at", "oracle_gemm_f16_nn_at"):
        getattr(lib, name).argtypes = [i64, i64, i64, u16p, u16p, i64, i64p, i64p, u16p, f64p]
        getattr(lib, name).restype = None
    lib.oracle_gemm_mxfp8_nt_at.argtypes = [i64, i64, i64, u8p, u8p, u8p, u8p,
                                            i64, i64p, i64p, u16p, f64p]
    lib.oracle_gemm_mxfp8_nt_at.restype = None
    for name in ("oracle_decode_bf16", "oracle_decode_f16"):
        getattr(lib, name).argtypes = [i64, u16p, f64p]
    for name in ("oracle_decode_e4m3fn", "oracle_decode_e8m0"):
        getattr(lib, name).argtypes = [i64, u8p, f64p]
    for name in ("oracle_encode_bf16", "oracle_encode_f16"):
        getattr(lib, name).argtypes = [i64, f64p, u16p]
    lib.oracle_encode_e4m3fn.argtypes = [i64, f64p, u8p]
    lib.oracle_decode_e2m1.argtypes = [i64, u8p, f64p]
    lib.oracle_gemm_mxfp4_nt.argtypes = [i64, i64, i64, u8p, u8p, u8p, u8p, u16p, f64p]
    lib.oracle_gemm_mxfp4_nt.restype = None
    lib.oracle_gemm_mxfp4_nt_at.argtypes = [i64, i64, i64, u8p, u8p, u8p, u8p, i64, i64p, i64p, u16p, f64p]
    lib.oracle_gemm_mxfp4_nt_at.restype = None
    lib.oracle_decode_fp6.argtypes = [i64, u8p, ctypes.c_int, f64p]
    lib.oracle_decode_fp6.restype = None
    lib.oracle_unpack_fp6.argtypes = [i64, i64, i64, u8p, u8p]
    lib.oracle_unpack_fp6.restype = None
    lib.oracle_gemm_mxfp6_nt.argtypes = [i64, i64, i64, ctypes.c_int, u8p, u8p, u8p, u8p, u16p, f64p]
    lib.oracle_gemm_mxfp6_nt.restype = None
    lib.oracle_gemm_mxfp6_nt_at.argtypes = [i64, i64, i64, ctypes.c_int, u8p, u8p, u8p, u8p, i64, i64p, i64p,
                                            u16p, f64p]
    lib.oracle_gemm_mxfp6_nt_at.restype = None
    lib.oracle_quantize_mxfp8.argtypes = [i64, i64, ctypes.c_void_p, u8p, u8p]
    lib.oracle_quantize_mxfp8.restype = None
    lib.oracle_num_threads.restype = ctypes.c_int
    _lib = lib
    return lib


def _ptr(a: np.ndarray | None):
    return None if a is None else a.ctypes.data


def _c(a, dtype) -> np.ndarray:
    a = np.ascontiguousarray(a)
    if a.dtype != dtype:
        raise TypeError(f"expected {np.dtype(dtype)} bit patterns, got {a.dtype}")
    return a


def num_threads() -> int:
    """OpenMP threads the oracle's parallel loops use."""
    return _load().oracle_num_threads()


# --- codecs (bit patterns <-> float64) --------------------------------------

def decode_bf16(bits) -> np.ndarray:
    bits = _c(bits, np.uint16)
    out = np.empty(bits.shape, np.float64)
    _load().oracle_decode_bf16(bits.size, _ptr(bits), _ptr(out))
    return out


def decode_f16(bits) -> np.ndarray:
    bits = _c(bits, np.uint16)
    out = np.empty(bits.shape, np.float64)
    _load().oracle_decode_f16(bits.size, _ptr(bits), _ptr(out))
    return out


def decode_e4m3fn(bits) -> np.ndarray:
    bits = _c(bits, np.uint8)
    out = np.empty(bits.shape, np.float64)
    _load().oracle_decode_e4m3fn(bits.size, _ptr(bits), _ptr(out))
    return out


def decode_e8m0(bits) -> np.ndarray:
    bits = _c(bits, np.uint8)
    out = np.empty(bits.shape, np.float64)
    _load().oracle_decode_e8m0(bits.size, _ptr(bits), _ptr(out))
    return out


def encode_bf16(x) -> np.ndarray:
    x = _c(np.asarray(x, np.float64), np.float64)
    out = np.empty(x.shape, np.uint16)
    _load().oracle_encode_bf16(x.size, _ptr(x), _ptr(out))
    return out


def encode_f16(x) -> np.ndarray:
    x = _c(np.asarray(x, np.float64), np.float64)
    out = np.empty(x.shape, np.uint16)
    _load().oracle_encode_f16(x.size, _ptr(x), _ptr(out))
    return out


def encode_e4m3fn(x) -> np.ndarray:
    """binary64 -> e4m3fn bytes, round to nearest even (|x| <= 448)."""
    x = _c(np.asarray(x, np.float64), np.float64)
    out = np.empty(x.shape, np.uint8)
    _load().oracle_encode_e4m3fn(x.size, _ptr(x), _ptr(out))
    return out


# --- block-scale quantiser -----------------------------------------------------

def quantize_mxfp8(x):
    """float32 (R, K) -> (q uint8 (R, K) e4m3fn, s uint8 (R, ceil(K/128)) e8m0):
    per row and 128-K block the smallest 2^e with absmax <= 448 * 2^e."""
    x = _c(np.asarray(x), np.float32)
    R, K = x.shape
    q = np.empty((R, K), np.uint8)
    s = np.empty((R, (K + 127) // 128), np.uint8)
    _load().oracle_quantize_mxfp8(R, K, _ptr(x), _ptr(q), _ptr(s))
    return q, s


# --- full GEMMs ---------------------------------------------------------------

def gemm_bf16_nt(A, B, want_f64: bool = False):
    """C = A . B^T; A (M,K), B (N,K) as uint16 bf16 bit patterns -> C (M,N) bf16 bits.

    With ``want_f64`` also returns the binary64 sums before rounding.
    """
    A, B = _c(A, np.uint16), _c(B, np.uint16)
    (M, K), (N, K2) = A.shape, B.shape
    if K != K2:
        raise ValueError("inner dimensions differ")
    C = np.empty((M, N), np.uint16)
    C64 = np.empty((M, N), np.float64) if want_f64 else None
    _load().oracle_gemm_bf16_nt(M, N, K, _ptr(A), _ptr(B), _ptr(C), _ptr(C64))
    return (C, C64) if want_f64 else C


def gemm_f16_nn(A, B, want_f64: bool = False):
    """C = A . B; A (M,K), B (K,N) as uint16 fp16 bit patterns -> C (M,N) fp16 bits."""
    A, B = _c(A, np.uint16), _c(B, np.uint16)
    (M, K), (K2, N) = A.shape, B.shape
    if K != K2:
        raise ValueError("inner dimensions differ")
    C = np.empty((M, N), np.uint16)
    C64 = np.empty((M, N), np.float64) if want_f64 else None
    _load().oracle_gemm_f16_nn(M, N, K, _ptr(A), _ptr(B), _ptr(C), _ptr(C64))
    return (C, C64) if want_f64 else C


def gemm_mxfp8_nt(qA, qB, sA, sB, want_f64: bool = False):
    """Block-scaled FP8 NT GEMM -> C (M,N) bf16 bits.

    qA (M,K), qB (N,K): e4m3fn bytes; sA (M,ceil(K/128)), sB (N,ceil(K/128)):
    e8m0 bytes, one per row per 128 K elements.
    """
    qA, qB, sA, sB = (_c(x, np.uint8) for x in (qA, qB, sA, sB))
    (M, K), (N, K2) = qA.shape, qB.shape
    KB = (K + 127) // 128
    if K != K2 or sA.shape != (M, KB) or sB.shape != (N, KB):
        raise ValueError("operand shapes do not match")
    C = np.empty((M, N), np.uint16)
    C64 = np.empty((M, N), np.float64) if want_f64 else None
    _load().oracle_gemm_mxfp8_nt(M, N, K, _ptr(qA), _ptr(qB), _ptr(sA), _ptr(sB),
                                 _ptr(C), _ptr(C64))
    return (C, C64) if want_f64 else C


# --- sampled GEMMs (selected outputs only) -----------------------------------

def _points(rows, cols):
    rows = np.ascontiguousarray(rows, np.int64)
    cols = np.ascontiguousarray(cols, np.int64)
    if rows.shape != cols.shape or rows.ndim != 1:
        raise ValueError("rows and cols must be equal-length 1-D arrays")
    return rows, cols


def gemm_bf16_nt_at(A, B, rows, cols, want_f64: bool = False):
    """C[rows[p], cols[p]] of C = A . B^T (bf16 bits), one output at a time."""
    A, B = _c(A, np.uint16), _c(B, np.uint16)
    (M, K), (N, K2) = A.shape, B.shape
    rows, cols = _points(rows, cols)
    if K != K2 or (rows.size and (rows.min() < 0 or rows.max() >= M or
                                  cols.min() < 0 or cols.max() >= N)):
        raise ValueError("bad shapes or sample positions")
    out = np.empty(rows.size, np.uint16)
    out64 = np.empty(rows.size, np.float64) if want_f64 else None
    _load().oracle_gemm_bf16_nt_at(M, N, K, _ptr(A), _ptr(B), rows.size,
                                   _ptr(rows), _ptr(cols), _ptr(out), _ptr(out64))
    return (out, out64) if want_f64 else out


def gemm_f16_nn_at(A, B, rows, cols, want_f64: bool = False):
    """C[rows[p], cols[p]] of C = A . B (fp16 bits), one output at a time."""
    A, B = _c(A, np.uint16), _c(B, np.uint16)
    (M, K), (K2, N) = A.shape, B.shape
    rows, cols = _points(rows, cols)
    if K != K2 or (rows.size and (rows.min() < 0 or rows.max() >= M or
                                  cols.min() < 0 or cols.max() >= N)):
        raise ValueError("bad shapes or sample positions")
    out = np.empty(rows.size, np.uint16)
    out64 = np.empty(rows.size, np.float64) if want_f64 else None
    _load().oracle_gemm_f16_nn_at(M, N, K, _ptr(A), _ptr(B), rows.size,
                                  _ptr(rows), _ptr(cols), _ptr(out), _ptr(out64))
    return (out, out64) if want_f64 else out


def gemm_mxfp8_nt_at(qA, qB, sA, sB, rows, cols, want_f64: bool = False):
    """C[rows[p], cols[p]] of the block-scaled FP8 NT GEMM (bf16 bits)."""
    qA, qB, sA, sB = (_c(x, np.uint8) for x in (qA, qB, sA, sB))
    (M, K), (N, K2) = qA.shape, qB.shape
    KB = (K + 127) // 128
    rows, cols = _points(rows, cols)
    if K != K2 or sA.shape != (M, KB) or sB.shape != (N, KB) or (
            rows.size and (rows.min() < 0 or rows.max() >= M or
                           cols.min() < 0 or cols.max() >= N)):
        raise ValueError("bad shapes or sample positions")
    out = np.empty(rows.size, np.uint16)
    out64 = np.empty(rows.size, np.float64) if want_f64 else None
    _load().oracle_gemm_mxfp8_nt_at(M, N, K, _ptr(qA), _ptr(qB), _ptr(sA), _ptr(sB),
                                    rows.size, _ptr(rows), _ptr(cols), _ptr(out),
                                    _ptr(out64))
    return (out, out64) if want_f64 else out


# --- MXFP4 ---------------------------------------------------------------------

def decode_e2m1(nibbles) -> np.ndarray:
    """FP4 E2M1 codes (0..15, one per byte) -> float64."""
    b = _c(np.asarray(nibbles, np.uint8), np.uint8)
    out = np.empty(b.shape, np.float64)
    _load().oracle_decode_e2m1(b.size, _ptr(b), _ptr(out))
    return out


def _mxfp4_shapes(qA, qB, sA, sB, K):
    (M, KH), (N, KH2) = qA.shape, qB.shape
    if K is None:
        K = 2 * KH
    KB = (K + 31) // 32
    if KH != (K + 1) // 2 or KH2 != KH or sA.shape != (M, KB) or sB.shape != (N, KB):
        raise ValueError("operand shapes do not match")
    return M, N, K


def gemm_mxfp4_nt(qA, qB, sA, sB, K=None, want_f64: bool = False):
    """Block-scaled FP4 NT GEMM -> C (M,N) bf16 bits.

    qA (M,K/2), qB (N,K/2): E2M1 elements packed two per byte (element 2i in
    the low nibble of byte i); sA (M,ceil(K/32)), sB (N,ceil(K/32)): e8m0
    bytes, one per row per 32 K elements.
    """
    qA, qB, sA, sB = (_c(x, np.uint8) for x in (qA, qB, sA, sB))
    M, N, K = _mxfp4_shapes(qA, qB, sA, sB, K)
    C = np.empty((M, N), np.uint16)
    C64 = np.empty((M, N), np.float64) if want_f64 else None
    _load().oracle_gemm_mxfp4_nt(M, N, K, _ptr(qA), _ptr(qB), _ptr(sA), _ptr(sB), _ptr(C), _ptr(C64))
    return (C, C64) if want_f64 else C


def gemm_mxfp4_nt_at(qA, qB, sA, sB, rows, cols, K=None, want_f64: bool = False):
    """C[rows[p], cols[p]] of the block-scaled FP4 NT GEMM (bf16 bits)."""
    qA, qB, sA, sB = (_c(x, np.uint8) for x in (qA, qB, sA, sB))
    M, N, K = _mxfp4_shapes(qA, qB, sA, sB, K)
    rows, cols = _points(rows, cols)
    if rows.size and (rows.min() < 0 or rows.max() >= M or cols.min() < 0 or cols.max() >= N):
        raise ValueError("bad sample positions")
    out = np.empty(rows.size, np.uint16)
    out64 = np.empty(rows.size, np.float64) if want_f64 else None
    _load().oracle_gemm_mxfp4_nt_at(M, N, K, _ptr(qA), _ptr(qB), _ptr(sA), _ptr(sB), rows.size,
                                    _ptr(rows), _ptr(cols), _ptr(out), _ptr(out64))
    return (out, out64) if want_f64 else out


# --- MXFP6 ---------------------------------------------------------------------

FP6_FORMATS = {"e2m3": 0, "e3m2": 1}


def decode_fp6(codes, fmt: str) -> np.ndarray:
    """FP6 codes (0..63, one per byte) of element type fmt ("e2m3" or
    "e3m2") -> float64."""
    b = _c(np.asarray(codes, np.uint8), np.uint8)
    out = np.empty(b.shape, np.float64)
    _load().oracle_decode_fp6(b.size, _ptr(b), FP6_FORMATS[fmt], _ptr(out))
    return out


def unpack_fp6(q, K: int) -> np.ndarray:
    """Packed FP6 rows (R, 3K/4) -> codes (R, K), as the GEMM reads them."""
    q = _c(q, np.uint8)
    R, RB = q.shape
    if K % 4 or RB != K // 4 * 3:
        raise ValueError("rows must hold 3K/4 bytes, K % 4 == 0")
    out = np.empty((R, K), np.uint8)
    _load().oracle_unpack_fp6(R, RB, K, _ptr(q), _ptr(out))
    return out


def _mxfp6_shapes(qA, qB, sA, sB, K):
    (M, RB), (N, RB2) = qA.shape, qB.shape
    if K is None:
        K = RB // 3 * 4
    KB = (K + 31) // 32
    if K % 4 or RB != K // 4 * 3 or RB2 != RB or sA.shape != (M, KB) or sB.shape != (N, KB):
        raise ValueError("operand shapes do not match")
    return M, N, K


def gemm_mxfp6_nt(qA, qB, sA, sB, fmt: str, K=None, want_f64: bool = False):
    """Block-scaled FP6 NT GEMM -> C (M,N) bf16 bits.

    qA (M,3K/4), qB (N,3K/4): FP6 elements of type fmt ("e2m3" or "e3m2")
    packed densely, element k at bits 6k .. 6k+5 of the row (little-endian);
    sA (M,ceil(K/32)), sB (N,ceil(K/32)): e8m0 bytes, one per row per 32 K.
    """
    qA, qB, sA, sB = (_c(x, np.uint8) for x in (qA, qB, sA, sB))
    M, N, K = _mxfp6_shapes(qA, qB, sA, sB, K)
    C = np.empty((M, N), np.uint16)
    C64 = np.empty((M, N), np.float64) if want_f64 else None
    _load().oracle_gemm_mxfp6_nt(M, N, K, FP6_FORMATS[fmt], _ptr(qA), _ptr(qB), _ptr(sA), _ptr(sB), _ptr(C),
                                 _ptr(C64))
    return (C, C64) if want_f64 else C


def gemm_mxfp6_nt_at(qA, qB, sA, sB, rows, cols, fmt: str, K=None, want_f64: bool = False):
    """C[rows[p], cols[p]] of the block-scaled FP6 NT GEMM (bf16 bits)."""
    qA, qB, sA, sB = (_c(x, np.uint8) for x in (qA, qB, sA, sB))
    M, N, K = _mxfp6_shapes(qA, qB, sA, sB, K)
    rows, cols = _points(rows, cols)
    if rows.size and (rows.min() < 0 or rows.max() >= M or cols.min() < 0 or cols.max() >= N):
        raise ValueError("bad sample positions")
    out = np.empty(rows.size, np.uint16)
    out64 = np.empty(rows.size, np.float64) if want_f64 else None
    _load().oracle_gemm_mxfp6_nt_at(M, N, K, FP6_FORMATS[fmt], _ptr(qA), _ptr(qB), _ptr(sA), _ptr(sB),
                                    rows.size, _ptr(rows), _ptr(cols), _ptr(out), _ptr(out64))
    return (out, out64) if want_f64 else out
