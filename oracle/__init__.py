"""CPU oracle for 2:4 structured-sparse compression and multiplication.

TEST INFRASTRUCTURE ONLY: imported by ``tests/``, ``__graft_entry__.smoke()``
and the CPU-baseline leg of ``bench.py``.  The product library never imports
or links it, and it shares no code with the GPU path.

The arithmetic lives in ``sp24_oracle.c`` (plain C, fp64 / int64); this module
only marshals numpy arrays through ctypes.  Element arrays carry raw bit
patterns: ``uint16`` for fp16/bf16, ``uint8`` for fp8 (E4M3) / bf8 (E5M2),
``int8`` for int8.  Compressed values keep the element type; metadata is
``uint32`` words, 16 two-bit position codes per word, LSB first (the code of
compressed element c of row i is bits [2(c%16), 2(c%16)+1] of
``meta[i, c // 16]``).

Every function is pinned by ``tests/test_oracle.py`` against facts that do
not come from this code (see that file's docstring).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

F16, BF16, I8, E4M3, E5M2 = 1, 2, 3, 4, 5
NAMES = {F16: "f16", BF16: "bf16", I8: "i8", E4M3: "fp8_e4m3", E5M2: "bf8_e5m2"}
_STORE = {F16: np.uint16, BF16: np.uint16, I8: np.int8, E4M3: np.uint8, E5M2: np.uint8}

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "sp24_oracle.c")
_LIB_PATH = os.path.join(_HERE, "libsp24_oracle.so")
_lib = None


def build(force: bool = True) -> str:
    """Compile the oracle with the host C compiler (no GPU toolchain)."""
    if force or not os.path.exists(_LIB_PATH):
        tmp = _LIB_PATH + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-O2", "-std=c11", "-ffp-contract=off", "-fPIC", "-shared",
                               _SRC, "-o", tmp, "-lm"])
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            build(force=False)
        lib = ctypes.CDLL(_LIB_PATH)
        P, I64, I = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
        D = ctypes.c_double
        lib.orc_decode.argtypes = [ctypes.c_uint32, I]
        lib.orc_decode.restype = D
        lib.orc_key.argtypes = [ctypes.c_uint32, I]
        lib.orc_key.restype = ctypes.c_uint32
        lib.orc_prune_compress.argtypes = [P, P, P, I64, I64, I]
        lib.orc_decompress.argtypes = [P, P, P, I64, I64, I]
        lib.orc_count_invalid.argtypes = [P, I64, I64]
        lib.orc_count_invalid.restype = I64
        lib.orc_gemm_f64.argtypes = [P, P, I, P, I, P, P, P, P, I64, I64, I64, D, D]
        lib.orc_round_to.argtypes = [D, I]
        lib.orc_round_to.restype = ctypes.c_uint32
        lib.orc_gemm_i64.argtypes = [P, P, P, P, P, I64, I64, I64, I]
        lib.orc_gemm_points_f64.argtypes = [P, P, I, P, I, P, I64, I64, I64, D, D, I64, P, P, P, P]
        lib.orc_gemm_points_i64.argtypes = [P, P, P, P, I64, I64, I64, I, I64, P, P, P]
        for f in ("orc_prune_compress", "orc_decompress", "orc_gemm_f64", "orc_gemm_i64",
                  "orc_gemm_points_f64", "orc_gemm_points_i64"):
            getattr(lib, f).restype = I
        _lib = lib
    return _lib


def _ptr(a):
    return None if a is None else ctypes.c_void_p(a.ctypes.data)


def _check(rc, what):
    if rc == 2:
        raise OverflowError(f"{what}: result outside int32 range")
    if rc != 0:
        raise ValueError(f"{what}: bad arguments (rc={rc})")


def _as_bits(a, dtype):
    a = np.ascontiguousarray(a)
    want = _STORE[dtype]
    if a.dtype != want:
        if a.dtype.itemsize != np.dtype(want).itemsize:
            raise TypeError(f"array of {a.dtype} cannot hold {NAMES[dtype]} bits")
        a = a.view(want)
    return a


def decode(bits, dtype) -> np.ndarray:
    """Exact value (float64) of every element of a bit-pattern array."""
    lib = _load()
    flat = np.ascontiguousarray(bits).reshape(-1)
    if dtype == I8:
        return flat.view(np.int8).astype(np.float64).reshape(np.shape(bits))
    mask = 0xFFFF if np.dtype(_STORE[dtype]).itemsize == 2 else 0xFF
    n = 1 << (16 if mask == 0xFFFF else 8)
    table = np.array([lib.orc_decode(b, dtype) for b in range(n)], dtype=np.float64)
    return table[flat.astype(np.int64) & mask].reshape(np.shape(bits))


def key(bits: int, dtype) -> int:
    """Magnitude key of one element (what pruning compares)."""
    return int(_load().orc_key(int(bits) & 0xFFFFFFFF, dtype))


def prune_compress(A, dtype):
    """Dense M x K bit array -> (vals M x K/2, meta M x K/32 uint32)."""
    lib = _load()
    A = _as_bits(A, dtype)
    M, K = A.shape
    vals = np.empty((M, K // 2), dtype=_STORE[dtype])
    meta = np.empty((M, max(K // 32, 0)), dtype=np.uint32)
    _check(lib.orc_prune_compress(_ptr(A), _ptr(vals), _ptr(meta), M, K, dtype), "prune_compress")
    return vals, meta


def decompress(vals, meta, dtype):
    """(vals M x K/2, meta M x K/32) -> dense M x K bit array (+0 at dropped slots)."""
    lib = _load()
    vals = _as_bits(vals, dtype)
    meta = np.ascontiguousarray(meta, dtype=np.uint32)
    M, KC = vals.shape
    K = 2 * KC
    out = np.empty((M, K), dtype=_STORE[dtype])
    _check(lib.orc_decompress(_ptr(vals), _ptr(meta), _ptr(out), M, K, dtype), "decompress")
    return out


def count_invalid(meta, K):
    """Number of groups of the M x K/32 metadata whose codes are not strictly increasing."""
    lib = _load()
    meta = np.ascontiguousarray(meta, dtype=np.uint32)
    n = lib.orc_count_invalid(_ptr(meta), meta.shape[0], K)
    if n < 0:
        raise ValueError("count_invalid: bad arguments")
    return int(n)


def round_to(x, dtype) -> np.ndarray:
    """Bit patterns (uint16) of the nearest fp16 / bf16 values to the float64
    array x, ties to even (C oracle, one element at a time)."""
    lib = _load()
    if dtype not in (F16, BF16):
        raise ValueError("round_to: fp16 or bf16 only")
    flat = np.ascontiguousarray(x, dtype=np.float64).reshape(-1)
    out = np.array([lib.orc_round_to(float(v), dtype) for v in flat], dtype=np.uint16)
    return out.reshape(np.shape(x))


def gemm_f64(vals, meta, a_type, B, b_type, C=None, alpha=1.0, beta=0.0, want_abs=True, bias=None):
    """alpha * expand(vals, meta) @ B + beta * C + bias in float64 (float types).

    C is given as float32 values (a 16-bit C widened, which is exact); bias is
    None or N float32 values.  Returns (D, S) where S = |alpha| * sum|a*b| +
    |beta*C| + |bias| per element (None if want_abs is False)."""
    lib = _load()
    vals = _as_bits(vals, a_type)
    B = _as_bits(B, b_type)
    meta = np.ascontiguousarray(meta, dtype=np.uint32)
    M, KC = vals.shape
    K, N = B.shape
    if K != 2 * KC:
        raise ValueError("K mismatch")
    if beta != 0.0:
        C = np.ascontiguousarray(C, dtype=np.float32)
        if C.shape != (M, N):
            raise ValueError("C shape")
    else:
        C = None
    if bias is not None:
        bias = np.ascontiguousarray(bias, dtype=np.float32)
        if bias.shape != (N,):
            raise ValueError("bias shape")
    D = np.empty((M, N), dtype=np.float64)
    S = np.empty((M, N), dtype=np.float64) if want_abs else None
    _check(lib.orc_gemm_f64(_ptr(vals), _ptr(meta), a_type, _ptr(B), b_type, _ptr(C), _ptr(bias), _ptr(D), _ptr(S),
                            M, N, K, float(alpha), float(beta)), "gemm_f64")
    return D, S


def gemm_i64(vals, meta, B, C=None, beta_one=False):
    """expand(vals, meta) @ B (+ C) exactly in int64 (int8 inputs)."""
    lib = _load()
    vals = _as_bits(vals, I8)
    B = _as_bits(B, I8)
    meta = np.ascontiguousarray(meta, dtype=np.uint32)
    M, KC = vals.shape
    K, N = B.shape
    if K != 2 * KC:
        raise ValueError("K mismatch")
    if beta_one:
        C = np.ascontiguousarray(C, dtype=np.int32)
    else:
        C = None
    D = np.empty((M, N), dtype=np.int64)
    _check(lib.orc_gemm_i64(_ptr(vals), _ptr(meta), _ptr(B), _ptr(C), _ptr(D), M, N, K, int(bool(beta_one))),
           "gemm_i64")
    return D


def gemm_points_f64(vals, meta, a_type, B, b_type, ii, jj, C=None, alpha=1.0, beta=0.0):
    """The float product at output points (ii[p], jj[p]) only; returns (D, S)."""
    lib = _load()
    vals = _as_bits(vals, a_type)
    B = _as_bits(B, b_type)
    meta = np.ascontiguousarray(meta, dtype=np.uint32)
    M, KC = vals.shape
    K, N = B.shape
    ii = np.ascontiguousarray(ii, dtype=np.int64)
    jj = np.ascontiguousarray(jj, dtype=np.int64)
    if beta != 0.0:
        C = np.ascontiguousarray(C, dtype=np.float32)
    else:
        C = None
    out = np.empty(len(ii), dtype=np.float64)
    S = np.empty(len(ii), dtype=np.float64)
    _check(lib.orc_gemm_points_f64(_ptr(vals), _ptr(meta), a_type, _ptr(B), b_type, _ptr(C), M, N, K,
                                   float(alpha), float(beta), len(ii), _ptr(ii), _ptr(jj), _ptr(out), _ptr(S)),
           "gemm_points_f64")
    return out, S


def gemm_points_i64(vals, meta, B, ii, jj, C=None, beta_one=False):
    """The int8 product at output points (ii[p], jj[p]) only."""
    lib = _load()
    vals = _as_bits(vals, I8)
    B = _as_bits(B, I8)
    meta = np.ascontiguousarray(meta, dtype=np.uint32)
    M, KC = vals.shape
    K, N = B.shape
    ii = np.ascontiguousarray(ii, dtype=np.int64)
    jj = np.ascontiguousarray(jj, dtype=np.int64)
    C = np.ascontiguousarray(C, dtype=np.int32) if beta_one else None
    out = np.empty(len(ii), dtype=np.int64)
    _check(lib.orc_gemm_points_i64(_ptr(vals), _ptr(meta), _ptr(B), _ptr(C), M, N, K, int(bool(beta_one)),
                                   len(ii), _ptr(ii), _ptr(jj), _ptr(out)), "gemm_points_i64")
    return out
