"""CPU fp64 attention oracle -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The HIP library never calls it and the
two share no code.

The arithmetic lives in ``attn_oracle.c`` (plain C, fp64, the textbook
definition of softmax attention and its chain-rule gradient, see that file's
header).  This module only compiles it with gcc and marshals numpy arrays.
Parity of every function here is pinned by ``tests/test_oracle.py`` (closed
forms, invariants, finite differences, brute force in long double).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "attn_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
_lib = None

_dp = ctypes.POINTER(ctypes.c_double)
_ip = ctypes.POINTER(ctypes.c_int64)
_i64 = ctypes.c_int64


def build(force: bool = False) -> str:
    """Compile attn_oracle.c into liboracle.so (gcc, -O2, no fast-math)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + f".tmp{os.getpid()}"
        subprocess.check_call(["gcc", "-O2", "-std=c99", "-fPIC", "-shared", "-pthread",
                               "-Wall", "-Wextra", "-Wno-unused-parameter",
                               "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is None:
        build()
        lib = ctypes.CDLL(_LIB)
        lib.oracle_attention_forward.argtypes = [_dp, _dp, _dp, _i64, _i64, _i64, ctypes.c_double,
                                                 ctypes.c_int, _dp, _dp, ctypes.c_int]
        lib.oracle_attention_backward.argtypes = [_dp, _dp, _dp, _dp, _i64, _i64, _i64,
                                                  ctypes.c_double, ctypes.c_int, _dp, _dp, _dp,
                                                  ctypes.c_int]
        lib.oracle_forward_rows.argtypes = [_dp, _dp, _dp, _i64, _i64, ctypes.c_double, ctypes.c_int,
                                            _ip, _i64, _dp, _dp, ctypes.c_int]
        lib.oracle_backward_dq_rows.argtypes = [_dp, _dp, _dp, _dp, _i64, _i64, ctypes.c_double,
                                                ctypes.c_int, _ip, _i64, _dp, ctypes.c_int]
        lib.oracle_backward_dkdv_cols.argtypes = [_dp, _dp, _dp, _dp, _i64, _i64, ctypes.c_double,
                                                  ctypes.c_int, _ip, _i64, _dp, _dp, ctypes.c_int]
        for f in (lib.oracle_attention_forward, lib.oracle_attention_backward,
                  lib.oracle_forward_rows, lib.oracle_backward_dq_rows,
                  lib.oracle_backward_dkdv_cols):
            f.restype = ctypes.c_int
        _lib = lib
    return _lib


def _f64(x):
    return np.ascontiguousarray(x, dtype=np.float64)


def _ptr(a):
    return a.ctypes.data_as(_dp)


def attention_forward(q, k, v, scale: float, causal: bool, nthreads: int = 0):
    """q, k, v: [..., S, d] float64 -> (o [..., S, d], lse [..., S])."""
    q, k, v = _f64(q), _f64(k), _f64(v)
    S, d = q.shape[-2], q.shape[-1]
    BH = int(np.prod(q.shape[:-2], dtype=np.int64)) if q.ndim > 2 else 1
    o = np.empty(q.shape, dtype=np.float64)
    lse = np.empty(q.shape[:-1], dtype=np.float64)
    if q.size:
        rc = _load().oracle_attention_forward(_ptr(q), _ptr(k), _ptr(v), BH, S, d, float(scale),
                                              int(bool(causal)), _ptr(o), _ptr(lse), int(nthreads))
        if rc:
            raise MemoryError("oracle forward failed")
    return o, lse


def attention_backward(q, k, v, do, scale: float, causal: bool, nthreads: int = 0):
    """Gradients of sum(do * O) -> (dq, dk, dv), all [..., S, d] float64."""
    q, k, v, do = _f64(q), _f64(k), _f64(v), _f64(do)
    S, d = q.shape[-2], q.shape[-1]
    BH = int(np.prod(q.shape[:-2], dtype=np.int64)) if q.ndim > 2 else 1
    dq, dk, dv = (np.empty(q.shape, dtype=np.float64) for _ in range(3))
    if q.size:
        rc = _load().oracle_attention_backward(_ptr(q), _ptr(k), _ptr(v), _ptr(do), BH, S, d,
                                               float(scale), int(bool(causal)), _ptr(dq), _ptr(dk),
                                               _ptr(dv), int(nthreads))
        if rc:
            raise MemoryError("oracle backward failed")
    return dq, dk, dv


def forward_rows(q, k, v, rows, scale: float, causal: bool, nthreads: int = 0):
    """One head ([S, d] each): O and LSE of the listed query rows."""
    q, k, v = _f64(q), _f64(k), _f64(v)
    rows = np.ascontiguousarray(rows, dtype=np.int64)
    S, d = q.shape
    assert rows.size == 0 or (rows.min() >= 0 and rows.max() < S)
    o = np.empty((rows.size, d), dtype=np.float64)
    lse = np.empty(rows.size, dtype=np.float64)
    if rows.size:
        rc = _load().oracle_forward_rows(_ptr(q), _ptr(k), _ptr(v), S, d, float(scale),
                                         int(bool(causal)), rows.ctypes.data_as(_ip), rows.size,
                                         _ptr(o), _ptr(lse), int(nthreads))
        if rc:
            raise MemoryError("oracle forward_rows failed")
    return o, lse


def backward_dq_rows(q, k, v, do, rows, scale: float, causal: bool, nthreads: int = 0):
    """One head: dQ of the listed query rows."""
    q, k, v, do = _f64(q), _f64(k), _f64(v), _f64(do)
    rows = np.ascontiguousarray(rows, dtype=np.int64)
    S, d = q.shape
    assert rows.size == 0 or (rows.min() >= 0 and rows.max() < S)
    dq = np.empty((rows.size, d), dtype=np.float64)
    if rows.size:
        rc = _load().oracle_backward_dq_rows(_ptr(q), _ptr(k), _ptr(v), _ptr(do), S, d, float(scale),
                                             int(bool(causal)), rows.ctypes.data_as(_ip), rows.size,
                                             _ptr(dq), int(nthreads))
        if rc:
            raise MemoryError("oracle backward_dq_rows failed")
    return dq


def backward_dkdv_cols(q, k, v, do, cols, scale: float, causal: bool, nthreads: int = 0):
    """One head: dK and dV of the listed key/value rows."""
    q, k, v, do = _f64(q), _f64(k), _f64(v), _f64(do)
    cols = np.ascontiguousarray(cols, dtype=np.int64)
    S, d = q.shape
    assert cols.size == 0 or (cols.min() >= 0 and cols.max() < S)
    dk = np.zeros((cols.size, d), dtype=np.float64)
    dv = np.zeros((cols.size, d), dtype=np.float64)
    if cols.size:
        rc = _load().oracle_backward_dkdv_cols(_ptr(q), _ptr(k), _ptr(v), _ptr(do), S, d,
                                               float(scale), int(bool(causal)),
                                               cols.ctypes.data_as(_ip), cols.size, _ptr(dk),
                                               _ptr(dv), int(nthreads))
        if rc:
            raise MemoryError("oracle backward_dkdv_cols failed")
    return dk, dv
