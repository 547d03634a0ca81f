"""fp64 CPU oracle for HSTU attention and HSTU LMSD -- test infrastructure only.

Only the tests, the smoke check and the benchmark's CPU-baseline leg may import
this package.  The product path (the HIP library and its Python binding) never
does, and this package imports nothing from it.

The arithmetic lives in ``hstu_oracle.c`` (attention) and ``lmsd_oracle.c``
(LayerNorm-multiply-SiLU), plain C, fp64, libm ``exp``/``sqrt``, gcc ``-O2``
without fast-math, OpenMP over independent output rows.  This module
only builds and loads that file and marshals numpy arrays into it.  bf16 inputs
are widened exactly to fp64 here (``widen``); the score scale is passed as the
fp64 widening of the fp32 value the GPU receives.

Every function takes packed ``(T, H, D)`` arrays and int32 cumulative offsets
(HSTU Attention page, "Tensor layout") and returns fp64 arrays of the requested
rows.  ``rows=None`` computes every row.  ``mask`` is the page's
``window_size=(left, right)`` ("Mask support"), -1 leaving a side unbounded;
``True`` stands for causal ``(-1, 0)`` and ``False`` for full ``(-1, -1)``; an
int32 array of shape ``(N, L)`` or ``(1, N, L)`` is the page's arbitrary mask
``func_tensor`` (row r's endpoints in column r).
"""

from __future__ import annotations

import ctypes
import os
import subprocess
import sys
import threading
from typing import Optional, Tuple

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRCS = [os.path.join(_HERE, "hstu_oracle.c"), os.path.join(_HERE, "lmsd_oracle.c")]
_LIB = os.path.join(_HERE, "liboracle_hstu.so")
_lock = threading.Lock()
_lib = None


def _stale() -> bool:
    return not os.path.exists(_LIB) or any(os.path.getmtime(_LIB) < os.path.getmtime(src) for src in _SRCS)


def build(force: bool = True) -> str:
    """Compile the oracle's C sources with gcc into ``liboracle_hstu.so``."""
    global _lib
    with _lock:
        if force or _stale():
            tmp = _LIB + f".tmp{os.getpid()}"
            cmd = ["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c11",
                   "-Wall", "-Wextra", "-o", tmp, *_SRCS, "-lm"]
            subprocess.run(cmd, check=True)
            os.replace(tmp, _LIB)
            _lib = None
    return _LIB


def _load():
    global _lib
    if _lib is None:
        if _stale():
            build(force=False)
        with _lock:
            lib = ctypes.CDLL(_LIB)
            i64, i32p, f64p, i64p = ctypes.c_int64, ctypes.POINTER(ctypes.c_int32), \
                ctypes.POINTER(ctypes.c_double), ctypes.POINTER(ctypes.c_int64)
            lib.oracle_num_threads.restype = ctypes.c_int
            lib.oracle_hstu_fwd.restype = ctypes.c_int
            lib.oracle_hstu_fwd.argtypes = [i64, i32p, i32p, i64, i64, f64p, f64p, f64p,
                                            ctypes.c_double, ctypes.c_double, i64, i64, i32p, i64, i64,
                                            i64p, i64, f64p]
            lib.oracle_hstu_bwd_dq.restype = ctypes.c_int
            lib.oracle_hstu_bwd_dq.argtypes = [i64, i32p, i32p, i64, i64, f64p, f64p, f64p, f64p,
                                               ctypes.c_double, ctypes.c_double, i64, i64, i32p, i64, i64,
                                               i64p, i64, f64p]
            lib.oracle_hstu_bwd_dkdv.restype = ctypes.c_int
            lib.oracle_hstu_bwd_dkdv.argtypes = [i64, i32p, i32p, i64, i64, f64p, f64p, f64p, f64p,
                                                 ctypes.c_double, ctypes.c_double, i64, i64, i32p, i64, i64,
                                                 i64p, i64, f64p, f64p]
            ci = ctypes.c_int
            lib.oracle_lmsd_fwd.restype = None
            lib.oracle_lmsd_fwd.argtypes = [i64, i64, f64p, i64, f64p, i64, f64p, f64p, ctypes.c_double,
                                            ci, ci, ci, f64p, f64p, f64p]
            lib.oracle_lmsd_bwd.restype = None
            lib.oracle_lmsd_bwd.argtypes = [i64, i64, f64p, i64, f64p, i64, f64p, i64, f64p, f64p, f64p, f64p,
                                            ci, ci, ci, f64p, f64p, f64p, f64p]
            _lib = lib
    return _lib


def num_threads() -> int:
    """OpenMP threads the oracle runs on (OMP_NUM_THREADS, else the core count)."""
    return int(_load().oracle_num_threads())


def widen(bits: np.ndarray) -> np.ndarray:
    """Exact fp64 value of bf16 bit patterns (uint16)."""
    b = np.ascontiguousarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)


def _f64(x: np.ndarray) -> np.ndarray:
    if x.dtype == np.uint16:
        return widen(x)
    return np.ascontiguousarray(x, dtype=np.float64)


def _ptr(a: np.ndarray, ctype):
    return a.ctypes.data_as(ctypes.POINTER(ctype))


def window(mask) -> Tuple[int, int]:
    """(left, right) of a mask given as a bool (causal / full) or a window pair."""
    if isinstance(mask, (bool, np.bool_)):
        return (-1, 0) if mask else (-1, -1)
    left, right = (int(x) for x in mask)
    if left < -1 or right < -1:
        raise ValueError("window bounds must be >= -1")
    return left, right


def _mask_args(mask, total_q: int):
    """The C oracle's mask arguments (left, right, func, func_n, func_ld) and the
    array they point into (kept alive by the caller)."""
    if isinstance(mask, np.ndarray):
        f = mask[0] if mask.ndim == 3 else mask
        if f.ndim != 2 or f.dtype != np.int32 or f.shape[0] < 1 or f.shape[0] % 2 != 1:
            raise ValueError("func mask must be int32 of shape (N, L) or (1, N, L) with N odd")
        if f.shape[1] < total_q:
            raise ValueError("func mask needs a column for every query row")
        f = np.ascontiguousarray(f)
        return (-1, -1, _ptr(f, ctypes.c_int32), f.shape[0], f.shape[1]), f
    left, right = window(mask)
    return (left, right, None, 0, 0), None


def _prep(cu_q, cu_k, q, k, v, rows, total):
    cu_q = np.ascontiguousarray(cu_q, dtype=np.int32)
    cu_k = np.ascontiguousarray(cu_k, dtype=np.int32)
    if cu_q.shape != cu_k.shape or cu_q.ndim != 1 or cu_q.size < 1:
        raise ValueError("cu_seqlens_q/k must be 1-D of equal length B+1")
    q, k, v = _f64(q), _f64(k), _f64(v)
    if q.ndim != 3 or k.shape != v.shape or q.shape[1:] != k.shape[1:]:
        raise ValueError("q/k/v must be (T, H, D) with matching H, D")
    if rows is None:
        rows_arr = None
        n = total
    else:
        rows_arr = np.ascontiguousarray(rows, dtype=np.int64)
        n = rows_arr.size
        if n and (rows_arr.min() < 0 or rows_arr.max() >= total):
            raise ValueError("requested row out of range")
    return cu_q, cu_k, q, k, v, rows_arr, n


def fwd(cu_q, cu_k, q, k, v, alpha, scaling_seqlen, mask,
        rows: Optional[np.ndarray] = None) -> np.ndarray:
    """O rows (fp64, shape (n, H, D)) of HSTU attention."""
    cu_q, cu_k, q, k, v, rows_arr, n = _prep(cu_q, cu_k, q, k, v, rows, q.shape[0])
    margs, _keep = _mask_args(mask, q.shape[0])
    H, D = q.shape[1], q.shape[2]
    out = np.empty((n, H, D), dtype=np.float64)
    rc = _load().oracle_hstu_fwd(
        cu_q.size - 1, _ptr(cu_q, ctypes.c_int32), _ptr(cu_k, ctypes.c_int32), H, D,
        _ptr(q, ctypes.c_double), _ptr(k, ctypes.c_double), _ptr(v, ctypes.c_double),
        float(alpha), float(scaling_seqlen), *margs,
        None if rows_arr is None else _ptr(rows_arr, ctypes.c_int64), n,
        _ptr(out, ctypes.c_double))
    if rc != 0:
        raise ValueError("oracle: a row lies outside every sequence")
    return out


def bwd_dq(cu_q, cu_k, dout, q, k, v, alpha, scaling_seqlen, mask,
           rows: Optional[np.ndarray] = None) -> np.ndarray:
    """dQ rows (fp64) given the upstream gradient ``dout``."""
    cu_q, cu_k, q, k, v, rows_arr, n = _prep(cu_q, cu_k, q, k, v, rows, q.shape[0])
    margs, _keep = _mask_args(mask, q.shape[0])
    dout = _f64(dout)
    if dout.shape != q.shape:
        raise ValueError("dout must match q")
    H, D = q.shape[1], q.shape[2]
    out = np.empty((n, H, D), dtype=np.float64)
    rc = _load().oracle_hstu_bwd_dq(
        cu_q.size - 1, _ptr(cu_q, ctypes.c_int32), _ptr(cu_k, ctypes.c_int32), H, D,
        _ptr(dout, ctypes.c_double), _ptr(q, ctypes.c_double), _ptr(k, ctypes.c_double),
        _ptr(v, ctypes.c_double), float(alpha), float(scaling_seqlen), *margs,
        None if rows_arr is None else _ptr(rows_arr, ctypes.c_int64), n,
        _ptr(out, ctypes.c_double))
    if rc != 0:
        raise ValueError("oracle: a row lies outside every sequence")
    return out


def bwd_dkdv(cu_q, cu_k, dout, q, k, v, alpha, scaling_seqlen, mask,
             rows: Optional[np.ndarray] = None) -> Tuple[np.ndarray, np.ndarray]:
    """(dK, dV) rows (fp64) for packed key rows ``rows``."""
    cu_q, cu_k, q, k, v, rows_arr, n = _prep(cu_q, cu_k, q, k, v, rows, k.shape[0])
    margs, _keep = _mask_args(mask, q.shape[0])
    dout = _f64(dout)
    if dout.shape != q.shape:
        raise ValueError("dout must match q")
    H, D = q.shape[1], q.shape[2]
    dk = np.empty((n, H, D), dtype=np.float64)
    dv = np.empty((n, H, D), dtype=np.float64)
    rc = _load().oracle_hstu_bwd_dkdv(
        cu_q.size - 1, _ptr(cu_q, ctypes.c_int32), _ptr(cu_k, ctypes.c_int32), H, D,
        _ptr(dout, ctypes.c_double), _ptr(q, ctypes.c_double), _ptr(k, ctypes.c_double),
        _ptr(v, ctypes.c_double), float(alpha), float(scaling_seqlen), *margs,
        None if rows_arr is None else _ptr(rows_arr, ctypes.c_int64), n,
        _ptr(dk, ctypes.c_double), _ptr(dv, ctypes.c_double))
    if rc != 0:
        raise ValueError("oracle: a row lies outside every sequence")
    return dk, dv


def fwd_workload(wl, rows=None) -> np.ndarray:
    """Oracle O for a ``Workload`` (its bf16 inputs widened exactly)."""
    return fwd(wl.cu_seqlens_q, wl.cu_seqlens_k, wl.q, wl.k, wl.v,
               float(wl.alpha), wl.scaling_seqlen, wl.mask_spec, rows)


def bwd_workload(wl, rows_q=None, rows_k=None):
    """Oracle (dQ, dK, dV) for a ``Workload`` with an upstream gradient."""
    if wl.do is None:
        raise ValueError("workload has no upstream gradient")
    dq = bwd_dq(wl.cu_seqlens_q, wl.cu_seqlens_k, wl.do, wl.q, wl.k, wl.v,
                float(wl.alpha), wl.scaling_seqlen, wl.mask_spec, rows_q)
    dk, dv = bwd_dkdv(wl.cu_seqlens_q, wl.cu_seqlens_k, wl.do, wl.q, wl.k, wl.v,
                      float(wl.alpha), wl.scaling_seqlen, wl.mask_spec, rows_k)
    return dq, dk, dv


if __name__ == "__main__":  # pragma: no cover - manual build helper
    print(build(force=True), file=sys.stderr)


# ---------------------------------------------------------------------------
# HSTU LMSD (LayerNorm, affine, times SiLU(u) or u; dropout off)
# ---------------------------------------------------------------------------
def _rows(a: np.ndarray, name: str) -> np.ndarray:
    a = _f64(a)
    if a.ndim != 2:
        raise ValueError(f"{name} must be (N, D)")
    return np.ascontiguousarray(a)


def lmsd_fwd(x, u, weight, bias, eps: float, silu_u: bool = True, concat_u: bool = False,
             concat_x: bool = False):
    """(y, mean, rstd) in fp64; y is (N, S D) with S = 1 + concat_u + concat_x."""
    x, u = _rows(x, "x"), _rows(u, "u")
    if x.shape != u.shape:
        raise ValueError("x and u must match")
    n, d = x.shape
    w, b = np.ascontiguousarray(_f64(weight)), np.ascontiguousarray(_f64(bias))
    if w.shape != (d,) or b.shape != (d,):
        raise ValueError("weight and bias must be (D,)")
    s = 1 + int(bool(concat_u)) + int(bool(concat_x))
    y = np.empty((n, s * d))
    mean, rstd = np.empty(n), np.empty(n)
    _load().oracle_lmsd_fwd(n, d, _ptr(x, ctypes.c_double), d, _ptr(u, ctypes.c_double), d,
                            _ptr(w, ctypes.c_double), _ptr(b, ctypes.c_double), float(eps), int(bool(silu_u)),
                            int(bool(concat_u)), int(bool(concat_x)), _ptr(y, ctypes.c_double),
                            _ptr(mean, ctypes.c_double), _ptr(rstd, ctypes.c_double))
    return y, mean, rstd


def lmsd_bwd(dy, x, u, weight, bias, mean, rstd, silu_u: bool = True, concat_u: bool = False,
             concat_x: bool = False):
    """(dx, du, dweight, dbias) in fp64 from the upstream gradient dy (N, S D) and the
    saved statistics."""
    x, u = _rows(x, "x"), _rows(u, "u")
    n, d = x.shape
    dy = _rows(dy, "dy")
    s = 1 + int(bool(concat_u)) + int(bool(concat_x))
    if dy.shape != (n, s * d):
        raise ValueError("dy must be (N, S D)")
    w, b = np.ascontiguousarray(_f64(weight)), np.ascontiguousarray(_f64(bias))
    mean = np.ascontiguousarray(mean, dtype=np.float64)
    rstd = np.ascontiguousarray(rstd, dtype=np.float64)
    if mean.shape != (n,) or rstd.shape != (n,):
        raise ValueError("mean and rstd must be (N,)")
    dx, du = np.empty((n, d)), np.empty((n, d))
    dw, db = np.empty(d), np.empty(d)
    _load().oracle_lmsd_bwd(n, d, _ptr(dy, ctypes.c_double), s * d, _ptr(x, ctypes.c_double), d,
                            _ptr(u, ctypes.c_double), d, _ptr(w, ctypes.c_double), _ptr(b, ctypes.c_double),
                            _ptr(mean, ctypes.c_double), _ptr(rstd, ctypes.c_double), int(bool(silu_u)),
                            int(bool(concat_u)), int(bool(concat_x)), _ptr(dx, ctypes.c_double),
                            _ptr(du, ctypes.c_double), _ptr(dw, ctypes.c_double), _ptr(db, ctypes.c_double))
    return dx, du, dw, db
