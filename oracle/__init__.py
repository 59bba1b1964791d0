"""fp64 sequential CPU oracle for the linear-recurrence scans.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this package.  The product path
(``linear_recurrence_scans_amd`` and its HIP library) never does, and this
package imports nothing from it.

The arithmetic lives in ``oracle.c`` (plain C, fp64, sequential in time); this
module only compiles it with gcc, loads it with ctypes and marshals numpy
arrays.  Definitions follow the minGRU documentation page "Triton kernels",
section "Kernel entry points" (linear_scan_fwd/bwd, parallel_scan_log_fwd,
affine_scan_fwd/bwd).  Every function is pinned by ``tests/test_oracle.py``.
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


def build(force: bool = True) -> str:
    """Compile oracle.c into liboracle.so with gcc (-O2, OpenMP, no SIMD intrinsics)."""
    if not force and os.path.exists(_LIB):
        return _LIB
    tmp = _LIB + ".tmp%d" % os.getpid()
    cmd = ["gcc", "-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared",
           "-Wall", "-Wextra", "-o", tmp, _SRC, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build()
        lib = ctypes.CDLL(_LIB)
        i64 = ctypes.c_int64
        p = ctypes.c_void_p
        lib.lrs_oracle_num_threads.restype = ctypes.c_int
        lib.lrs_oracle_set_threads.argtypes = [ctypes.c_int]
        lib.lrs_oracle_set_threads.restype = None
        lib.lrs_oracle_linear_fwd.argtypes = [i64, i64, i64, p, p, p, p]
        lib.lrs_oracle_linear_bwd.argtypes = [i64, i64, i64] + [p] * 7
        lib.lrs_oracle_scan_log_fwd.argtypes = [i64, i64, i64, p, p, p]
        lib.lrs_oracle_scan_log_fwd_logspace.argtypes = [i64, i64, i64, p, p, p]
        lib.lrs_oracle_scan_log_bwd.argtypes = [i64, i64, i64] + [p] * 6
        lib.lrs_oracle_linear_fwd_h0.argtypes = [i64, i64, i64] + [p] * 5
        lib.lrs_oracle_linear_bwd_h0.argtypes = [i64, i64, i64] + [p] * 9
        lib.lrs_oracle_affine_fwd_h0.argtypes = [i64] * 5 + [p] * 5
        lib.lrs_oracle_affine_bwd_h0.argtypes = [i64] * 5 + [p] * 9
        lib.lrs_oracle_affine_fwd.argtypes = [i64] * 5 + [p] * 4
        lib.lrs_oracle_affine_bwd.argtypes = [i64] * 5 + [p] * 7
        for f in ("lrs_oracle_linear_fwd", "lrs_oracle_linear_bwd",
                  "lrs_oracle_scan_log_fwd", "lrs_oracle_scan_log_fwd_logspace",
                  "lrs_oracle_scan_log_bwd", "lrs_oracle_linear_fwd_h0", "lrs_oracle_linear_bwd_h0",
                  "lrs_oracle_affine_fwd_h0", "lrs_oracle_affine_bwd_h0",
                  "lrs_oracle_affine_fwd", "lrs_oracle_affine_bwd"):
            getattr(lib, f).restype = None
        _lib = lib
    return _lib


def num_threads() -> int:
    """OpenMP threads the oracle uses for independent channels/heads."""
    return int(_load().lrs_oracle_num_threads())


def set_threads(n: int) -> None:
    """Threads for the independent channels/heads of later calls."""
    _load().lrs_oracle_set_threads(int(n))


def _f64(x) -> np.ndarray:
    return np.ascontiguousarray(np.asarray(x, dtype=np.float64))


def _ptr(x: np.ndarray):
    return x.ctypes.data_as(ctypes.c_void_p)


def linear_scan_fwd(a, b):
    """(A, Bc) for a, b of shape (B, T, D): A = running product, Bc = h_0=0 states."""
    a, b = _f64(a), _f64(b)
    if a.shape != b.shape or a.ndim != 3:
        raise ValueError("a and b must both be (B, T, D)")
    Bn, T, D = a.shape
    A = np.empty_like(a)
    Bc = np.empty_like(a)
    _load().lrs_oracle_linear_fwd(Bn, T, D, _ptr(a), _ptr(b), _ptr(A), _ptr(Bc))
    return A, Bc


def linear_scan_bwd(a, A, Bc, gA, gBc):
    """(da, db) for the k=1 scan, reading the given a, A, Bc and upstream gA, gBc."""
    a, A, Bc, gA, gBc = (_f64(x) for x in (a, A, Bc, gA, gBc))
    for x in (A, Bc, gA, gBc):
        if x.shape != a.shape:
            raise ValueError("all inputs must share the (B, T, D) shape of a")
    Bn, T, D = a.shape
    da = np.empty_like(a)
    db = np.empty_like(a)
    _load().lrs_oracle_linear_bwd(Bn, T, D, _ptr(a), _ptr(A), _ptr(Bc), _ptr(gA),
                                  _ptr(gBc), _ptr(da), _ptr(db))
    return da, db


def _log_shapes(lc, lv):
    if lc.ndim != 3 or lv.ndim != 3:
        raise ValueError("log_coeffs must be (B, T, D) and log_values (B, T+1, D)")
    Bn, T, D = lc.shape
    if lv.shape != (Bn, T + 1, D):
        raise ValueError("log_values must be (B, T+1, D)")
    return Bn, T, D


def scan_log_fwd(log_coeffs, log_values):
    """h_1..h_T (B, T, D) from log_coeffs (B,T,D) and log_values (B,T+1,D), linear space."""
    lc, lv = _f64(log_coeffs), _f64(log_values)
    Bn, T, D = _log_shapes(lc, lv)
    h = np.empty_like(lc)
    _load().lrs_oracle_scan_log_fwd(Bn, T, D, _ptr(lc), _ptr(lv), _ptr(h))
    return h


def scan_log_fwd_logspace(log_coeffs, log_values):
    """Same states as scan_log_fwd, computed entirely in log space (logaddexp)."""
    lc, lv = _f64(log_coeffs), _f64(log_values)
    Bn, T, D = _log_shapes(lc, lv)
    h = np.empty_like(lc)
    _load().lrs_oracle_scan_log_fwd_logspace(Bn, T, D, _ptr(lc), _ptr(lv), _ptr(h))
    return h


def scan_log_bwd(log_coeffs, log_values, h, g):
    """(dlog_coeffs (B,T,D), dlog_values (B,T+1,D)): gradient of scan_log_fwd,
    with the forward output h and the upstream gradient g = dL/dh."""
    lc, lv, h, g = _f64(log_coeffs), _f64(log_values), _f64(h), _f64(g)
    Bn, T, D = _log_shapes(lc, lv)
    if h.shape != lc.shape or g.shape != lc.shape:
        raise ValueError("h and g must be (B, T, D)")
    dlc = np.empty_like(lc)
    dlv = np.empty_like(lv)
    _load().lrs_oracle_scan_log_bwd(Bn, T, D, _ptr(lc), _ptr(lv), _ptr(h), _ptr(g), _ptr(dlc), _ptr(dlv))
    return dlc, dlv


def affine_scan_fwd(A, Bm):
    """(Abar, Bbar) for A (B,T,n,k,k) and Bm (B,T,n,k,v)."""
    A, Bm = _f64(A), _f64(Bm)
    if A.ndim != 5 or Bm.ndim != 5 or A.shape[3] != A.shape[4] or A.shape[:4] != Bm.shape[:4]:
        raise ValueError("A must be (B,T,n,k,k) and Bm (B,T,n,k,v)")
    Bn, T, n, k, _ = A.shape
    v = Bm.shape[4]
    Abar = np.empty_like(A)
    Bbar = np.empty_like(Bm)
    _load().lrs_oracle_affine_fwd(Bn, T, n, k, v, _ptr(A), _ptr(Bm), _ptr(Abar), _ptr(Bbar))
    return Abar, Bbar


def affine_scan_bwd(A, Abar, Bbar, gAbar, gBbar):
    """(dA, dB) for the k x k scan, reading the given A, Abar, Bbar and grads."""
    A, Abar, Bbar, gAbar, gBbar = (_f64(x) for x in (A, Abar, Bbar, gAbar, gBbar))
    if A.ndim != 5 or Abar.shape != A.shape or gAbar.shape != A.shape:
        raise ValueError("A, Abar, gAbar must be (B,T,n,k,k)")
    if Bbar.ndim != 5 or gBbar.shape != Bbar.shape or Bbar.shape[:4] != A.shape[:4]:
        raise ValueError("Bbar, gBbar must be (B,T,n,k,v)")
    Bn, T, n, k, _ = A.shape
    v = Bbar.shape[4]
    dA = np.empty_like(A)
    dB = np.empty_like(Bbar)
    _load().lrs_oracle_affine_bwd(Bn, T, n, k, v, _ptr(A), _ptr(Abar), _ptr(Bbar),
                                  _ptr(gAbar), _ptr(gBbar), _ptr(dA), _ptr(dB))
    return dA, dB


# ---------------------------------------------------------------------------
# given initial state (h0 / H0; None = zero)
# ---------------------------------------------------------------------------

def _opt(x, shape):
    if x is None:
        return None
    x = _f64(x)
    if x.shape != shape:
        raise ValueError("initial state must have shape %s" % (shape,))
    return x


def _optptr(x):
    return None if x is None else _ptr(x)


def linear_scan_fwd_h0(a, b, h0):
    """(A, H) with H_t = a_t H_{t-1} + b_t from H_0 = h0 (B, D)."""
    a, b = _f64(a), _f64(b)
    Bn, T, D = a.shape
    h0 = _opt(h0, (Bn, D))
    A, H = np.empty_like(a), np.empty_like(a)
    _load().lrs_oracle_linear_fwd_h0(Bn, T, D, _ptr(a), _ptr(b), _optptr(h0), _ptr(A), _ptr(H))
    return A, H


def linear_scan_bwd_h0(a, A, H, h0, gA, gH):
    """(da, db, dh0): gradient of linear_scan_fwd_h0."""
    a, A, H, gA, gH = (_f64(x) for x in (a, A, H, gA, gH))
    Bn, T, D = a.shape
    h0 = _opt(h0, (Bn, D))
    da, db, dh0 = np.empty_like(a), np.empty_like(a), np.empty((Bn, D))
    _load().lrs_oracle_linear_bwd_h0(Bn, T, D, _ptr(a), _ptr(A), _ptr(H), _optptr(h0), _ptr(gA), _ptr(gH),
                                     _ptr(da), _ptr(db), _ptr(dh0))
    return da, db, dh0


def affine_scan_fwd_h0(A, Bm, H0):
    """(Abar, H) from X_0 = [I | H0], H0 (B, n, k, v)."""
    A, Bm = _f64(A), _f64(Bm)
    Bn, T, n, k, _ = A.shape
    v = Bm.shape[4]
    H0 = _opt(H0, (Bn, n, k, v))
    Abar, H = np.empty_like(A), np.empty_like(Bm)
    _load().lrs_oracle_affine_fwd_h0(Bn, T, n, k, v, _ptr(A), _ptr(Bm), _optptr(H0), _ptr(Abar), _ptr(H))
    return Abar, H


def affine_scan_bwd_h0(A, Abar, H, H0, gAbar, gH):
    """(dA, dB, dH0): gradient of affine_scan_fwd_h0."""
    A, Abar, H, gAbar, gH = (_f64(x) for x in (A, Abar, H, gAbar, gH))
    Bn, T, n, k, _ = A.shape
    v = H.shape[4]
    H0 = _opt(H0, (Bn, n, k, v))
    dA, dB, dH0 = np.empty_like(A), np.empty_like(H), np.empty((Bn, n, k, v))
    _load().lrs_oracle_affine_bwd_h0(Bn, T, n, k, v, _ptr(A), _ptr(Abar), _ptr(H), _optptr(H0), _ptr(gAbar),
                                     _ptr(gH), _ptr(dA), _ptr(dB), _ptr(dH0))
    return dA, dB, dH0
