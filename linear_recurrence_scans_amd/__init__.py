"""linear_recurrence_scans_amd -- MI355X (gfx950) scans of h_t = a_t h_{t-1} + b_t.

Thin ctypes binding over ``libmiscan.so`` (C ABI in ``include/miscan.h``).  This
module only marshals arguments: it checks tensor shapes, makes inputs
contiguous, allocates outputs and the workspace with torch, and passes raw
device pointers plus torch's current HIP stream.  Every step of every scan runs
in the library's HIP kernels; there is no CPU or eager fallback, and a missing
library raises at first use.

Names follow the C ABI (``mi_linear_scan_fwd`` ...); the minGRU "Triton
kernels" page's op names (``linear_scan_fwd(a, b) -> (A, Bc)`` ...) are
provided as aliases with the same argument order and returns.
"""
from __future__ import annotations

import contextlib
import ctypes
import os

import torch

__all__ = [
    "MiscanError", "available", "library_path",
    "mi_status_string", "mi_device_check",
    "mi_linear_scan_workspace", "mi_linear_scan_fwd", "mi_linear_scan_bwd",
    "mi_linear_scan_fwd_h0", "mi_linear_scan_bwd_h0",
    "mi_linear_scan_fwd_noalloc", "NOALLOC_SCRATCH_BYTES",
    "set_checked", "workspace_timeouts",
    "mi_scan_log_workspace", "mi_scan_log_fwd", "mi_scan_log_bwd",
    "mi_affine_scan_workspace", "mi_affine_scan_fwd", "mi_affine_scan_bwd",
    "mi_affine_scan_fwd_h0", "mi_affine_scan_bwd_h0",
    "linear_scan_fwd", "linear_scan_bwd", "parallel_scan_log_fwd", "parallel_scan_log_bwd",
    "affine_scan_fwd", "affine_scan_bwd",
]

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libmiscan.so")

MI_F32, MI_BF16, MI_F16 = 0, 1, 2
# Bytes of the per-device scratch array behind mi_linear_scan_fwd_noalloc
# (MI_NOALLOC_SCRATCH_BYTES in include/miscan.h).
NOALLOC_SCRATCH_BYTES = 72 << 20
_DTYPES = {torch.float32: MI_F32, torch.bfloat16: MI_BF16, torch.float16: MI_F16}

# C ABI entry points and their argument types.
_V, _I64, _SZ = ctypes.c_void_p, ctypes.c_int64, ctypes.c_size_t
_I = ctypes.c_int
_SIGS = {
    "mi_status_string": ([_I], ctypes.c_char_p),
    "mi_device_check": ([_I, ctypes.c_char_p, _SZ], _I),
    "mi_linear_scan_workspace": ([_I64, _I64, _I64, _I], _SZ),
    "mi_linear_scan_fwd": ([_V] * 4 + [_I64] * 3 + [_I, _V, _SZ, _V], _I),
    "mi_linear_scan_bwd": ([_V] * 7 + [_I64] * 3 + [_I, _V, _SZ, _V], _I),
    "mi_linear_scan_fwd_noalloc": ([_V] * 4 + [_I64] * 3 + [_I, _V], _I),
    "mi_linear_scan_fwd_h0": ([_V] * 5 + [_I64] * 3 + [_I, _V, _SZ, _V], _I),
    "mi_linear_scan_bwd_h0": ([_V] * 9 + [_I64] * 3 + [_I, _V, _SZ, _V], _I),
    "mi_scan_log_workspace": ([_I64, _I64, _I64, _I], _SZ),
    "mi_scan_log_fwd": ([_V] * 3 + [_I64] * 3 + [_I, _V, _SZ, _V], _I),
    "mi_scan_log_bwd": ([_V] * 6 + [_I64] * 3 + [_I, _V, _SZ, _V], _I),
    "mi_affine_scan_workspace": ([_I64] * 5 + [_I], _SZ),
    "mi_affine_scan_fwd": ([_V] * 4 + [_I64] * 5 + [_I, _V, _SZ, _V], _I),
    "mi_affine_scan_bwd": ([_V] * 7 + [_I64] * 5 + [_I, _V, _SZ, _V], _I),
    "mi_affine_scan_fwd_h0": ([_V] * 5 + [_I64] * 5 + [_I, _V, _SZ, _V], _I),
    "mi_affine_scan_bwd_h0": ([_V] * 9 + [_I64] * 5 + [_I, _V, _SZ, _V], _I),
}

_lib = None


class MiscanError(RuntimeError):
    """A libmiscan call returned a status other than MI_OK."""

    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__("%s: %s" % (where, mi_status_string(status)))


def library_path() -> str:
    return _LIB_PATH


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            raise ImportError(
                "libmiscan.so is not built at %s; build it with "
                "`python -m linear_recurrence_scans_amd.build` (hipcc, gfx950)" % _LIB_PATH)
        lib = ctypes.CDLL(_LIB_PATH)
        for name, (argtypes, restype) in _SIGS.items():
            f = getattr(lib, name)
            f.argtypes = argtypes
            f.restype = restype
        _lib = lib
    return _lib


def mi_status_string(status: int) -> str:
    return _load().mi_status_string(int(status)).decode()


def mi_device_check(device: int = 0):
    """(ok, reason): whether `device` is a gfx950 GPU the library can launch on."""
    buf = ctypes.create_string_buffer(256)
    st = _load().mi_device_check(int(device), buf, 256)
    return st == 0, buf.value.decode()


def available():
    """True if the HIP scans can run here, else a reason string (the page's
    available() contract)."""
    try:
        _load()
    except (ImportError, OSError) as e:
        return "libmiscan not loadable: %s" % e
    if not torch.cuda.is_available():
        return "no GPU visible to torch"
    ok, reason = mi_device_check(torch.cuda.current_device())
    return True if ok else reason


# ---------------------------------------------------------------------------
# marshalling helpers
# ---------------------------------------------------------------------------

def _dt(t: torch.Tensor) -> int:
    try:
        return _DTYPES[t.dtype]
    except KeyError:
        raise TypeError("unsupported dtype %s (float32, bfloat16 or float16)" % t.dtype) from None


def _dev_tensor(t: torch.Tensor, name: str) -> torch.Tensor:
    if not isinstance(t, torch.Tensor):
        raise TypeError("%s must be a torch.Tensor" % name)
    if not t.is_cuda:
        raise ValueError("%s must be a GPU tensor (the scans run only on the GPU)" % name)
    return t.contiguous()


def _out(t, like: torch.Tensor, name: str) -> torch.Tensor:
    if t is None:
        return torch.empty_like(like)
    if t.shape != like.shape or t.dtype != like.dtype or t.device != like.device or not t.is_contiguous():
        raise ValueError("%s must be a contiguous %s tensor of shape %s on %s"
                         % (name, like.dtype, tuple(like.shape), like.device))
    return t


# Checked mode: after every call, wait for the stream and raise if a
# cross-workgroup wait gave up (word 1 of the workspace, zero after every
# correct run).  Off by default (it synchronises); the environment variable
# MISCAN_CHECK=1 or set_checked(True) turns it on.
_checked = os.environ.get("MISCAN_CHECK", "0") not in ("", "0")


def set_checked(on: bool = True):
    """Turn checked mode (synchronise and verify the workspace after each call) on or off."""
    global _checked
    _checked = bool(on)


def workspace_timeouts(ws: torch.Tensor) -> int:
    """Cross-workgroup waits that hit their spin limit during the last call that
    used workspace `ws` (word 1; synchronises with the device)."""
    return int(ws[4:8].cpu().view(torch.int32).item())


class _Call:
    """Stream and device context of one library call.

    The kernels run on `stream` (default: torch's current stream).  When it is
    another stream, it first waits for the current one (so inputs produced
    there are ready), every tensor the call allocates (contiguous copies,
    outputs, workspace) is allocated on it, and every caller tensor it touches
    is recorded on it, so the caching allocator reuses none of that memory
    before the kernels are done.
    """

    def __init__(self, stream, device):
        self.device = device
        cur = torch.cuda.current_stream(device)
        self.side = stream is not None and stream != cur
        self.stream = stream if self.side else cur
        if self.side:
            self.stream.wait_stream(cur)
        self._ctx = contextlib.ExitStack()

    def __enter__(self):
        self._ctx.enter_context(torch.cuda.device(self.device))
        if self.side:
            self._ctx.enter_context(torch.cuda.stream(self.stream))
        return self

    def __exit__(self, *exc):
        return self._ctx.__exit__(*exc)

    def keep(self, *ts):
        """Record caller tensors on a side stream."""
        if self.side:
            for t in ts:
                if t is not None and t.numel():
                    t.record_stream(self.stream)

    @property
    def handle(self) -> int:
        return self.stream.cuda_stream


def _workspace(ws, nbytes: int, device):
    if ws is None:
        return torch.empty(max(int(nbytes), 8), dtype=torch.uint8, device=device)
    if ws.device != device or ws.numel() * ws.element_size() < nbytes:
        raise ValueError("workspace too small: %d bytes needed" % nbytes)
    return ws


def _check(st: int, where: str, call=None, ws=None):
    if st != 0:
        raise MiscanError(st, where)
    # (a call with nothing to scan launches no scan and leaves ws untouched)
    if _checked and call is not None and ws is not None and ws.numel() >= 8:
        call.stream.synchronize()
        n = workspace_timeouts(ws)
        if n:
            raise RuntimeError("%s: %d cross-workgroup wait(s) hit the spin limit; the result is not valid"
                               % (where, n))


def _nonempty(t: torch.Tensor) -> bool:
    return t.numel() > 0


def _same(ref: torch.Tensor, *ts):
    for t in ts:
        if t.device != ref.device or t.dtype != ref.dtype:
            raise ValueError("all tensors must share device and dtype (%s, %s)" % (ref.device, ref.dtype))


# ---------------------------------------------------------------------------
# k = 1 channel scan
# ---------------------------------------------------------------------------

def _device(t, name: str):
    if not isinstance(t, torch.Tensor):
        raise TypeError("%s must be a torch.Tensor" % name)
    if not t.is_cuda:
        raise ValueError("%s must be a GPU tensor (the scans run only on the GPU)" % name)
    return t.device


def _nbytes(t) -> int:
    return t.numel() * t.element_size()


def mi_linear_scan_workspace(B: int, T: int, D: int, dtype=torch.float32) -> int:
    return int(_load().mi_linear_scan_workspace(B, T, D, _DTYPES[dtype]))


def mi_linear_scan_fwd(a, b, A=None, Bc=None, *, ws=None, stream=None):
    """(A, Bc) = linear_scan_fwd(a, b); a, b (B, T, D) float32 or bfloat16.

    Runs on `stream` (default: torch's current stream); see _Call for how a
    side stream is ordered against the current one."""
    with _Call(stream, _device(a, "a")) as c:
        a, b = _dev_tensor(a, "a"), _dev_tensor(b, "b")
        if a.dim() != 3 or b.shape != a.shape:
            raise ValueError("a and b must both be (B, T, D)")
        _same(a, b)
        A, Bc = _out(A, a, "A"), _out(Bc, a, "Bc")
        Bn, T, D = a.shape
        dt = _dt(a)
        ws = _workspace(ws, _load().mi_linear_scan_workspace(Bn, T, D, dt), a.device)
        c.keep(a, b, A, Bc, ws)
        st = _load().mi_linear_scan_fwd(a.data_ptr(), b.data_ptr(), A.data_ptr(), Bc.data_ptr(),
                                        Bn, T, D, dt, ws.data_ptr(), _nbytes(ws), c.handle)
        _check(st, "mi_linear_scan_fwd", c, ws if _nonempty(a) else None)
    return A, Bc


def mi_linear_scan_bwd(a, A, Bc, gA, gBc, da=None, db=None, *, ws=None, stream=None):
    """(da, db) = linear_scan_bwd(a, A, Bc, gA, gBc); all (B, T, D)."""
    with _Call(stream, _device(a, "a")) as c:
        a, A, Bc, gA, gBc = (_dev_tensor(t, n) for t, n in
                             ((a, "a"), (A, "A"), (Bc, "Bc"), (gA, "gA"), (gBc, "gBc")))
        if a.dim() != 3 or any(t.shape != a.shape for t in (A, Bc, gA, gBc)):
            raise ValueError("a, A, Bc, gA, gBc must all be (B, T, D)")
        _same(a, A, Bc, gA, gBc)
        da, db = _out(da, a, "da"), _out(db, a, "db")
        Bn, T, D = a.shape
        dt = _dt(a)
        ws = _workspace(ws, _load().mi_linear_scan_workspace(Bn, T, D, dt), a.device)
        c.keep(a, A, Bc, gA, gBc, da, db, ws)
        st = _load().mi_linear_scan_bwd(a.data_ptr(), A.data_ptr(), Bc.data_ptr(), gA.data_ptr(),
                                        gBc.data_ptr(), da.data_ptr(), db.data_ptr(), Bn, T, D, dt,
                                        ws.data_ptr(), _nbytes(ws), c.handle)
        _check(st, "mi_linear_scan_bwd", c, ws if _nonempty(a) else None)
    return da, db


def mi_linear_scan_fwd_noalloc(a, b, A=None, Bc=None, *, stream=None):
    """(A, Bc) = linear_scan_fwd(a, b) through the entry point that allocates
    nothing: its look-back state lives in the library's fixed per-device
    scratch array (NOALLOC_SCRATCH_BYTES).  Calls that overlap on one GPU
    share that array and must not run concurrently."""
    with _Call(stream, _device(a, "a")) as c:
        a, b = _dev_tensor(a, "a"), _dev_tensor(b, "b")
        if a.dim() != 3 or b.shape != a.shape:
            raise ValueError("a and b must both be (B, T, D)")
        _same(a, b)
        A, Bc = _out(A, a, "A"), _out(Bc, a, "Bc")
        Bn, T, D = a.shape
        c.keep(a, b, A, Bc)
        st = _load().mi_linear_scan_fwd_noalloc(a.data_ptr(), b.data_ptr(), A.data_ptr(), Bc.data_ptr(),
                                                Bn, T, D, _dt(a), c.handle)
        _check(st, "mi_linear_scan_fwd_noalloc")
    return A, Bc


def _state(t, like: torch.Tensor, shape, name: str):
    """Optional initial state (None = zero); same device and dtype as `like`."""
    if t is None:
        return None
    t = _dev_tensor(t, name)
    if tuple(t.shape) != tuple(shape) or t.dtype != like.dtype or t.device != like.device:
        raise ValueError("%s must be a %s tensor of shape %s on %s" % (name, like.dtype, tuple(shape), like.device))
    return t


def _ptr(t):
    return None if t is None else t.data_ptr()


def mi_linear_scan_fwd_h0(a, b, h0=None, A=None, H=None, *, ws=None, stream=None):
    """(A, H): the scan from the initial state h0 (B, D) (None = zero);
    H_t = a_t H_{t-1} + b_t with H_0 = h0.  The final state is (A[:, -1], H[:, -1])."""
    with _Call(stream, _device(a, "a")) as c:
        a, b = _dev_tensor(a, "a"), _dev_tensor(b, "b")
        if a.dim() != 3 or b.shape != a.shape:
            raise ValueError("a and b must both be (B, T, D)")
        _same(a, b)
        Bn, T, D = a.shape
        h0 = _state(h0, a, (Bn, D), "h0")
        A, H = _out(A, a, "A"), _out(H, a, "H")
        dt = _dt(a)
        ws = _workspace(ws, _load().mi_linear_scan_workspace(Bn, T, D, dt), a.device)
        c.keep(a, b, h0, A, H, ws)
        st = _load().mi_linear_scan_fwd_h0(a.data_ptr(), b.data_ptr(), _ptr(h0), A.data_ptr(), H.data_ptr(),
                                           Bn, T, D, dt, ws.data_ptr(), _nbytes(ws), c.handle)
        _check(st, "mi_linear_scan_fwd_h0", c, ws if _nonempty(a) else None)
    return A, H


def mi_linear_scan_bwd_h0(a, A, H, h0, gA, gH, da=None, db=None, dh0=None, *, ws=None, stream=None):
    """(da, db, dh0): gradient of mi_linear_scan_fwd_h0 for upstream grads gA, gH."""
    with _Call(stream, _device(a, "a")) as c:
        a, A, H, gA, gH = (_dev_tensor(t, n) for t, n in ((a, "a"), (A, "A"), (H, "H"), (gA, "gA"), (gH, "gH")))
        if a.dim() != 3 or any(t.shape != a.shape for t in (A, H, gA, gH)):
            raise ValueError("a, A, H, gA, gH must all be (B, T, D)")
        _same(a, A, H, gA, gH)
        Bn, T, D = a.shape
        h0 = _state(h0, a, (Bn, D), "h0")
        da, db = _out(da, a, "da"), _out(db, a, "db")
        dh0 = _out(dh0, a.new_empty((Bn, D)), "dh0")
        dt = _dt(a)
        ws = _workspace(ws, _load().mi_linear_scan_workspace(Bn, T, D, dt), a.device)
        c.keep(a, A, H, h0, gA, gH, da, db, dh0, ws)
        st = _load().mi_linear_scan_bwd_h0(a.data_ptr(), A.data_ptr(), H.data_ptr(), _ptr(h0), gA.data_ptr(),
                                           gH.data_ptr(), da.data_ptr(), db.data_ptr(), dh0.data_ptr(), Bn, T, D,
                                           dt, ws.data_ptr(), _nbytes(ws), c.handle)
        _check(st, "mi_linear_scan_bwd_h0", c, ws if _nonempty(a) else None)
    return da, db, dh0


# ---------------------------------------------------------------------------
# log-space scan
# ---------------------------------------------------------------------------

def mi_scan_log_workspace(B: int, T: int, D: int, dtype=torch.float32) -> int:
    return int(_load().mi_scan_log_workspace(B, T, D, _DTYPES[dtype]))


def mi_scan_log_fwd(log_coeffs, log_values, h=None, *, ws=None, stream=None):
    """h (B, T, D) = parallel_scan_log_fwd(log_coeffs (B,T,D), log_values (B,T+1,D))."""
    with _Call(stream, _device(log_coeffs, "log_coeffs")) as c:
        lc, lv = _dev_tensor(log_coeffs, "log_coeffs"), _dev_tensor(log_values, "log_values")
        if lc.dim() != 3 or lv.dim() != 3 or lv.shape != (lc.shape[0], lc.shape[1] + 1, lc.shape[2]):
            raise ValueError("log_coeffs must be (B, T, D) and log_values (B, T+1, D)")
        _same(lc, lv)
        h = _out(h, lc, "h")
        Bn, T, D = lc.shape
        dt = _dt(lc)
        ws = _workspace(ws, _load().mi_scan_log_workspace(Bn, T, D, dt), lc.device)
        c.keep(lc, lv, h, ws)
        st = _load().mi_scan_log_fwd(lc.data_ptr(), lv.data_ptr(), h.data_ptr(), Bn, T, D, dt,
                                     ws.data_ptr(), _nbytes(ws), c.handle)
        _check(st, "mi_scan_log_fwd", c, ws if _nonempty(lc) else None)
    return h


def mi_scan_log_bwd(log_coeffs, log_values, h, g, dlog_coeffs=None, dlog_values=None, *, ws=None, stream=None):
    """(dlog_coeffs (B,T,D), dlog_values (B,T+1,D)): gradient of parallel_scan_log_fwd
    given its output h (B,T,D) and the upstream gradient g = dL/dh (B,T,D)."""
    with _Call(stream, _device(log_coeffs, "log_coeffs")) as c:
        lc, lv = _dev_tensor(log_coeffs, "log_coeffs"), _dev_tensor(log_values, "log_values")
        h, g = _dev_tensor(h, "h"), _dev_tensor(g, "g")
        if lc.dim() != 3 or lv.dim() != 3 or lv.shape != (lc.shape[0], lc.shape[1] + 1, lc.shape[2]):
            raise ValueError("log_coeffs must be (B, T, D) and log_values (B, T+1, D)")
        if h.shape != lc.shape or g.shape != lc.shape:
            raise ValueError("h and g must be (B, T, D)")
        _same(lc, lv, h, g)
        dlc, dlv = _out(dlog_coeffs, lc, "dlog_coeffs"), _out(dlog_values, lv, "dlog_values")
        Bn, T, D = lc.shape
        dt = _dt(lc)
        ws = _workspace(ws, _load().mi_scan_log_workspace(Bn, T, D, dt), lc.device)
        c.keep(lc, lv, h, g, dlc, dlv, ws)
        st = _load().mi_scan_log_bwd(lc.data_ptr(), lv.data_ptr(), h.data_ptr(), g.data_ptr(), dlc.data_ptr(),
                                     dlv.data_ptr(), Bn, T, D, dt, ws.data_ptr(), _nbytes(ws), c.handle)
        _check(st, "mi_scan_log_bwd", c, ws if _nonempty(lc) else None)
    return dlc, dlv


# ---------------------------------------------------------------------------
# k x k matrix-affine scan
# ---------------------------------------------------------------------------

def mi_affine_scan_workspace(B: int, T: int, n: int, k: int, v: int, dtype=torch.float32) -> int:
    return int(_load().mi_affine_scan_workspace(B, T, n, k, v, _DTYPES[dtype]))


def _affine_shapes(A, Bm):
    if A.dim() != 5 or A.shape[3] != A.shape[4]:
        raise ValueError("A must be (B, T, n, k, k)")
    if Bm.dim() != 5 or Bm.shape[:4] != A.shape[:4]:
        raise ValueError("Bm/Bbar must be (B, T, n, k, v) with the B, T, n, k of A")
    Bn, T, n, k, _ = A.shape
    return Bn, T, n, k, Bm.shape[4]


def mi_affine_scan_fwd(A, Bm, Abar=None, Bbar=None, *, ws=None, stream=None):
    """(Abar, Bbar) = affine_scan_fwd(A (B,T,n,k,k), Bm (B,T,n,k,v))."""
    with _Call(stream, _device(A, "A")) as c:
        A, Bm = _dev_tensor(A, "A"), _dev_tensor(Bm, "Bm")
        _same(A, Bm)
        Bn, T, n, k, v = _affine_shapes(A, Bm)
        Abar, Bbar = _out(Abar, A, "Abar"), _out(Bbar, Bm, "Bbar")
        dt = _dt(A)
        ws = _workspace(ws, _load().mi_affine_scan_workspace(Bn, T, n, k, v, dt), A.device)
        c.keep(A, Bm, Abar, Bbar, ws)
        st = _load().mi_affine_scan_fwd(A.data_ptr(), Bm.data_ptr(), Abar.data_ptr(), Bbar.data_ptr(),
                                        Bn, T, n, k, v, dt, ws.data_ptr(), _nbytes(ws), c.handle)
        _check(st, "mi_affine_scan_fwd", c, ws if _nonempty(A) else None)
    return Abar, Bbar


def mi_affine_scan_bwd(A, Abar, Bbar, gAbar, gBbar, dA=None, dB=None, *, ws=None, stream=None):
    """(dA, dB) = affine_scan_bwd(A, Abar, Bbar, gAbar, gBbar)."""
    with _Call(stream, _device(A, "A")) as c:
        A, Abar, Bbar, gAbar, gBbar = (_dev_tensor(t, nm) for t, nm in
                                       ((A, "A"), (Abar, "Abar"), (Bbar, "Bbar"),
                                        (gAbar, "gAbar"), (gBbar, "gBbar")))
        _same(A, Abar, Bbar, gAbar, gBbar)
        Bn, T, n, k, v = _affine_shapes(A, Bbar)
        if Abar.shape != A.shape or gAbar.shape != A.shape or gBbar.shape != Bbar.shape:
            raise ValueError("Abar, gAbar must match A; gBbar must match Bbar")
        dA, dB = _out(dA, A, "dA"), _out(dB, Bbar, "dB")
        dt = _dt(A)
        ws = _workspace(ws, _load().mi_affine_scan_workspace(Bn, T, n, k, v, dt), A.device)
        c.keep(A, Abar, Bbar, gAbar, gBbar, dA, dB, ws)
        st = _load().mi_affine_scan_bwd(A.data_ptr(), Abar.data_ptr(), Bbar.data_ptr(),
                                        gAbar.data_ptr(), gBbar.data_ptr(), dA.data_ptr(),
                                        dB.data_ptr(), Bn, T, n, k, v, dt, ws.data_ptr(),
                                        _nbytes(ws), c.handle)
        _check(st, "mi_affine_scan_bwd", c, ws if _nonempty(A) else None)
    return dA, dB


def mi_affine_scan_fwd_h0(A, Bm, H0=None, Abar=None, H=None, *, ws=None, stream=None):
    """(Abar, H): the k x k scan from X_0 = [I | H0], H0 (B, n, k, v) (None = zero)."""
    with _Call(stream, _device(A, "A")) as c:
        A, Bm = _dev_tensor(A, "A"), _dev_tensor(Bm, "Bm")
        _same(A, Bm)
        Bn, T, n, k, v = _affine_shapes(A, Bm)
        H0 = _state(H0, A, (Bn, n, k, v), "H0")
        Abar, H = _out(Abar, A, "Abar"), _out(H, Bm, "H")
        dt = _dt(A)
        ws = _workspace(ws, _load().mi_affine_scan_workspace(Bn, T, n, k, v, dt), A.device)
        c.keep(A, Bm, H0, Abar, H, ws)
        st = _load().mi_affine_scan_fwd_h0(A.data_ptr(), Bm.data_ptr(), _ptr(H0), Abar.data_ptr(), H.data_ptr(),
                                           Bn, T, n, k, v, dt, ws.data_ptr(), _nbytes(ws), c.handle)
        _check(st, "mi_affine_scan_fwd_h0", c, ws if _nonempty(A) else None)
    return Abar, H


def mi_affine_scan_bwd_h0(A, Abar, H, H0, gAbar, gH, dA=None, dB=None, dH0=None, *, ws=None, stream=None):
    """(dA, dB, dH0): gradient of mi_affine_scan_fwd_h0."""
    with _Call(stream, _device(A, "A")) as c:
        A, Abar, H, gAbar, gH = (_dev_tensor(t, nm) for t, nm in
                                 ((A, "A"), (Abar, "Abar"), (H, "H"), (gAbar, "gAbar"), (gH, "gH")))
        _same(A, Abar, H, gAbar, gH)
        Bn, T, n, k, v = _affine_shapes(A, H)
        if Abar.shape != A.shape or gAbar.shape != A.shape or gH.shape != H.shape:
            raise ValueError("Abar, gAbar must match A; gH must match H")
        H0 = _state(H0, A, (Bn, n, k, v), "H0")
        dA, dB = _out(dA, A, "dA"), _out(dB, H, "dB")
        dH0 = _out(dH0, A.new_empty((Bn, n, k, v)), "dH0")
        dt = _dt(A)
        ws = _workspace(ws, _load().mi_affine_scan_workspace(Bn, T, n, k, v, dt), A.device)
        c.keep(A, Abar, H, H0, gAbar, gH, dA, dB, dH0, ws)
        st = _load().mi_affine_scan_bwd_h0(A.data_ptr(), Abar.data_ptr(), H.data_ptr(), _ptr(H0),
                                           gAbar.data_ptr(), gH.data_ptr(), dA.data_ptr(), dB.data_ptr(),
                                           dH0.data_ptr(), Bn, T, n, k, v, dt, ws.data_ptr(), _nbytes(ws),
                                           c.handle)
        _check(st, "mi_affine_scan_bwd_h0", c, ws if _nonempty(A) else None)
    return dA, dB, dH0


# Op names of the minGRU "Triton kernels" page (same arguments and returns).
def linear_scan_fwd(a, b):
    return mi_linear_scan_fwd(a, b)


def linear_scan_bwd(a, A, Bc, gA, gBc):
    return mi_linear_scan_bwd(a, A, Bc, gA, gBc)


def parallel_scan_log_fwd(log_coeffs, log_values):
    return mi_scan_log_fwd(log_coeffs, log_values)


def parallel_scan_log_bwd(log_coeffs, log_values, h, g):
    """Adjoint of parallel_scan_log_fwd (not an op of the page: added for training)."""
    return mi_scan_log_bwd(log_coeffs, log_values, h, g)


def affine_scan_fwd(A, Bm):
    return mi_affine_scan_fwd(A, Bm)


def affine_scan_bwd(A, Abar, Bbar, gAbar, gBbar):
    return mi_affine_scan_bwd(A, Abar, Bbar, gAbar, gBbar)
