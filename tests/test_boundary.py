"""C-ABI boundary checks that need no GPU.

The library must load, export every function include/miscan.h declares, and
reject bad arguments with the documented status *before* anything is launched.
Every call below is built to fail validation (or to be a zero-sized no-op), so
no kernel is ever enqueued and the fake pointers are never dereferenced.
"""
import ctypes
import os
import re

import pytest

import linear_recurrence_scans_amd as lrs

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "miscan.h")

(MI_OK, MI_ERR_INVALID_ARG, MI_ERR_UNSUPPORTED, MI_ERR_WORKSPACE, MI_ERR_LAUNCH, MI_ERR_DEVICE,
 MI_ERR_CAPACITY) = range(7)
F32, BF16, F16 = 0, 1, 2
P = 1 << 20        # fake, 256-byte aligned "device" addresses; never dereferenced
STEP = 1 << 30     # far apart: no overlap unless a test wants one


def lib():
    return lrs._load()


def declared_functions(header=HEADER):
    text = open(header).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(mi_[a-z0-9_]+)\s*\(", text)))


def test_bench_header_symbols_exported():
    """include/miscan_bench.h is the ABI of the benchmark's probe library."""
    from linear_recurrence_scans_amd import build as B
    names = declared_functions(os.path.join(ROOT, "include", "miscan_bench.h"))
    assert names == ["mi_bench_flush", "mi_bench_stream"], names
    so = ctypes.CDLL(B.BENCH_LIB)
    for n in names:
        assert hasattr(so, n), "libmiscan_bench.so does not export %s" % n
    # every header under include/ is covered by one of the two checks
    headers = sorted(f for f in os.listdir(os.path.join(ROOT, "include")) if f.endswith(".h"))
    assert headers == ["miscan.h", "miscan_bench.h"], headers
    # argument errors are reported before anything is enqueued
    V = ctypes.c_void_p
    arr = (V * 5)(*[P + i * STEP for i in range(5)])
    so.mi_bench_stream.argtypes = [ctypes.POINTER(V), ctypes.c_int, ctypes.POINTER(V), ctypes.c_int,
                                   ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, ctypes.c_int, V]
    assert so.mi_bench_stream(arr, 3, arr, 2, 1, 4, 64, F32, None) == MI_ERR_UNSUPPORTED  # (3, 2) not built
    assert so.mi_bench_stream(arr, 2, arr, 2, 0, 4, 64, F32, None) == MI_ERR_INVALID_ARG
    so.mi_bench_flush.argtypes = [V, ctypes.c_size_t, V]
    assert so.mi_bench_flush(None, 1 << 20, None) == MI_ERR_INVALID_ARG


def test_header_symbols_exported():
    names = declared_functions()
    assert len(names) >= 10, names
    so = ctypes.CDLL(lrs.library_path())
    for n in names:
        assert hasattr(so, n), "libmiscan.so does not export %s" % n
    # the binding wraps every declared entry point under the same name
    for n in names:
        assert hasattr(lrs, n), "binding lacks %s" % n


def test_status_strings():
    for code in range(7):
        s = lrs.mi_status_string(code)
        assert s.startswith("MI_"), s
    assert "unknown" in lrs.mi_status_string(99)


def ptrs(n, base=P):
    return [base + i * STEP for i in range(n)]


def fwd(a, b, A, Bc, Bn, T, D, dt=F32, ws=None, wsb=0):
    return lib().mi_linear_scan_fwd(a, b, A, Bc, Bn, T, D, dt, ws, wsb, None)


def test_linear_fwd_validation():
    a, b, A, Bc, ws = ptrs(5)
    big = 1 << 40
    assert fwd(a, b, A, Bc, -1, 4, 4) == MI_ERR_INVALID_ARG                 # negative size
    assert fwd(None, b, A, Bc, 1, 4, 4, ws=ws, wsb=big) == MI_ERR_INVALID_ARG  # null pointer
    assert fwd(a, b, A, Bc, 1, 4, 4, dt=7) == MI_ERR_UNSUPPORTED            # unknown dtype
    assert fwd(a + 2, b, A, Bc, 1, 4, 4, ws=ws, wsb=big) == MI_ERR_INVALID_ARG  # misaligned f32
    assert fwd(a + 2, b, A, Bc, 1, 4, 4, dt=BF16, ws=None) == MI_ERR_WORKSPACE  # bf16 aligned ok
    assert fwd(a + 2, b, A, Bc, 1, 4, 4, dt=F16, ws=None) == MI_ERR_WORKSPACE   # fp16 too
    assert fwd(a + 1, b, A, Bc, 1, 4, 4, dt=F16, ws=ws, wsb=big) == MI_ERR_INVALID_ARG  # odd address
    assert fwd(a, b, A, Bc, 1, 4, 4, dt=3) == MI_ERR_UNSUPPORTED
    assert fwd(a, b, a + 8, Bc, 1, 4, 4, ws=ws, wsb=big) == MI_ERR_INVALID_ARG  # output overlaps input
    assert fwd(a, b, A, A + 4, 1, 4, 4, ws=ws, wsb=big) == MI_ERR_INVALID_ARG  # outputs overlap
    assert fwd(a, b, A, Bc, 1, 4, 4, ws=None) == MI_ERR_WORKSPACE           # no workspace
    need = lib().mi_linear_scan_workspace(1, 4, 4, F32)
    assert need > 0
    assert fwd(a, b, A, Bc, 1, 4, 4, ws=ws, wsb=need - 1) == MI_ERR_WORKSPACE
    assert fwd(a, b, A, Bc, 1, 4, 4, ws=ws + 16, wsb=big) == MI_ERR_INVALID_ARG  # ws not 256-aligned
    assert fwd(a, b, A, Bc, 1, 4, 4, ws=a + 64, wsb=big) == MI_ERR_INVALID_ARG   # ws overlaps a
    # int64 overflow of the byte size
    assert fwd(a, b, A, Bc, 1 << 40, 1 << 20, 1 << 10) == MI_ERR_INVALID_ARG


def test_zero_sized_problems_launch_nothing():
    # zero-sized axes: MI_OK with null pointers and no workspace
    assert fwd(None, None, None, None, 0, 5, 5) == MI_OK
    assert fwd(None, None, None, None, 2, 0, 5) == MI_OK
    assert fwd(None, None, None, None, 2, 5, 0) == MI_OK
    L = lib()
    assert L.mi_linear_scan_bwd(*([None] * 7), 3, 0, 2, BF16, None, 0, None) == MI_OK
    assert L.mi_scan_log_fwd(None, None, None, 0, 3, 3, F32, None, 0, None) == MI_OK
    assert L.mi_affine_scan_fwd(None, None, None, None, 1, 0, 2, 4, 4, F32, None, 0, None) == MI_OK
    assert L.mi_affine_scan_bwd(*([None] * 7), 1, 2, 0, 4, 4, F32, None, 0, None) == MI_OK
    assert L.mi_linear_scan_workspace(0, 5, 5, F32) == 0


def test_linear_bwd_validation():
    L = lib()
    p = ptrs(8)
    assert L.mi_linear_scan_bwd(*p[:7], 1, 8, 8, F32, None, 0, None) == MI_ERR_WORKSPACE
    q = list(p[:7])
    q[6] = q[0]  # db aliases a
    assert L.mi_linear_scan_bwd(*q, 1, 8, 8, F32, p[7], 1 << 40, None) == MI_ERR_INVALID_ARG
    q = list(p[:7])
    q[3] = None
    assert L.mi_linear_scan_bwd(*q, 1, 8, 8, F32, p[7], 1 << 40, None) == MI_ERR_INVALID_ARG


def test_log_validation():
    L = lib()
    lc, lv, h, ws = ptrs(4)
    assert L.mi_scan_log_fwd(lc, lv, h, 2, 8, 8, F32, None, 0, None) == MI_ERR_WORKSPACE
    # h overlapping log_values' last row (log_values has T+1 rows)
    assert L.mi_scan_log_fwd(lc, lv, lv + 2 * 8 * 8 * 4, 2, 8, 8, F32, ws, 1 << 40, None) == MI_ERR_INVALID_ARG
    assert L.mi_scan_log_fwd(lc, lv, h, 2, 8, 8, 5, None, 0, None) == MI_ERR_UNSUPPORTED


def test_log_bwd_validation():
    L = lib()
    lc, lv, h, g, dlc, dlv, ws = ptrs(7)
    args = lambda **kw: [kw.get(k, v) for k, v in
                         (("lc", lc), ("lv", lv), ("h", h), ("g", g), ("dlc", dlc), ("dlv", dlv))]
    assert L.mi_scan_log_bwd(*args(), 2, 8, 8, F32, None, 0, None) == MI_ERR_WORKSPACE
    # dlog_values (T+1 rows) overlapping the start of g
    assert L.mi_scan_log_bwd(*args(dlv=g - 8 * 4), 2, 8, 8, F32, ws, 1 << 40, None) == MI_ERR_INVALID_ARG
    # dlog_coeffs aliasing h
    assert L.mi_scan_log_bwd(*args(dlc=h), 2, 8, 8, F32, ws, 1 << 40, None) == MI_ERR_INVALID_ARG
    assert L.mi_scan_log_bwd(*args(g=None), 2, 8, 8, F32, ws, 1 << 40, None) == MI_ERR_INVALID_ARG
    assert L.mi_scan_log_bwd(*args(), 2, 8, 8, 5, ws, 1 << 40, None) == MI_ERR_UNSUPPORTED
    assert L.mi_scan_log_bwd(*args(), 0, 5, 8, F32, None, 0, None) == MI_OK  # B = 0: nothing to do
    # T = 0 still zeroes dlog_values' slot 0 (a launch), but checks its pointer first
    assert L.mi_scan_log_bwd(*args(dlv=None), 2, 0, 8, F32, None, 0, None) == MI_ERR_INVALID_ARG


def test_initial_state_validation():
    L = lib()
    a, b, h0, A, H, ws = ptrs(6)
    # h0 may be NULL (zero state); outputs must not overlap it
    assert L.mi_linear_scan_fwd_h0(a, b, h0, A, H, 2, 8, 8, F32, None, 0, None) == MI_ERR_WORKSPACE
    assert L.mi_linear_scan_fwd_h0(a, b, None, A, H, 2, 8, 8, F32, None, 0, None) == MI_ERR_WORKSPACE
    assert L.mi_linear_scan_fwd_h0(a, b, h0, A, h0, 2, 8, 8, F32, ws, 1 << 40, None) == MI_ERR_INVALID_ARG
    q = ptrs(10)
    # dh0 aliasing h0
    assert L.mi_linear_scan_bwd_h0(*q[:8], q[3], 2, 8, 8, F32, q[9], 1 << 40, None) == MI_ERR_INVALID_ARG
    assert L.mi_linear_scan_bwd_h0(*q[:8], None, 2, 8, 8, F32, q[9], 1 << 40, None) == MI_ERR_INVALID_ARG
    # T = 0 still zeroes dh0 (a launch) after checking its pointer
    assert L.mi_linear_scan_bwd_h0(*q[:8], None, 2, 0, 8, F32, None, 0, None) == MI_ERR_INVALID_ARG
    r = ptrs(10)
    assert L.mi_affine_scan_fwd_h0(*r[:5], 1, 4, 2, 4, 8, F32, None, 0, None) == MI_ERR_WORKSPACE
    assert L.mi_affine_scan_fwd_h0(*r[:5], 1, 4, 2, 17, 8, F32, None, 0, None) == MI_ERR_UNSUPPORTED
    assert L.mi_affine_scan_bwd_h0(*r[:8], r[3], 1, 4, 2, 4, 8, F32, r[9], 1 << 40, None) == MI_ERR_INVALID_ARG
    assert L.mi_affine_scan_bwd_h0(*r[:8], None, 1, 0, 2, 4, 8, F32, None, 0, None) == MI_ERR_INVALID_ARG


def test_affine_plan_whole_envelope():
    """The k x k host planning (column tiling, waves, LDS budget) runs for every
    k in [1, 16] and v in [1, 128], forward and backward: the workspace query
    drives the same code as the launchers and must return a size for each."""
    L = lib()
    for k in range(1, 17):
        for v in range(1, 129):
            assert L.mi_affine_scan_workspace(2, 37, 3, k, v, F32) > 0, (k, v)


def test_affine_envelope():
    L = lib()
    A, Bm, Ab, Bb, ws = ptrs(5)
    call = lambda k, v, dt=F32, w=None, wb=0: L.mi_affine_scan_fwd(A, Bm, Ab, Bb, 1, 4, 2, k, v, dt, w, wb, None)
    assert call(0, 4) == MI_ERR_UNSUPPORTED
    assert call(17, 4) == MI_ERR_UNSUPPORTED
    assert call(4, 0) == MI_ERR_UNSUPPORTED
    assert call(4, 129) == MI_ERR_UNSUPPORTED
    assert call(4, 4, BF16) == MI_ERR_WORKSPACE      # bf16 storage is inside the envelope
    assert call(4, 4, F16) == MI_ERR_WORKSPACE       # and fp16
    assert call(4, 4, 7) == MI_ERR_UNSUPPORTED       # unknown dtype
    assert call(16, 128) == MI_ERR_WORKSPACE        # inside the envelope
    assert call(1, 1) == MI_ERR_WORKSPACE
    assert L.mi_affine_scan_workspace(1, 4, 2, 17, 4, F32) == 0
    assert L.mi_affine_scan_bwd(A, Ab, Bb, Bm, Bm, ws, ws, 1, 4, 2, 4, 4, F32, P, 1 << 40, None) == MI_ERR_INVALID_ARG
    # head indices (B * n) run in 32 bits in the kernels: 2^31 heads or more are
    # refused by the plan, before anything is launched
    # (tensors of 128 GiB: fake pointers 1 TiB apart)
    G = [P + i * (1 << 40) for i in range(8)]
    wsz = L.mi_affine_scan_workspace(1 << 16, 1, 1 << 15, 4, 4, F32)
    assert L.mi_affine_scan_fwd(G[0], G[1], G[2], G[3], 1 << 16, 1, 1 << 15, 4, 4, F32, G[7], wsz,
                                None) == MI_ERR_UNSUPPORTED
    assert L.mi_affine_scan_bwd(G[0], G[2], G[3], G[4], G[5], G[1], G[6], 1 << 16, 1, 1 << 15, 4, 4, F32, G[7],
                                wsz, None) == MI_ERR_UNSUPPORTED


def test_workspace_sizes_cover_every_shape():
    L = lib()
    for Bn, T, D in ((1, 1, 1), (1, 1024, 64), (8, 8192, 4096), (3, 1000, 100)):
        for dt in (F32, BF16, F16):
            w = L.mi_linear_scan_workspace(Bn, T, D, dt)
            assert w >= 256 + 256
            assert L.mi_scan_log_workspace(Bn, T, D, dt) >= 512
    for args in ((2, 2048, 64, 4, 16), (4, 4096, 32, 8, 32), (1, 1, 1, 1, 1), (1, 7, 3, 16, 128), (2, 5, 3, 3, 5)):
        assert L.mi_affine_scan_workspace(*args, F32) > 0
    # larger problems never need less
    assert L.mi_linear_scan_workspace(8, 8192, 4096, BF16) > L.mi_linear_scan_workspace(8, 4096, 4096, BF16)


def test_binding_refuses_cpu_tensors():
    torch = pytest.importorskip("torch")
    a = torch.rand(1, 4, 4)
    with pytest.raises(ValueError, match="GPU"):
        lrs.linear_scan_fwd(a, a)
    with pytest.raises(ValueError, match="GPU"):
        lrs.parallel_scan_log_fwd(a, torch.rand(1, 5, 4))


def test_available_reports_reason_without_gpu():
    torch = pytest.importorskip("torch")
    r = lrs.available()
    if not torch.cuda.is_available():
        assert isinstance(r, str) and r


def test_product_path_does_not_import_oracle():
    """The HIP binding never imports or links the oracle."""
    pkg = os.path.join(ROOT, "linear_recurrence_scans_amd")
    for dirpath, _, files in os.walk(pkg):
        for f in files:
            if f.endswith((".py", ".hip", ".hpp", ".cpp", ".h")):
                text = open(os.path.join(dirpath, f)).read()
                assert "import oracle" not in text and "from oracle" not in text, f
                assert "lrs_oracle" not in text and "liboracle" not in text, f


def test_noalloc_checks_before_any_device_call():
    """The no-allocation forward validates like mi_linear_scan_fwd and rejects a
    problem larger than its fixed scratch with MI_ERR_CAPACITY, all before it
    touches a device (no GPU here)."""
    L = lib()
    a, b, A, Bc = ptrs(4)
    call = lambda *args: L.mi_linear_scan_fwd_noalloc(*args, None)
    assert call(None, None, None, None, 0, 5, 5, F32) == MI_OK          # zero-sized: nothing to do
    assert call(a, b, A, Bc, -1, 4, 4, F32) == MI_ERR_INVALID_ARG
    assert call(None, b, A, Bc, 1, 4, 4, F32) == MI_ERR_INVALID_ARG
    assert call(a, b, a + 8, Bc, 1, 4, 4, F32) == MI_ERR_INVALID_ARG  # output overlaps input
    assert call(a, b, A, Bc, 1, 4, 4, 7) == MI_ERR_UNSUPPORTED
    # 2^31 channel-steps need far more than the scratch holds (buffers 1 TiB apart)
    a, b, A, Bc = [P + i * (1 << 40) for i in range(4)]
    assert call(a, b, A, Bc, 64, 8192, 4096, BF16) == MI_ERR_CAPACITY
    assert call(a, b, A, Bc, 64, 8192, 4096, F32) == MI_ERR_CAPACITY


def test_noalloc_capacity_constant_matches_header():
    text = open(HEADER).read()
    m = re.search(r"#define\s+MI_NOALLOC_SCRATCH_BYTES\s+\((\d+)u\s*<<\s*(\d+)\)", text)
    assert m, "MI_NOALLOC_SCRATCH_BYTES not found"
    assert lrs.NOALLOC_SCRATCH_BYTES == int(m.group(1)) << int(m.group(2))
    # the documented workload (B=8, T=8192, D=4096) fits: its forward workspace
    # at the widest vectors is at most the scratch
    for dt in (F32, BF16):
        assert lib().mi_linear_scan_workspace(8, 8192, 4096, dt) > 0
