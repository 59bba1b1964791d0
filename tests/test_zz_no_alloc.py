"""The entry point that allocates nothing (mi_linear_scan_fwd_noalloc), called
through the C ABI: its output must equal the workspace entry point's
(mi_linear_scan_fwd) on the same inputs, on two calls in a row whose second is
smaller, and both must match the fp64 oracle within the stated tolerance."""
import sys

import numpy as np
import pytest
import torch

import linear_recurrence_scans_amd as lrs
import oracle
from parity import TOL, quantise, scaled_err, to_np
from workloads import linear_inputs

pytestmark = pytest.mark.gpu


def say(*args):
    print("[case]", *args, flush=True)
    sys.stdout.flush()


def noalloc_fwd(a_d, b_d):
    """Direct C-ABI call; outputs allocated here, no workspace passed."""
    A = torch.empty_like(a_d)
    Bc = torch.empty_like(a_d)
    Bn, T, D = a_d.shape
    dt = 1 if a_d.dtype == torch.bfloat16 else 0
    st = lrs._load().mi_linear_scan_fwd_noalloc(a_d.data_ptr(), b_d.data_ptr(), A.data_ptr(), Bc.data_ptr(),
                                                Bn, T, D, dt, torch.cuda.current_stream().cuda_stream)
    assert st == 0, lrs.mi_status_string(st)
    return A, Bc


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_noalloc_matches_workspace_entry_point(dtype):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    tol = TOL[dtype]
    # the second call is smaller, so it reuses the first call's scratch contents
    for (Bn, T, D, seed) in ((2, 3000, 1032, 61), (1, 300, 96, 62)):
        say("noalloc linear fwd", dtype, "B=%d T=%d D=%d" % (Bn, T, D))
        x = linear_inputs(Bn, T, D, seed, 0.9, 0.9999)
        a_d, a = quantise(x["a"], dtype)
        b_d, b = quantise(x["b"], dtype)
        A_n, Bc_n = noalloc_fwd(a_d, b_d)
        A_w, Bc_w = lrs.mi_linear_scan_fwd(a_d, b_d)
        torch.cuda.synchronize()
        A_r, Bc_r = oracle.linear_scan_fwd(a, b)
        _, Bc_s = oracle.linear_scan_fwd(np.abs(a), np.abs(b))
        assert scaled_err(to_np(A_n), to_np(A_w), to_np(A_w).__abs__()) <= tol
        assert scaled_err(to_np(Bc_n), to_np(Bc_w), Bc_s) <= tol
        # the kernels and the carry association are the same: bit for bit
        assert torch.equal(A_n, A_w) and torch.equal(Bc_n, Bc_w)
        assert scaled_err(to_np(A_n), A_r, A_r) <= tol
        assert scaled_err(to_np(Bc_n), Bc_r, Bc_s) <= tol


def test_noalloc_rejects_oversized_problem():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    say("noalloc linear fwd: capacity check")
    a = torch.empty(1, 1, 1, device="cuda")
    # sizes whose workspace exceeds the scratch; rejected before any access
    st = lrs._load().mi_linear_scan_fwd_noalloc(a.data_ptr(), a.data_ptr() + (1 << 40), a.data_ptr() + (2 << 40),
                                                a.data_ptr() + (3 << 40), 64, 8192, 4096, 1,
                                                torch.cuda.current_stream().cuda_stream)
    assert st == 6, lrs.mi_status_string(st)
