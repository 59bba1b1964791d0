"""GPU parity: the HIP path (through the C ABI) against the fp64 oracle.

Inputs are seeded and synthetic with the workloads' distributions
(workloads.py); both sides see the same quantised values.  Error readings and
tolerances are described in tests/parity.py.  Every case prints what it runs
before touching the GPU.
"""
import sys

import numpy as np
import pytest
import torch

import linear_recurrence_scans_amd as lrs
import oracle
from parity import FLOOR, TOL, block_err, quantise, scaled_err, timeouts, to_np
from workloads import (affine_inputs_diag, affine_inputs_rotation, linear_inputs, log_inputs,
                       workload_inputs)

pytestmark = pytest.mark.gpu


def say(*args):
    print("[case]", *args, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module", autouse=True)
def _gpu_ready():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    ok, reason = lrs.mi_device_check(0)
    assert ok, reason


# ---------------------------------------------------------------------------
# k = 1 channel scan
# ---------------------------------------------------------------------------

def run_linear(x, dtype, with_bwd=True, check_ws=True):
    """GPU fwd (+ bwd) on quantised inputs; returns dict of errors vs the oracle."""
    a_d, a = quantise(x["a"], dtype)
    b_d, b = quantise(x["b"], dtype)
    Bn, T, D = a.shape
    ws = torch.empty(max(lrs.mi_linear_scan_workspace(Bn, T, D, dtype), 8), dtype=torch.uint8,
                     device="cuda")
    A_d, Bc_d = lrs.mi_linear_scan_fwd(a_d, b_d, ws=ws)
    torch.cuda.synchronize()
    if check_ws and ws.numel() >= 8:
        assert timeouts(ws) == 0
    A_r, Bc_r = oracle.linear_scan_fwd(a, b)
    _, Bc_s = oracle.linear_scan_fwd(np.abs(a), np.abs(b))
    errs = {"A": scaled_err(to_np(A_d), A_r, A_r, FLOOR[dtype]), "Bc": scaled_err(to_np(Bc_d), Bc_r, Bc_s, FLOOR[dtype])}
    if with_bwd:
        # backward inputs: the oracle's forward states, quantised like any input
        A_in_d, A_in = quantise(A_r, dtype)
        Bc_in_d, Bc_in = quantise(Bc_r, dtype)
        gA_d, gA = quantise(x["gA"], dtype)
        gB_d, gB = quantise(x["gBc"], dtype)
        da_d, db_d = lrs.mi_linear_scan_bwd(a_d, A_in_d, Bc_in_d, gA_d, gB_d, ws=ws)
        torch.cuda.synchronize()
        if check_ws and ws.numel() >= 8:
            assert timeouts(ws) == 0
        da_r, db_r = oracle.linear_scan_bwd(a, A_in, Bc_in, gA, gB)
        da_s, db_s = oracle.linear_scan_bwd(np.abs(a), np.abs(A_in), np.abs(Bc_in), np.abs(gA),
                                            np.abs(gB))
        errs["da"] = scaled_err(to_np(da_d), da_r, da_s, FLOOR[dtype])
        errs["db"] = scaled_err(to_np(db_d), db_r, db_s, FLOOR[dtype])
    return errs


def lin_case(Bn, T, D, seed, a_lo=0.5, a_hi=0.999):
    return linear_inputs(Bn, T, D, seed, a_lo, a_hi, grads=True)


@pytest.mark.parametrize("seed", [1, 11])
def test_linear_fwd_workload1(seed):
    """Workload 1 at its own size: B=1, T=1024, D=64, fp32."""
    say("linear fwd+bwd fp32 B=1 T=1024 D=64 seed", seed)
    errs = run_linear(lin_case(1, 1024, 64, seed), torch.float32)
    assert max(errs.values()) <= TOL[torch.float32], errs


@pytest.mark.parametrize("shape", [(1, 1, 1), (2, 2, 3), (1, 63, 100), (3, 65, 1), (2, 1000, 3),
                                   (1, 4097, 100), (2, 130, 520), (1, 64, 256), (2, 129, 257),
                                   (1, 31, 260), (2, 32, 256), (1, 33, 516)])
def test_linear_edge_shapes_f32(shape):
    say("linear fwd+bwd fp32 edge shape", shape)
    errs = run_linear(lin_case(*shape, seed=sum(shape)), torch.float32)
    assert max(errs.values()) <= TOL[torch.float32], (shape, errs)


@pytest.mark.parametrize("shape", [(2, 1000, 4104), (1, 77, 37), (3, 33, 6), (1, 300, 12), (2, 32, 512),
                                   (1, 97, 1024)])
def test_linear_bf16_reduced(shape):
    """bf16 storage / fp32 arithmetic on the workload-3 distribution; D values
    pick the 8-, 4-, 2- and 1-wide vector kernels and ragged tiles."""
    say("linear fwd+bwd bf16 shape", shape)
    errs = run_linear(lin_case(*shape, seed=13, a_lo=0.9, a_hi=0.9999), torch.bfloat16)
    assert max(errs.values()) <= TOL[torch.bfloat16], (shape, errs)


def test_linear_misaligned_views():
    """A view starting one element into its storage takes the 1-wide kernel."""
    say("linear fwd fp32 misaligned view B=2 T=300 D=64")
    x = lin_case(2, 300, 64, seed=21)
    a_full = torch.from_numpy(np.concatenate([[0.0], x["a"].ravel()])).float().cuda()
    b_full = torch.from_numpy(np.concatenate([[0.0], x["b"].ravel()])).float().cuda()
    a_d = a_full[1:].view(2, 300, 64)
    b_d = b_full[1:].view(2, 300, 64)
    assert a_d.data_ptr() % 16 != 0
    A_d, Bc_d = lrs.linear_scan_fwd(a_d, b_d)
    a = a_d.double().cpu().numpy()
    b = b_d.double().cpu().numpy()
    A_r, Bc_r = oracle.linear_scan_fwd(a, b)
    _, Bc_s = oracle.linear_scan_fwd(np.abs(a), np.abs(b))
    assert scaled_err(to_np(A_d), A_r, A_r) <= 1e-5
    assert scaled_err(to_np(Bc_d), Bc_r, Bc_s) <= 1e-5


def test_linear_lookback_long_sequence():
    """Many more workgroups than fit on the GPU along one tile's time axis:
    B=1, T=2^20, D=64 -- forward progress of the look-back and correctness."""
    say("linear fwd+bwd fp32 B=1 T=1048576 D=64 (look-back stress)")
    errs = run_linear(lin_case(1, 1 << 20, 64, seed=8, a_lo=0.9, a_hi=0.9999), torch.float32)
    assert max(errs.values()) <= TOL[torch.float32], errs


def test_linear_repeated_runs():
    """Race check over ten runs: the carry's association is fixed by the chunk's
    position alone (grouped look-back), so every run must match the oracle and
    the first run bit for bit."""
    say("linear fwd+bwd bf16 ten repeated runs B=2 T=4096 D=1024")
    dt = torch.bfloat16
    x = lin_case(2, 4096, 1024, seed=5, a_lo=0.9, a_hi=0.9999)
    a_d, a = quantise(x["a"], dt)
    b_d, b = quantise(x["b"], dt)
    gA_d, gA = quantise(x["gA"], dt)
    gB_d, gB = quantise(x["gBc"], dt)
    A_r, Bc_r = oracle.linear_scan_fwd(a, b)
    _, Bc_s = oracle.linear_scan_fwd(np.abs(a), np.abs(b))
    A_in_d, A_in = quantise(A_r, dt)
    Bc_in_d, Bc_in = quantise(Bc_r, dt)
    da_r, db_r = oracle.linear_scan_bwd(a, A_in, Bc_in, gA, gB)
    da_s, db_s = oracle.linear_scan_bwd(np.abs(a), np.abs(A_in), np.abs(Bc_in), np.abs(gA), np.abs(gB))
    first = None
    for run in range(10):
        A_d, Bc_d = lrs.linear_scan_fwd(a_d, b_d)
        da_d, db_d = lrs.linear_scan_bwd(a_d, A_in_d, Bc_in_d, gA_d, gB_d)
        outs = [to_np(t) for t in (A_d, Bc_d, da_d, db_d)]
        errs = [scaled_err(outs[0], A_r, A_r), scaled_err(outs[1], Bc_r, Bc_s),
                scaled_err(outs[2], da_r, da_s), scaled_err(outs[3], db_r, db_s)]
        assert max(errs) <= TOL[dt], (run, errs)
        if first is None:
            first = outs
        else:
            for f, o in zip(first, outs):
                assert np.array_equal(f, o), run


def test_linear_many_tiles():
    """Many channel tiles per chunk row (512 tiles of 256 fp32 channels): the
    look-back groups shrink to two chunks, so most chunks wait on an anchor."""
    say("linear fwd+bwd fp32 B=2 T=300 D=65536 (two-chunk look-back groups)")
    errs = run_linear(lin_case(2, 300, 65536, seed=17, a_lo=0.9, a_hi=0.9999), torch.float32)
    assert max(errs.values()) <= TOL[torch.float32], errs


def test_linear_side_stream():
    """A call on a stream other than the current one: the binding orders it
    after the current stream's work and keeps its own allocations on it; the
    results match the oracle and the current-stream call bit for bit."""
    say("linear fwd+bwd fp32 on a side stream B=2 T=2000 D=512")
    x = lin_case(2, 2000, 512, seed=33)
    a_d, a = quantise(x["a"], torch.float32)
    b_d, b = quantise(x["b"], torch.float32)
    A_ref, Bc_ref = lrs.linear_scan_fwd(a_d, b_d)
    side = torch.cuda.Stream()
    # produce the inputs on the current stream right before the side-stream call
    a2 = a_d * 1.0
    b2 = b_d * 1.0
    A_s, Bc_s = lrs.mi_linear_scan_fwd(a2, b2, stream=side)
    da_s, db_s = lrs.mi_linear_scan_bwd(a2, A_s, Bc_s, b2, a2, stream=side)
    torch.cuda.current_stream().wait_stream(side)
    da_r, db_r = lrs.mi_linear_scan_bwd(a_d, A_ref, Bc_ref, b_d, a_d)
    torch.cuda.synchronize()
    assert torch.equal(A_s, A_ref) and torch.equal(Bc_s, Bc_ref)
    assert torch.equal(da_s, da_r) and torch.equal(db_s, db_r)
    A_o, Bc_o = oracle.linear_scan_fwd(a, b)
    _, Bc_sc = oracle.linear_scan_fwd(np.abs(a), np.abs(b))
    assert scaled_err(to_np(A_s), A_o, A_o) <= TOL[torch.float32]
    assert scaled_err(to_np(Bc_s), Bc_o, Bc_sc) <= TOL[torch.float32]


def test_linear_workload3_full():
    """Workload 3 at its full size (B=8, T=8192, D=4096, bf16), the launch
    configuration the benchmark times; every output element is compared."""
    say("linear fwd+bwd bf16 B=8 T=8192 D=4096 seed 3 (full size)")
    errs = run_linear(workload_inputs(3), torch.bfloat16)
    print("errors", errs, flush=True)
    assert max(errs.values()) <= TOL[torch.bfloat16], errs


# ---------------------------------------------------------------------------
# k = 1 scan from a given initial state
# ---------------------------------------------------------------------------

def run_linear_h0(x, dtype, seed, with_h0=True):
    """GPU fwd + bwd from an initial state h0 against the oracle."""
    a_d, a = quantise(x["a"], dtype)
    b_d, b = quantise(x["b"], dtype)
    Bn, T, D = a.shape
    rg = np.random.Generator(np.random.PCG64(2000 + seed))
    if with_h0:
        h0_d, h0 = quantise(rg.standard_normal((Bn, D)), dtype)
    else:
        h0_d, h0 = None, None
    A_d, H_d = lrs.mi_linear_scan_fwd_h0(a_d, b_d, h0_d)
    torch.cuda.synchronize()
    A_r, H_r = oracle.linear_scan_fwd_h0(a, b, h0)
    _, H_s = oracle.linear_scan_fwd_h0(np.abs(a), np.abs(b), None if h0 is None else np.abs(h0))
    errs = {"A": scaled_err(to_np(A_d), A_r, A_r), "H": scaled_err(to_np(H_d), H_r, H_s)}
    A_in_d, A_in = quantise(A_r, dtype)
    H_in_d, H_in = quantise(H_r, dtype)
    gA_d, gA = quantise(x["gA"], dtype)
    gH_d, gH = quantise(x["gBc"], dtype)
    da_d, db_d, dh0_d = lrs.mi_linear_scan_bwd_h0(a_d, A_in_d, H_in_d, h0_d, gA_d, gH_d)
    torch.cuda.synchronize()
    da_r, db_r, dh0_r = oracle.linear_scan_bwd_h0(a, A_in, H_in, h0, gA, gH)
    ab = [np.abs(t) for t in (a, A_in, H_in)]
    da_s, db_s, dh0_s = oracle.linear_scan_bwd_h0(*ab, None if h0 is None else np.abs(h0), np.abs(gA), np.abs(gH))
    errs.update(da=scaled_err(to_np(da_d), da_r, da_s), db=scaled_err(to_np(db_d), db_r, db_s),
                dh0=scaled_err(to_np(dh0_d), dh0_r, dh0_s))
    return errs


@pytest.mark.parametrize("shape", [(1, 1, 1), (2, 63, 3), (1, 300, 100), (2, 1000, 520), (1, 4097, 64)])
def test_linear_h0_edge_shapes_f32(shape):
    say("linear fwd+bwd from h0, fp32, shape", shape)
    errs = run_linear_h0(lin_case(*shape, seed=sum(shape)), torch.float32, sum(shape))
    assert max(errs.values()) <= TOL[torch.float32], (shape, errs)


@pytest.mark.parametrize("shape", [(2, 1000, 4104), (1, 77, 37)])
def test_linear_h0_bf16(shape):
    say("linear fwd+bwd from h0, bf16, shape", shape)
    errs = run_linear_h0(lin_case(*shape, seed=19, a_lo=0.9, a_hi=0.9999), torch.bfloat16, 19)
    assert max(errs.values()) <= TOL[torch.bfloat16], (shape, errs)


def test_linear_h0_none_is_zero_state():
    say("linear fwd+bwd from h0 = None, fp32 B=2 T=300 D=64")
    errs = run_linear_h0(lin_case(2, 300, 64, seed=23), torch.float32, 23, with_h0=False)
    assert max(errs.values()) <= TOL[torch.float32], errs


def test_linear_h0_resume_matches_one_pass():
    """Two calls, the second started from the first's last state, give the states
    of one call over the whole sequence."""
    say("linear fwd resume fp32 B=2 T=3000 D=256 split at 1234")
    x = lin_case(2, 3000, 256, seed=24)
    a_d, a = quantise(x["a"], torch.float32)
    b_d, b = quantise(x["b"], torch.float32)
    _, H_full = lrs.mi_linear_scan_fwd_h0(a_d, b_d, None)
    _, H1 = lrs.mi_linear_scan_fwd_h0(a_d[:, :1234].contiguous(), b_d[:, :1234].contiguous(), None)
    _, H2 = lrs.mi_linear_scan_fwd_h0(a_d[:, 1234:].contiguous(), b_d[:, 1234:].contiguous(),
                                      H1[:, -1].contiguous())
    torch.cuda.synchronize()
    _, H_r = oracle.linear_scan_fwd(a, b)
    _, H_s = oracle.linear_scan_fwd(np.abs(a), np.abs(b))
    e = scaled_err(np.concatenate([to_np(H1), to_np(H2)], axis=1), H_r, H_s)
    assert e <= TOL[torch.float32], e
    assert scaled_err(to_np(H_full), H_r, H_s) <= TOL[torch.float32]


def test_linear_h0_no_steps():
    say("linear bwd from h0, T=0 B=2 D=8")
    z = torch.empty(2, 0, 8, device="cuda")
    h0 = torch.ones(2, 8, device="cuda")
    dh0 = torch.full((2, 8), float("nan"), device="cuda")
    _, _, dh0 = lrs.mi_linear_scan_bwd_h0(z, z, z, h0, z, z, dh0=dh0)
    torch.cuda.synchronize()
    assert bool(torch.all(dh0 == 0))


# ---------------------------------------------------------------------------
# log-space scan
# ---------------------------------------------------------------------------

def run_log(x, dtype):
    lc_d, lc = quantise(x["log_coeffs"], dtype)
    lv_d, lv = quantise(x["log_values"], dtype)
    Bn, T, D = lc.shape
    ws = torch.empty(max(lrs.mi_scan_log_workspace(Bn, T, D, dtype), 8), dtype=torch.uint8,
                     device="cuda")
    h_d = lrs.mi_scan_log_fwd(lc_d, lv_d, ws=ws)
    torch.cuda.synchronize()
    assert timeouts(ws) == 0
    h_r = oracle.scan_log_fwd_logspace(lc, lv)
    return scaled_err(to_np(h_d), h_r, h_r, FLOOR[dtype])


@pytest.mark.parametrize("seed", [2, 12])
def test_log_workload2_full(seed):
    say("log fwd fp32 B=4 T=4096 D=512 seed", seed)
    e = run_log(workload_inputs(2, seed=seed), torch.float32)
    print("error", e, flush=True)
    assert e <= TOL[torch.float32], e


@pytest.mark.parametrize("shape", [(1, 1, 1), (2, 63, 3), (1, 65, 100), (2, 1000, 5), (1, 4097, 64),
                                   (3, 200, 260)])
def test_log_edge_shapes(shape):
    say("log fwd fp32 edge shape", shape)
    e = run_log(log_inputs(*shape, seed=sum(shape)), torch.float32)
    assert e <= TOL[torch.float32], (shape, e)


def test_log_bf16():
    say("log fwd bf16 B=2 T=500 D=136")
    e = run_log(log_inputs(2, 500, 136, seed=7), torch.bfloat16)
    assert e <= TOL[torch.bfloat16], e


def test_log_extreme_range():
    """Magnitudes whose linear form would underflow fp32: a = e^-120 on some
    steps, b = e^-90; the log-space result is still exact to fp32."""
    say("log fwd fp32 extreme range B=1 T=256 D=64")
    r = np.random.Generator(np.random.PCG64(99))
    lc = np.where(r.random((1, 256, 64)) < 0.1, -120.0, -0.01)
    lv = np.full((1, 257, 64), -90.0) + r.normal(0, 1, (1, 257, 64))
    e = run_log({"log_coeffs": lc, "log_values": lv}, torch.float32)
    assert e <= TOL[torch.float32], e


def run_log_bwd(x, dtype, seed=0):
    """GPU backward of the log scan against the oracle.  Both sides get the
    same quantised log_coeffs, log_values, forward output h (the oracle's, cast
    like any input) and upstream gradient g."""
    lc_d, lc = quantise(x["log_coeffs"], dtype)
    lv_d, lv = quantise(x["log_values"], dtype)
    Bn, T, D = lc.shape
    h_d, h = quantise(oracle.scan_log_fwd(lc, lv), dtype)
    g_d, g = quantise(np.random.Generator(np.random.PCG64(1000 + seed)).standard_normal(lc.shape), dtype)
    ws = torch.empty(max(lrs.mi_scan_log_workspace(Bn, T, D, dtype), 8), dtype=torch.uint8, device="cuda")
    dlc_d, dlv_d = lrs.mi_scan_log_bwd(lc_d, lv_d, h_d, g_d, ws=ws)
    torch.cuda.synchronize()
    assert timeouts(ws) == 0
    dlc_r, dlv_r = oracle.scan_log_bwd(lc, lv, h, g)
    dlc_s, dlv_s = oracle.scan_log_bwd(lc, lv, h, np.abs(g))  # every other factor is positive
    return {"dlc": scaled_err(to_np(dlc_d), dlc_r, dlc_s, FLOOR[dtype]), "dlv": scaled_err(to_np(dlv_d), dlv_r, dlv_s, FLOOR[dtype])}


@pytest.mark.parametrize("seed", [2, 12])
def test_log_bwd_workload2_full(seed):
    """Backward of the log scan at the workload-2 size (B=4, T=4096, D=512, fp32)."""
    say("log bwd fp32 B=4 T=4096 D=512 seed", seed)
    errs = run_log_bwd(workload_inputs(2, seed=seed), torch.float32, seed)
    print("errors", errs, flush=True)
    assert max(errs.values()) <= TOL[torch.float32], errs


@pytest.mark.parametrize("shape", [(1, 1, 1), (2, 63, 3), (1, 65, 100), (2, 1000, 5), (1, 4097, 64),
                                   (3, 200, 260)])
def test_log_bwd_edge_shapes(shape):
    say("log bwd fp32 edge shape", shape)
    errs = run_log_bwd(log_inputs(*shape, seed=sum(shape)), torch.float32, sum(shape))
    assert max(errs.values()) <= TOL[torch.float32], (shape, errs)


@pytest.mark.parametrize("shape", [(2, 500, 136), (1, 77, 37), (3, 129, 6)])
def test_log_bwd_bf16(shape):
    """bf16 storage, fp32 arithmetic; D values pick 8-, 1- and 2-wide vectors."""
    say("log bwd bf16 shape", shape)
    errs = run_log_bwd(log_inputs(*shape, seed=7), torch.bfloat16, 7)
    assert max(errs.values()) <= TOL[torch.bfloat16], (shape, errs)


def test_log_bwd_no_steps():
    """T = 0: the only output is d log h_0, which is zero."""
    say("log bwd fp32 T=0 B=2 D=8")
    lc = torch.empty(2, 0, 8, device="cuda")
    lv = torch.zeros(2, 1, 8, device="cuda")
    h = torch.empty(2, 0, 8, device="cuda")
    dlv = torch.full((2, 1, 8), float("nan"), device="cuda")
    dlc, dlv = lrs.mi_scan_log_bwd(lc, lv, h, h, dlog_values=dlv)
    torch.cuda.synchronize()
    assert dlc.numel() == 0 and bool(torch.all(dlv == 0))


def test_log_repeated_runs():
    """Ten runs of the log-space forward and backward are bitwise identical
    (fixed carry association) and match the oracle."""
    say("log fwd+bwd fp32 ten repeated runs B=2 T=3000 D=256")
    x = log_inputs(2, 3000, 256, seed=21)
    lc_d, lc = quantise(x["log_coeffs"], torch.float32)
    lv_d, lv = quantise(x["log_values"], torch.float32)
    h_r = oracle.scan_log_fwd_logspace(lc, lv)
    hq_d, hq = quantise(oracle.scan_log_fwd(lc, lv), torch.float32)
    g_d, g = quantise(np.random.Generator(np.random.PCG64(1021)).standard_normal(lc.shape), torch.float32)
    dlc_r, dlv_r = oracle.scan_log_bwd(lc, lv, hq, g)
    dlc_s, dlv_s = oracle.scan_log_bwd(lc, lv, hq, np.abs(g))
    first = None
    for run in range(10):
        h_d = lrs.mi_scan_log_fwd(lc_d, lv_d)
        dlc_d, dlv_d = lrs.mi_scan_log_bwd(lc_d, lv_d, hq_d, g_d)
        outs = [to_np(t) for t in (h_d, dlc_d, dlv_d)]
        errs = [scaled_err(outs[0], h_r, h_r), scaled_err(outs[1], dlc_r, dlc_s), scaled_err(outs[2], dlv_r, dlv_s)]
        assert max(errs) <= TOL[torch.float32], (run, errs)
        if first is None:
            first = outs
        else:
            for f, o in zip(first, outs):
                assert np.array_equal(f, o), run


def test_log_lookback_long_sequence():
    """One channel tile along T = 2^20 (8192 chunks in a chain of look-back
    groups): forward progress of the log carry, forward and backward."""
    say("log fwd+bwd fp32 B=1 T=1048576 D=64 (look-back stress)")
    x = log_inputs(1, 1 << 20, 64, seed=41)
    e = run_log(x, torch.float32)
    assert e <= TOL[torch.float32], e
    errs = run_log_bwd(x, torch.float32, 41)
    assert max(errs.values()) <= TOL[torch.float32], errs


# ---------------------------------------------------------------------------
# k x k scan
# ---------------------------------------------------------------------------

def run_affine(x, with_bwd, metric, dtype=torch.float32):
    """metric "block": per (b, t, head) block relative to the block's largest
    entry -- for rotation inputs, whose elementwise-absolute products grow
    geometrically.  metric "abs": the condition-normalised reading of the k = 1
    scan (oracle on absolute values as the scale) -- for diagonally dominant
    inputs, whose absolute products stay bounded."""
    A_d, A = quantise(x["A"], dtype)
    B_d, Bm = quantise(x["Bm"], dtype)
    Bn, T, n, k, _ = A.shape
    v = Bm.shape[4]
    ws = torch.empty(max(lrs.mi_affine_scan_workspace(Bn, T, n, k, v, dtype), 8), dtype=torch.uint8,
                     device="cuda")
    Abar_d, Bbar_d = lrs.mi_affine_scan_fwd(A_d, B_d, ws=ws)
    torch.cuda.synchronize()
    assert timeouts(ws) == 0
    Abar_r, Bbar_r = oracle.affine_scan_fwd(A, Bm)
    if metric == "block":
        errs = {"Abar": block_err(to_np(Abar_d), Abar_r), "Bbar": block_err(to_np(Bbar_d), Bbar_r)}
        # reported, not asserted: element-wise relative error over entries at least a
        # tenth of their block's largest (the tolerance is read per block)
        for name, G, R in (("Abar", to_np(Abar_d), Abar_r), ("Bbar", to_np(Bbar_d), Bbar_r)):
            big = np.abs(R) >= 0.1 * np.max(np.abs(R), axis=(-2, -1), keepdims=True)
            rel = np.abs(G - R)[big] / np.abs(R)[big]
            print("element-wise relative error of %s over entries >= 0.1 x block max: %.3g"
                  % (name, float(rel.max()) if rel.size else 0.0), flush=True)
    else:
        Abar_s, Bbar_s = oracle.affine_scan_fwd(np.abs(A), np.abs(Bm))
        assert np.all(np.isfinite(Abar_s)) and np.all(np.isfinite(Bbar_s))
        errs = {"Abar": scaled_err(to_np(Abar_d), Abar_r, Abar_s, FLOOR[dtype]),
                "Bbar": scaled_err(to_np(Bbar_d), Bbar_r, Bbar_s, FLOOR[dtype])}
    if with_bwd:
        assert metric == "abs"
        Ab_in_d, Ab_in = quantise(Abar_r, dtype)
        Bb_in_d, Bb_in = quantise(Bbar_r, dtype)
        gA_d, gA = quantise(x["gAbar"], dtype)
        gB_d, gB = quantise(x["gBbar"], dtype)
        dA_d, dB_d = lrs.mi_affine_scan_bwd(A_d, Ab_in_d, Bb_in_d, gA_d, gB_d, ws=ws)
        torch.cuda.synchronize()
        assert timeouts(ws) == 0
        dA_r, dB_r = oracle.affine_scan_bwd(A, Ab_in, Bb_in, gA, gB)
        dA_s, dB_s = oracle.affine_scan_bwd(np.abs(A), np.abs(Ab_in), np.abs(Bb_in), np.abs(gA),
                                            np.abs(gB))
        assert np.all(np.isfinite(dA_s)) and np.all(np.isfinite(dB_s))
        errs["dA"] = scaled_err(to_np(dA_d), dA_r, dA_s, FLOOR[dtype])
        errs["dB"] = scaled_err(to_np(dB_d), dB_r, dB_s, FLOOR[dtype])
    return errs


@pytest.mark.parametrize("seed", [4, 14])
def test_affine_workload4_full(seed):
    say("affine fwd fp32 B=2 T=2048 n=64 k=4 v=16 seed", seed)
    errs = run_affine(workload_inputs(4, seed=seed), with_bwd=False, metric="block")
    print("errors", errs, flush=True)
    assert max(errs.values()) <= TOL[torch.float32], errs


@pytest.mark.parametrize("seed", [5, 15])
def test_affine_workload5_full(seed):
    say("affine fwd+bwd fp32 B=4 T=4096 n=32 k=8 v=32 seed", seed)
    errs = run_affine(workload_inputs(5, seed=seed), with_bwd=True, metric="abs")
    print("errors", errs, flush=True)
    assert max(errs.values()) <= TOL[torch.float32], errs


# (4, 6), (8, 6) and (16, 6) leave 2k + v = 2 (mod 4): the backward's dA rows
# then read two zeroed pad columns; at k = 16 a lane forms up to four groups.
@pytest.mark.parametrize("kv", [(1, 1), (2, 2), (3, 5), (4, 16), (8, 32), (16, 1), (2, 128),
                                (16, 128), (5, 3), (4, 6), (8, 6), (16, 6)])
def test_affine_edge_shapes(kv):
    k, v = kv
    for (Bn, T, n) in ((1, 1, 1), (2, 33, 3), (1, 130, 5)):
        say("affine fwd+bwd fp32 edge B,T,n,k,v =", (Bn, T, n, k, v))
        x = affine_inputs_diag(Bn, T, n, k, v, seed=k * 100 + v + T, grads=True)
        errs = run_affine(x, with_bwd=True, metric="abs")
        assert max(errs.values()) <= TOL[torch.float32], ((Bn, T, n, k, v), errs)


def run_affine_h0(x, seed, with_h0=True):
    """GPU k x k fwd + bwd from an initial state H0 (condition-normalised error,
    diagonally dominant inputs)."""
    A_d, A = quantise(x["A"], torch.float32)
    B_d, Bm = quantise(x["Bm"], torch.float32)
    Bn, T, n, k, _ = A.shape
    v = Bm.shape[4]
    rg = np.random.Generator(np.random.PCG64(3000 + seed))
    H0_d, H0 = quantise(rg.standard_normal((Bn, n, k, v)), torch.float32) if with_h0 else (None, None)
    Ab_d, H_d = lrs.mi_affine_scan_fwd_h0(A_d, B_d, H0_d)
    torch.cuda.synchronize()
    Ab_r, H_r = oracle.affine_scan_fwd_h0(A, Bm, H0)
    Ab_s, H_s = oracle.affine_scan_fwd_h0(np.abs(A), np.abs(Bm), None if H0 is None else np.abs(H0))
    errs = {"Abar": scaled_err(to_np(Ab_d), Ab_r, Ab_s), "H": scaled_err(to_np(H_d), H_r, H_s)}
    Ab_in_d, Ab_in = quantise(Ab_r, torch.float32)
    H_in_d, H_in = quantise(H_r, torch.float32)
    gA_d, gA = quantise(x["gAbar"], torch.float32)
    gH_d, gH = quantise(x["gBbar"], torch.float32)
    dA_d, dB_d, dH0_d = lrs.mi_affine_scan_bwd_h0(A_d, Ab_in_d, H_in_d, H0_d, gA_d, gH_d)
    torch.cuda.synchronize()
    dA_r, dB_r, dH0_r = oracle.affine_scan_bwd_h0(A, Ab_in, H_in, H0, gA, gH)
    dA_s, dB_s, dH0_s = oracle.affine_scan_bwd_h0(np.abs(A), np.abs(Ab_in), np.abs(H_in),
                                                  None if H0 is None else np.abs(H0), np.abs(gA), np.abs(gH))
    errs.update(dA=scaled_err(to_np(dA_d), dA_r, dA_s), dB=scaled_err(to_np(dB_d), dB_r, dB_s),
                dH0=scaled_err(to_np(dH0_d), dH0_r, dH0_s))
    return errs


@pytest.mark.parametrize("kv", [(4, 16), (8, 32), (3, 5), (1, 1), (16, 4)])
def test_affine_h0(kv):
    k, v = kv
    for (Bn, T, n) in ((1, 1, 1), (2, 130, 5)):
        say("affine fwd+bwd from H0 fp32 B,T,n,k,v =", (Bn, T, n, k, v))
        x = affine_inputs_diag(Bn, T, n, k, v, seed=k * 10 + v + T, grads=True)
        errs = run_affine_h0(x, k + v + T)
        assert max(errs.values()) <= TOL[torch.float32], ((Bn, T, n, k, v), errs)


def test_affine_h0_none_and_workload5_size():
    say("affine fwd+bwd from H0 = None at workload-5 size, and with H0")
    x = workload_inputs(5)
    errs = run_affine_h0(x, 5, with_h0=False)
    assert max(errs.values()) <= TOL[torch.float32], errs
    errs = run_affine_h0(x, 5, with_h0=True)
    print("errors", errs, flush=True)
    assert max(errs.values()) <= TOL[torch.float32], errs


@pytest.mark.parametrize("kv", [(4, 16), (8, 32), (3, 5), (2, 2), (16, 8)])
def test_affine_bf16(kv):
    """bf16 storage, fp32 arithmetic (k x k, forward and backward)."""
    k, v = kv
    for (Bn, T, n) in ((1, 1, 1), (2, 300, 5)):
        say("affine fwd+bwd bf16 B,T,n,k,v =", (Bn, T, n, k, v))
        x = affine_inputs_diag(Bn, T, n, k, v, seed=k * 7 + v + T, grads=True)
        errs = run_affine(x, with_bwd=True, metric="abs", dtype=torch.bfloat16)
        assert max(errs.values()) <= TOL[torch.bfloat16], ((Bn, T, n, k, v), errs)


def test_affine_bf16_workload_shapes():
    """bf16 storage at the workload-5 size (fwd + bwd) and the workload-4 size
    (fwd; rotations, block metric)."""
    say("affine fwd+bwd bf16 at workload-5 size")
    errs = run_affine(workload_inputs(5), with_bwd=True, metric="abs", dtype=torch.bfloat16)
    print("errors", errs, flush=True)
    assert max(errs.values()) <= TOL[torch.bfloat16], errs
    say("affine fwd bf16 at workload-4 size")
    errs = run_affine(workload_inputs(4), with_bwd=False, metric="block", dtype=torch.bfloat16)
    print("errors", errs, flush=True)
    assert max(errs.values()) <= TOL[torch.bfloat16], errs


# Forward chunks hold SEG time segments of NW * L steps: (k, v) = (4, 16)
# gives 2 segments of 32 steps (64-step chunks, 3 heads a workgroup), (8, 32)
# one segment of 32 steps (32-step chunks, 3 heads).  T just below, at and
# past a chunk or segment boundary, and head counts that leave slots idle,
# exercise the segment map.
@pytest.mark.parametrize("case", [(4, 16, 31), (4, 16, 32), (4, 16, 33), (4, 16, 63), (4, 16, 64),
                                  (4, 16, 65), (4, 16, 129), (4, 16, 17), (8, 32, 31), (8, 32, 32),
                                  (8, 32, 33), (8, 32, 65), (8, 32, 16), (8, 32, 97)])
def test_affine_chunk_boundaries(case):
    k, v, T = case
    for (Bn, n) in ((1, 1), (2, 3)):
        say("affine fwd+bwd B,T,n,k,v =", (Bn, T, n, k, v))
        x = affine_inputs_diag(Bn, T, n, k, v, seed=T + k, grads=True)
        errs = run_affine(x, with_bwd=True, metric="abs")
        assert max(errs.values()) <= TOL[torch.float32], ((Bn, T, n, k, v), errs)


def test_affine_rotation_long():
    """Rotations (non-commuting products) over a long sequence."""
    say("affine fwd fp32 rotation B=1 T=5000 n=3 k=4 v=3")
    x = affine_inputs_rotation(1, 5000, 3, 4, 3, seed=31, rho=0.999)
    errs = run_affine(x, with_bwd=False, metric="block")
    assert max(errs.values()) <= TOL[torch.float32], errs


@pytest.mark.parametrize("kv", [(4, 16), (8, 32)])
def test_affine_lookback_long_sequence(kv):
    """One head along T = 2^18: thousands of chunks in a chain of look-back
    groups of 64, staged in several LDS batches per fold; forward and
    backward must finish, match the oracle and leave the timeout counter at 0."""
    k, v = kv
    say("affine fwd+bwd fp32 B=1 T=262144 n=1 k=%d v=%d (look-back stress)" % (k, v))
    x = affine_inputs_diag(1, 1 << 18, 1, k, v, seed=43 + k, grads=True)
    errs = run_affine(x, with_bwd=True, metric="abs")
    assert max(errs.values()) <= TOL[torch.float32], errs


def test_affine_repeated_runs():
    """Race check over ten runs: bitwise identical, each matching the oracle."""
    say("affine fwd+bwd ten repeated runs B=2 T=1024 n=16 k=8 v=32")
    x = affine_inputs_diag(2, 1024, 16, 8, 32, seed=3, grads=True)
    A_d, A = quantise(x["A"], torch.float32)
    B_d, Bm = quantise(x["Bm"], torch.float32)
    gA_d, gA = quantise(x["gAbar"], torch.float32)
    gB_d, gB = quantise(x["gBbar"], torch.float32)
    Abar_r, Bbar_r = oracle.affine_scan_fwd(A, Bm)
    Abar_s, Bbar_s = oracle.affine_scan_fwd(np.abs(A), np.abs(Bm))
    Ab_in_d, Ab_in = quantise(Abar_r, torch.float32)
    Bb_in_d, Bb_in = quantise(Bbar_r, torch.float32)
    dA_r, dB_r = oracle.affine_scan_bwd(A, Ab_in, Bb_in, gA, gB)
    dA_s, dB_s = oracle.affine_scan_bwd(np.abs(A), np.abs(Ab_in), np.abs(Bb_in), np.abs(gA), np.abs(gB))
    first = None
    for run in range(10):
        Abar_d, Bbar_d = lrs.affine_scan_fwd(A_d, B_d)
        dA_d, dB_d = lrs.affine_scan_bwd(A_d, Ab_in_d, Bb_in_d, gA_d, gB_d)
        outs = [to_np(t) for t in (Abar_d, Bbar_d, dA_d, dB_d)]
        errs = [scaled_err(outs[0], Abar_r, Abar_s), scaled_err(outs[1], Bbar_r, Bbar_s),
                scaled_err(outs[2], dA_r, dA_s), scaled_err(outs[3], dB_r, dB_s)]
        assert max(errs) <= TOL[torch.float32], (run, errs)
        if first is None:
            first = outs
        else:
            for f, o in zip(first, outs):
                assert np.array_equal(f, o), run


# ---------------------------------------------------------------------------
# fp16 storage (fp32 arithmetic) for every op
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("shape", [(2, 1000, 4104), (1, 77, 37), (3, 33, 6), (2, 300, 512)])
def test_linear_f16(shape):
    """fp16 storage on the workload-3 distribution; D values pick the 8-, 1-
    and 2-wide vector kernels and ragged tiles."""
    say("linear fwd+bwd fp16 shape", shape)
    errs = run_linear(lin_case(*shape, seed=29, a_lo=0.9, a_hi=0.9999), torch.float16)
    assert max(errs.values()) <= TOL[torch.float16], (shape, errs)


def test_linear_f16_workload3_size():
    """fp16 storage at the workload-3 size (B=8, T=8192, D=4096)."""
    say("linear fwd+bwd fp16 B=8 T=8192 D=4096 seed 3")
    errs = run_linear(workload_inputs(3), torch.float16)
    print("errors", errs, flush=True)
    assert max(errs.values()) <= TOL[torch.float16], errs


@pytest.mark.parametrize("shape", [(2, 500, 136), (1, 77, 37), (4, 4096, 512)])
def test_log_f16(shape):
    """Log-space forward and backward with fp16 storage (the last shape is the
    workload-2 size)."""
    say("log fwd+bwd fp16 shape", shape)
    x = log_inputs(*shape, seed=31)
    e = run_log(x, torch.float16)
    assert e <= TOL[torch.float16], (shape, e)
    errs = run_log_bwd(x, torch.float16, 31)
    assert max(errs.values()) <= TOL[torch.float16], (shape, errs)


@pytest.mark.parametrize("kv", [(4, 16), (8, 32), (3, 5), (2, 2), (16, 8)])
def test_affine_f16(kv):
    """k x k forward and backward with fp16 storage."""
    k, v = kv
    for (Bn, T, n) in ((1, 1, 1), (2, 300, 5)):
        say("affine fwd+bwd fp16 B,T,n,k,v =", (Bn, T, n, k, v))
        x = affine_inputs_diag(Bn, T, n, k, v, seed=k * 11 + v + T, grads=True)
        errs = run_affine(x, with_bwd=True, metric="abs", dtype=torch.float16)
        assert max(errs.values()) <= TOL[torch.float16], ((Bn, T, n, k, v), errs)


def test_affine_f16_workload5_size():
    say("affine fwd+bwd fp16 at workload-5 size")
    errs = run_affine(workload_inputs(5), with_bwd=True, metric="abs", dtype=torch.float16)
    print("errors", errs, flush=True)
    assert max(errs.values()) <= TOL[torch.float16], errs
