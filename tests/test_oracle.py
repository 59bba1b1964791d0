"""Pins of the fp64 CPU oracle against facts fixed outside the oracle itself.

None of these tests re-types an oracle formula.  Each checks the oracle against
something independent: a library routine (numpy.cumprod / cumsum, matrix
products, torch autograd), a closed form, brute force by a *different* formula,
exact rational arithmetic, finite differences, or a hand-worked example stored
under tests/golden/.  The definitions come from the minGRU docs page "Triton
kernels", section "Kernel entry points".
"""
import json
import os
from fractions import Fraction

import numpy as np
import pytest

import oracle
from workloads import rng

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


# --------------------------------------------------------------------------
# k = 1 forward
# --------------------------------------------------------------------------

def test_golden_linear():
    g = _golden("linear_k1_T4.json")
    A, Bc = oracle.linear_scan_fwd(g["a"], g["b"])
    np.testing.assert_array_equal(A, np.array(g["A"]))
    np.testing.assert_array_equal(Bc, np.array(g["Bc"]))
    da, db = oracle.linear_scan_bwd(g["a"], g["A"], g["Bc"], g["gA"], g["gBc"])
    np.testing.assert_array_equal(da, np.array(g["da"]))
    np.testing.assert_array_equal(db, np.array(g["db"]))


def test_running_product_is_cumprod():
    """A_t is the running product of a: numpy.cumprod along time."""
    r = rng(101)
    a = r.uniform(-1.5, 1.5, size=(3, 257, 5))
    b = r.standard_normal((3, 257, 5))
    A, _ = oracle.linear_scan_fwd(a, b)
    np.testing.assert_allclose(A, np.cumprod(a, axis=1), rtol=1e-15, atol=0)


@pytest.mark.parametrize("aval", [0.5, 0.9, 0.999])
def test_constant_coefficients_closed_form(aval):
    """Constant a and b: Bc_t = b (1 - a^t) / (1 - a)."""
    T, bval = 4096, 0.7
    a = np.full((1, T, 1), aval)
    b = np.full((1, T, 1), bval)
    A, Bc = oracle.linear_scan_fwd(a, b)
    t = np.arange(1, T + 1, dtype=np.float64)
    np.testing.assert_allclose(Bc[0, :, 0], bval * (1 - aval ** t) / (1 - aval), rtol=1e-12)
    np.testing.assert_allclose(A[0, :, 0], aval ** t, rtol=1e-12)


def test_special_cases():
    r = rng(102)
    b = r.standard_normal((2, 300, 3))
    # a == 1: Bc is the cumulative sum of b
    _, Bc = oracle.linear_scan_fwd(np.ones_like(b), b)
    np.testing.assert_allclose(Bc, np.cumsum(b, axis=1), rtol=1e-13, atol=1e-13)
    # a == 0: every step forgets the past, Bc = b
    A, Bc = oracle.linear_scan_fwd(np.zeros_like(b), b)
    np.testing.assert_array_equal(Bc, b)
    np.testing.assert_array_equal(A, np.zeros_like(b))
    # T == 1: (A, Bc) = (a, b) and (da, db) = (gA, gBc)
    a1 = r.standard_normal((2, 1, 4))
    b1 = r.standard_normal((2, 1, 4))
    A, Bc = oracle.linear_scan_fwd(a1, b1)
    np.testing.assert_array_equal(A, a1)
    np.testing.assert_array_equal(Bc, b1)
    gA, gBc = r.standard_normal((2, 1, 4)), r.standard_normal((2, 1, 4))
    da, db = oracle.linear_scan_bwd(a1, A, Bc, gA, gBc)
    np.testing.assert_array_equal(da, gA)
    np.testing.assert_array_equal(db, gBc)


def _brute_linear(a, b):
    """Bc_t = sum_{s<=t} (prod_{r=s+1..t} a_r) b_s, A_t = prod_{r<=t} a_r (T tiny)."""
    Bn, T, D = a.shape
    A = np.zeros_like(a)
    Bc = np.zeros_like(a)
    for bb in range(Bn):
        for d in range(D):
            for t in range(T):
                A[bb, t, d] = np.prod(a[bb, :t + 1, d])
                Bc[bb, t, d] = sum(np.prod(a[bb, s + 1:t + 1, d]) * b[bb, s, d]
                                   for s in range(t + 1))
    return A, Bc


def test_linear_brute_force_tiny():
    r = rng(103)
    for T in range(1, 9):
        a = r.uniform(-2, 2, size=(2, T, 3))
        b = r.standard_normal((2, T, 3))
        A, Bc = oracle.linear_scan_fwd(a, b)
        A2, Bc2 = _brute_linear(a, b)
        np.testing.assert_allclose(A, A2, rtol=1e-13, atol=1e-13)
        np.testing.assert_allclose(Bc, Bc2, rtol=1e-13, atol=1e-13)


def test_linear_exact_rationals():
    """Exact rational arithmetic on dyadic inputs: the fp64 oracle must be exact."""
    r = rng(104)
    T = 6
    num_a = r.integers(-8, 9, size=T)
    num_b = r.integers(-8, 9, size=T)
    a = [Fraction(int(x), 4) for x in num_a]
    b = [Fraction(int(x), 2) for x in num_b]
    h, P = Fraction(0), Fraction(1)
    exp_A, exp_Bc = [], []
    for t in range(T):
        P, h = a[t] * P, a[t] * h + b[t]
        exp_A.append(P)
        exp_Bc.append(h)
    A, Bc = oracle.linear_scan_fwd(np.array([float(x) for x in a]).reshape(1, T, 1),
                                   np.array([float(x) for x in b]).reshape(1, T, 1))
    assert [Fraction(x) for x in A[0, :, 0]] == exp_A
    assert [Fraction(x) for x in Bc[0, :, 0]] == exp_Bc


def test_split_time_carry():
    """Scanning [1,T] equals scanning [1,T1], then [T1+1,T] from zero, composed with
    the carry (A_T1, h_T1): A = A2*A_T1, Bc = A2*h_T1 + Bc2."""
    r = rng(105)
    a = r.uniform(0.5, 1.0, size=(2, 500, 4))
    b = r.standard_normal((2, 500, 4))
    A, Bc = oracle.linear_scan_fwd(a, b)
    T1 = 173
    A1, Bc1 = oracle.linear_scan_fwd(a[:, :T1], b[:, :T1])
    A2, Bc2 = oracle.linear_scan_fwd(a[:, T1:], b[:, T1:])
    np.testing.assert_allclose(A[:, T1:], A2 * A1[:, -1:], rtol=1e-13)
    np.testing.assert_allclose(Bc[:, T1:], A2 * Bc1[:, -1:] + Bc2, rtol=1e-12, atol=1e-13)


# --------------------------------------------------------------------------
# k = 1 backward
# --------------------------------------------------------------------------

def _loss_linear(a, b, gA, gBc):
    A, Bc = oracle.linear_scan_fwd(a, b)
    return float(np.sum(gA * A) + np.sum(gBc * Bc))


def test_linear_bwd_finite_differences():
    r = rng(106)
    eps = 1e-6
    for T in (1, 2, 5, 8):
        a = r.uniform(-1.2, 1.2, size=(1, T, 2))
        b = r.standard_normal((1, T, 2))
        gA, gBc = r.standard_normal((1, T, 2)), r.standard_normal((1, T, 2))
        A, Bc = oracle.linear_scan_fwd(a, b)
        da, db = oracle.linear_scan_bwd(a, A, Bc, gA, gBc)
        for idx in np.ndindex(a.shape):
            for x, g in ((a, da), (b, db)):
                xp, xm = x.copy(), x.copy()
                xp[idx] += eps
                xm[idx] -= eps
                if x is a:
                    fd = (_loss_linear(xp, b, gA, gBc) - _loss_linear(xm, b, gA, gBc)) / (2 * eps)
                else:
                    fd = (_loss_linear(a, xp, gA, gBc) - _loss_linear(a, xm, gA, gBc)) / (2 * eps)
                assert abs(fd - g[idx]) <= 1e-7 * max(1.0, abs(fd)), (T, idx, fd, g[idx])


def test_linear_bwd_autograd_bruteforce():
    """Jacobian^T g from torch autograd (fp64, CPU) on an explicit unrolled forward
    built from products/sums (not the recurrence), T <= 8."""
    torch = pytest.importorskip("torch")
    r = rng(107)
    for T in (1, 3, 8):
        a = r.uniform(-1.5, 1.5, size=(2, T, 3))
        b = r.standard_normal((2, T, 3))
        gA, gBc = r.standard_normal((2, T, 3)), r.standard_normal((2, T, 3))
        ta = torch.tensor(a, requires_grad=True)
        tb = torch.tensor(b, requires_grad=True)
        As, Bcs = [], []
        for t in range(T):
            As.append(torch.prod(ta[:, :t + 1], dim=1))
            acc = 0
            for s in range(t + 1):
                acc = acc + torch.prod(ta[:, s + 1:t + 1], dim=1) * tb[:, s]
            Bcs.append(acc)
        L = (torch.stack(As, 1) * torch.tensor(gA)).sum() + (torch.stack(Bcs, 1) * torch.tensor(gBc)).sum()
        L.backward()
        A, Bc = oracle.linear_scan_fwd(a, b)
        da, db = oracle.linear_scan_bwd(a, A, Bc, gA, gBc)
        np.testing.assert_allclose(da, ta.grad.numpy(), rtol=1e-12, atol=1e-12)
        np.testing.assert_allclose(db, tb.grad.numpy(), rtol=1e-12, atol=1e-12)


def test_linear_bwd_dot_product_long():
    """<g, J d> = <J^T g, d> at T=600: J d by central differences along a random
    direction d, J^T g from the oracle backward."""
    r = rng(108)
    T = 600
    a = r.uniform(0.8, 0.99, size=(1, T, 3))
    b = r.standard_normal((1, T, 3))
    gA, gBc = r.standard_normal((1, T, 3)), r.standard_normal((1, T, 3))
    ua, ub = r.standard_normal(a.shape), r.standard_normal(b.shape)
    eps = 1e-6
    jd = (_loss_linear(a + eps * ua, b + eps * ub, gA, gBc)
          - _loss_linear(a - eps * ua, b - eps * ub, gA, gBc)) / (2 * eps)
    A, Bc = oracle.linear_scan_fwd(a, b)
    da, db = oracle.linear_scan_bwd(a, A, Bc, gA, gBc)
    jtg = float(np.sum(da * ua) + np.sum(db * ub))
    assert abs(jd - jtg) <= 1e-7 * abs(jtg), (jd, jtg)


# --------------------------------------------------------------------------
# log-space forward
# --------------------------------------------------------------------------

def test_golden_log():
    g = _golden("log_T3.json")
    lc = np.log(np.array(g["a"])).reshape(1, 3, 1)
    lv = np.log(np.array([g["h0"]] + g["b"])).reshape(1, 4, 1)
    for f in (oracle.scan_log_fwd, oracle.scan_log_fwd_logspace):
        np.testing.assert_allclose(f(lc, lv)[0, :, 0], g["h"], rtol=1e-15)


def test_log_closed_form():
    """Constant a, b and h0: h_t = a^t h0 + b (1 - a^t) / (1 - a)."""
    T = 3000
    for aval, bval, h0 in ((0.5, 0.3, 0.9), (0.99, 0.01, 2.0), (0.9999, 1e-3, 0.1)):
        lc = np.full((1, T, 1), np.log(aval))
        lv = np.full((1, T + 1, 1), np.log(bval))
        lv[0, 0, 0] = np.log(h0)
        t = np.arange(1, T + 1, dtype=np.float64)
        want = aval ** t * h0 + bval * (1 - aval ** t) / (1 - aval)
        for f in (oracle.scan_log_fwd, oracle.scan_log_fwd_logspace):
            np.testing.assert_allclose(f(lc, lv)[0, :, 0], want, rtol=1e-11)


def test_log_two_ways_and_linear_scan():
    """exp of the log-space scan equals the linear-space scan seeded with h0:
    h_t = A_t h0 + Bc_t, on the log workload's distribution."""
    from workloads import log_inputs
    x = log_inputs(2, 700, 6, seed=109)
    lc, lv = x["log_coeffs"], x["log_values"]
    h_lin = oracle.scan_log_fwd(lc, lv)
    h_log = oracle.scan_log_fwd_logspace(lc, lv)
    np.testing.assert_allclose(h_log, h_lin, rtol=1e-13)
    A, Bc = oracle.linear_scan_fwd(np.exp(lc), np.exp(lv[:, 1:]))
    np.testing.assert_allclose(h_lin, A * np.exp(lv[:, :1]) + Bc, rtol=1e-13)


def test_log_extreme_range():
    """Log space survives values whose linear form under/overflows fp64 in the
    intermediate product: a = e^-800 per step then a = 1, b = e^-700."""
    T = 4
    lc = np.array([-800.0, 0.0, 0.0, 0.0]).reshape(1, T, 1)
    lv = np.array([0.0, -700.0, -700.0, -700.0, -700.0]).reshape(1, T + 1, 1)
    h = oracle.scan_log_fwd_logspace(lc, lv)[0, :, 0]
    # h1 = e^-800 + e^-700 ~= e^-700 ; then + e^-700 per step
    want = np.array([1, 2, 3, 4]) * np.exp(-700.0)
    np.testing.assert_allclose(h, want, rtol=1e-12)
    # -inf log value (b = 0) with h0 = 0: everything stays 0
    lv0 = np.full((1, T + 1, 1), -np.inf)
    h0 = oracle.scan_log_fwd_logspace(np.zeros((1, T, 1)), lv0)
    assert np.all(h0 == 0.0)


# --------------------------------------------------------------------------
# log-space backward (the adjoint of parallel_scan_log_fwd)
# --------------------------------------------------------------------------

def _loss_log(lc, lv, g):
    return float(np.sum(g * oracle.scan_log_fwd(lc, lv)))


def test_log_bwd_finite_differences():
    """Central differences of L = <g, h(lc, lv)> with respect to every entry of
    log_coeffs and log_values (slot 0 included), fp64, T <= 8."""
    from workloads import log_inputs
    eps = 1e-6
    for T in (1, 2, 5, 8):
        x = log_inputs(1, T, 2, seed=120 + T)
        lc, lv = x["log_coeffs"], x["log_values"]
        g = rng(130 + T).standard_normal(lc.shape)
        h = oracle.scan_log_fwd(lc, lv)
        dlc, dlv = oracle.scan_log_bwd(lc, lv, h, g)
        for arr, grad in ((lc, dlc), (lv, dlv)):
            for idx in np.ndindex(arr.shape):
                xp, xm = arr.copy(), arr.copy()
                xp[idx] += eps
                xm[idx] -= eps
                if arr is lc:
                    fd = (_loss_log(xp, lv, g) - _loss_log(xm, lv, g)) / (2 * eps)
                else:
                    fd = (_loss_log(lc, xp, g) - _loss_log(lc, xm, g)) / (2 * eps)
                assert abs(fd - grad[idx]) <= 1e-7 * max(1.0, abs(fd)), (T, idx, fd, grad[idx])


def test_log_bwd_matches_linear_adjoint():
    """The log scan is the linear scan with a = e^lc, b = e^lv and h = A h0 + Bc.
    By the chain rule dlc = a * da and dlv_t = b_t * db_t, where (da, db) is the
    linear backward with gA = h0 g and gBc = g; and d log h0 = h0 * sum_t g_t A_t
    (a plain numpy sum, a formula of its own)."""
    from workloads import log_inputs
    x = log_inputs(2, 700, 5, seed=131)
    lc, lv = x["log_coeffs"], x["log_values"]
    g = rng(132).standard_normal(lc.shape)
    h = oracle.scan_log_fwd(lc, lv)
    dlc, dlv = oracle.scan_log_bwd(lc, lv, h, g)
    a, b, h0 = np.exp(lc), np.exp(lv[:, 1:]), np.exp(lv[:, :1])
    A, Bc = oracle.linear_scan_fwd(a, b)
    da, db = oracle.linear_scan_bwd(a, A, Bc, g * h0, g)
    np.testing.assert_allclose(dlc, a * da, rtol=1e-11, atol=1e-300)
    np.testing.assert_allclose(dlv[:, 1:], b * db, rtol=1e-11, atol=1e-300)
    np.testing.assert_allclose(dlv[:, 0], h0[:, 0] * np.sum(g * A, axis=1), rtol=1e-11)


def test_log_bwd_autograd_bruteforce():
    """Jacobian^T g from torch autograd (fp64, CPU) on the explicit unrolled
    forward h_t = h0 prod_{s<=t} a_s + sum_s b_s prod_{s<r<=t} a_r, T <= 8."""
    torch = pytest.importorskip("torch")
    from workloads import log_inputs
    for T in (1, 3, 8):
        x = log_inputs(2, T, 3, seed=140 + T)
        lc, lv = x["log_coeffs"], x["log_values"]
        g = rng(150 + T).standard_normal(lc.shape)
        tlc = torch.tensor(lc, requires_grad=True)
        tlv = torch.tensor(lv, requires_grad=True)
        a, b, h0 = torch.exp(tlc), torch.exp(tlv[:, 1:]), torch.exp(tlv[:, 0])
        hs = []
        for t in range(T):
            acc = h0 * torch.prod(a[:, :t + 1], dim=1)
            for s in range(t + 1):
                acc = acc + torch.prod(a[:, s + 1:t + 1], dim=1) * b[:, s]
            hs.append(acc)
        L = (torch.stack(hs, 1) * torch.tensor(g)).sum()
        L.backward()
        h = oracle.scan_log_fwd(lc, lv)
        dlc, dlv = oracle.scan_log_bwd(lc, lv, h, g)
        np.testing.assert_allclose(dlc, tlc.grad.numpy(), rtol=1e-12, atol=1e-14)
        np.testing.assert_allclose(dlv, tlv.grad.numpy(), rtol=1e-12, atol=1e-14)


def test_log_bwd_unit_coefficients():
    """log a = 0 (a = 1): lam is the reverse cumulative sum of g (numpy), so
    dlc_t = lam_t h_{t-1}, dlv_t = lam_t b_t and d log h0 = lam_1 h0."""
    r = rng(160)
    T, D = 50, 4
    lc = np.zeros((1, T, D))
    lv = np.log(r.uniform(0.1, 1.0, size=(1, T + 1, D)))
    g = r.standard_normal((1, T, D))
    h = oracle.scan_log_fwd(lc, lv)
    dlc, dlv = oracle.scan_log_bwd(lc, lv, h, g)
    lam = np.cumsum(g[:, ::-1], axis=1)[:, ::-1]
    h_prev = np.concatenate([np.exp(lv[:, :1]), h[:, :-1]], axis=1)
    np.testing.assert_allclose(dlc, lam * h_prev, rtol=1e-12)
    np.testing.assert_allclose(dlv[:, 1:], lam * np.exp(lv[:, 1:]), rtol=1e-12)
    np.testing.assert_allclose(dlv[:, 0], lam[:, 0] * np.exp(lv[:, 0]), rtol=1e-12)


# --------------------------------------------------------------------------
# k x k forward
# --------------------------------------------------------------------------

def test_golden_affine():
    g = _golden("affine_k2_v1_T3.json")
    A = np.array(g["A"], dtype=np.float64)[None, :, None]
    Bm = np.array(g["Bm"], dtype=np.float64)[None, :, None]
    Abar, Bbar = oracle.affine_scan_fwd(A, Bm)
    np.testing.assert_array_equal(Abar[0, :, 0], np.array(g["Abar"]))
    np.testing.assert_array_equal(Bbar[0, :, 0], np.array(g["Bbar"]))
    gAbar = np.array(g["gAbar"], dtype=np.float64)[None, :, None]
    gBbar = np.array(g["gBbar"], dtype=np.float64)[None, :, None]
    dA, dB = oracle.affine_scan_bwd(A, Abar, Bbar, gAbar, gBbar)
    np.testing.assert_array_equal(dA[0, :, 0], np.array(g["dA"]))
    np.testing.assert_array_equal(dB[0, :, 0], np.array(g["dB"]))


def _brute_affine(A, Bm):
    """Abar_t = A_t ... A_1 and H_t = sum_s (A_t ... A_{s+1}) B_s by explicit products."""
    Bn, T, n, k, _ = A.shape
    Abar = np.zeros_like(A)
    Bbar = np.zeros_like(Bm)
    for t in range(T):
        for s in range(t + 1):
            P = np.eye(k)
            for r in range(s + 1, t + 1):
                P = A[:, r] @ P
            Bbar[:, t] += P @ Bm[:, s]
        P = np.eye(k)
        for r in range(t + 1):
            P = A[:, r] @ P
        Abar[:, t] = P
    return Abar, Bbar


def test_affine_brute_force_tiny():
    r = rng(110)
    for T, k, v in ((1, 3, 2), (4, 2, 5), (8, 4, 3), (7, 16, 1)):
        A = r.standard_normal((2, T, 3, k, k)) / np.sqrt(k)
        Bm = r.standard_normal((2, T, 3, k, v))
        Abar, Bbar = oracle.affine_scan_fwd(A, Bm)
        Abar2, Bbar2 = _brute_affine(A, Bm)
        np.testing.assert_allclose(Abar, Abar2, rtol=1e-12, atol=1e-13)
        np.testing.assert_allclose(Bbar, Bbar2, rtol=1e-12, atol=1e-13)


def test_affine_k1_matches_channel_scan():
    """k = 1, v = 1 with n = D heads is the channel scan."""
    r = rng(111)
    a = r.uniform(-1.1, 1.1, size=(2, 333, 7))
    b = r.standard_normal((2, 333, 7))
    A, Bc = oracle.linear_scan_fwd(a, b)
    Abar, Bbar = oracle.affine_scan_fwd(a[..., None, None], b[..., None, None])
    np.testing.assert_array_equal(Abar[..., 0, 0], A)
    np.testing.assert_array_equal(Bbar[..., 0, 0], Bc)
    gA, gBc = r.standard_normal(a.shape), r.standard_normal(a.shape)
    da, db = oracle.linear_scan_bwd(a, A, Bc, gA, gBc)
    dA, dB = oracle.affine_scan_bwd(a[..., None, None], Abar, Bbar,
                                    gA[..., None, None], gBc[..., None, None])
    np.testing.assert_allclose(dA[..., 0, 0], da, rtol=1e-15, atol=1e-15)
    np.testing.assert_array_equal(dB[..., 0, 0], db)


def test_affine_diagonal_and_identity():
    r = rng(112)
    T, k, v = 400, 4, 3
    diag = r.uniform(0.8, 0.99, size=(1, T, 2, k))
    A = np.zeros((1, T, 2, k, k))
    A[..., np.arange(k), np.arange(k)] = diag
    Bm = r.standard_normal((1, T, 2, k, v))
    Abar, Bbar = oracle.affine_scan_fwd(A, Bm)
    # diagonal A: Abar diagonal = cumprod, each row i of Bbar is a channel scan with a = diag_i
    np.testing.assert_allclose(np.diagonal(Abar, axis1=-2, axis2=-1), np.cumprod(diag, axis=1), rtol=1e-13)
    off = Abar.copy()
    off[..., np.arange(k), np.arange(k)] = 0
    assert np.all(off == 0)
    for i in range(k):
        _, Bc = oracle.linear_scan_fwd(np.repeat(diag[..., i][..., None], v, -1).reshape(1, T, 2 * v),
                                       Bm[..., i, :].reshape(1, T, 2 * v))
        np.testing.assert_allclose(Bbar[..., i, :].reshape(1, T, 2 * v), Bc, rtol=1e-13, atol=1e-13)
    # identity A: Bbar = cumsum(Bm), Abar = I
    Ai = np.broadcast_to(np.eye(k), (1, T, 2, k, k)).copy()
    Abar, Bbar = oracle.affine_scan_fwd(Ai, Bm)
    np.testing.assert_array_equal(Abar, Ai)
    np.testing.assert_allclose(Bbar, np.cumsum(Bm, axis=1), rtol=1e-12, atol=1e-12)


def test_affine_rotation_closed_form():
    """A_t = rho R(theta_t) (2x2 rotation): Abar_t = rho^t R(theta_1 + ... + theta_t);
    order-sensitive check: with non-commuting shears the composition must be
    A_current @ A_earlier (brute force covers that; here the closed form)."""
    r = rng(113)
    T, rho = 2000, 0.999
    theta = r.uniform(-np.pi, np.pi, size=T)
    c, s = np.cos(theta), np.sin(theta)
    A = np.zeros((1, T, 1, 2, 2))
    A[0, :, 0, 0, 0], A[0, :, 0, 0, 1] = rho * c, -rho * s
    A[0, :, 0, 1, 0], A[0, :, 0, 1, 1] = rho * s, rho * c
    Abar, _ = oracle.affine_scan_fwd(A, np.zeros((1, T, 1, 2, 1)))
    cum = np.cumsum(theta)
    t = np.arange(1, T + 1)
    np.testing.assert_allclose(Abar[0, :, 0, 0, 0], rho ** t * np.cos(cum), atol=1e-11)
    np.testing.assert_allclose(Abar[0, :, 0, 1, 0], rho ** t * np.sin(cum), atol=1e-11)


def test_affine_composition_order():
    """Abar_2 must be A_2 @ A_1, not A_1 @ A_2 (non-commuting pair)."""
    A1 = np.array([[1.0, 1.0], [0.0, 1.0]])
    A2 = np.array([[1.0, 0.0], [1.0, 1.0]])
    A = np.stack([A1, A2])[None, :, None]
    Abar, _ = oracle.affine_scan_fwd(A, np.zeros((1, 2, 1, 2, 1)))
    np.testing.assert_array_equal(Abar[0, 1, 0], A2 @ A1)
    assert not np.array_equal(A2 @ A1, A1 @ A2)


def test_affine_split_time_carry():
    r = rng(114)
    T, T1, k, v = 300, 111, 3, 4
    A = 0.9 * r.standard_normal((1, T, 2, k, k)) / np.sqrt(k)
    Bm = r.standard_normal((1, T, 2, k, v))
    Abar, Bbar = oracle.affine_scan_fwd(A, Bm)
    Abar1, Bbar1 = oracle.affine_scan_fwd(A[:, :T1], Bm[:, :T1])
    Abar2, Bbar2 = oracle.affine_scan_fwd(A[:, T1:], Bm[:, T1:])
    np.testing.assert_allclose(Abar[:, T1:], Abar2 @ Abar1[:, -1:], rtol=1e-10, atol=1e-14)
    np.testing.assert_allclose(Bbar[:, T1:], Abar2 @ Bbar1[:, -1:] + Bbar2, rtol=1e-10, atol=1e-13)


# --------------------------------------------------------------------------
# k x k backward
# --------------------------------------------------------------------------

def _loss_affine(A, Bm, gAbar, gBbar):
    Abar, Bbar = oracle.affine_scan_fwd(A, Bm)
    return float(np.sum(gAbar * Abar) + np.sum(gBbar * Bbar))


def test_affine_bwd_finite_differences():
    r = rng(115)
    eps = 1e-6
    for T, k, v in ((1, 2, 1), (3, 2, 3), (6, 3, 2)):
        A = r.standard_normal((1, T, 1, k, k)) / np.sqrt(k)
        Bm = r.standard_normal((1, T, 1, k, v))
        gAbar, gBbar = r.standard_normal(A.shape), r.standard_normal(Bm.shape)
        Abar, Bbar = oracle.affine_scan_fwd(A, Bm)
        dA, dB = oracle.affine_scan_bwd(A, Abar, Bbar, gAbar, gBbar)
        for x, g in ((A, dA), (Bm, dB)):
            for idx in np.ndindex(x.shape):
                xp, xm = x.copy(), x.copy()
                xp[idx] += eps
                xm[idx] -= eps
                if x is A:
                    fd = (_loss_affine(xp, Bm, gAbar, gBbar) - _loss_affine(xm, Bm, gAbar, gBbar)) / (2 * eps)
                else:
                    fd = (_loss_affine(A, xp, gAbar, gBbar) - _loss_affine(A, xm, gAbar, gBbar)) / (2 * eps)
                assert abs(fd - g[idx]) <= 1e-7 * max(1.0, abs(fd)), (T, k, v, idx, fd, g[idx])


def test_affine_bwd_autograd_bruteforce():
    """J^T g via torch autograd (fp64 CPU) on the explicit-product forward, T <= 8."""
    torch = pytest.importorskip("torch")
    r = rng(116)
    for T, k, v in ((2, 2, 2), (5, 3, 4), (8, 4, 2)):
        A = r.standard_normal((1, T, 2, k, k)) / np.sqrt(k)
        Bm = r.standard_normal((1, T, 2, k, v))
        gAbar, gBbar = r.standard_normal(A.shape), r.standard_normal(Bm.shape)
        tA = torch.tensor(A, requires_grad=True)
        tB = torch.tensor(Bm, requires_grad=True)
        eye = torch.eye(k, dtype=torch.float64)
        L = 0
        for t in range(T):
            P = eye
            for rr in range(t + 1):
                P = tA[:, rr] @ P
            L = L + (P * torch.tensor(gAbar[:, t])).sum()
            H = 0
            for s in range(t + 1):
                Q = eye
                for rr in range(s + 1, t + 1):
                    Q = tA[:, rr] @ Q
                H = H + Q @ tB[:, s]
            L = L + (H * torch.tensor(gBbar[:, t])).sum()
        L.backward()
        Abar, Bbar = oracle.affine_scan_fwd(A, Bm)
        dA, dB = oracle.affine_scan_bwd(A, Abar, Bbar, gAbar, gBbar)
        np.testing.assert_allclose(dA, tA.grad.numpy(), rtol=1e-11, atol=1e-12)
        np.testing.assert_allclose(dB, tB.grad.numpy(), rtol=1e-11, atol=1e-12)


def test_affine_bwd_dot_product_long():
    r = rng(117)
    T, k, v = 400, 4, 3
    A = 0.95 * r.standard_normal((1, T, 2, k, k)) / np.sqrt(k)
    Bm = r.standard_normal((1, T, 2, k, v))
    gAbar, gBbar = r.standard_normal(A.shape), r.standard_normal(Bm.shape)
    uA, uB = r.standard_normal(A.shape), r.standard_normal(Bm.shape)
    eps = 1e-6
    jd = (_loss_affine(A + eps * uA, Bm + eps * uB, gAbar, gBbar)
          - _loss_affine(A - eps * uA, Bm - eps * uB, gAbar, gBbar)) / (2 * eps)
    Abar, Bbar = oracle.affine_scan_fwd(A, Bm)
    dA, dB = oracle.affine_scan_bwd(A, Abar, Bbar, gAbar, gBbar)
    jtg = float(np.sum(dA * uA) + np.sum(dB * uB))
    assert abs(jd - jtg) <= 1e-6 * abs(jtg), (jd, jtg)


# --------------------------------------------------------------------------
# given initial state (h0 / H0)
# --------------------------------------------------------------------------

def test_h0_linear_is_the_composed_state():
    """H from h0 equals A * h0 + Bc of the zero-state scan (a numpy product of
    two independent oracle outputs); h0 = None is the zero-state scan."""
    r = rng(170)
    a = r.uniform(0.5, 0.999, size=(2, 300, 4))
    b = r.standard_normal((2, 300, 4))
    h0 = r.standard_normal((2, 4))
    A, H = oracle.linear_scan_fwd_h0(a, b, h0)
    A0, Bc = oracle.linear_scan_fwd(a, b)
    np.testing.assert_array_equal(A, A0)
    np.testing.assert_allclose(H, A0 * h0[:, None, :] + Bc, rtol=1e-12, atol=1e-12)
    _, H_none = oracle.linear_scan_fwd_h0(a, b, None)
    np.testing.assert_array_equal(H_none, Bc)


def test_h0_linear_closed_form():
    """Constant a, b: H_t = a^t h0 + b (1 - a^t) / (1 - a)."""
    T = 2000
    for aval, bval, h0 in ((0.5, 0.3, -2.0), (0.99, 0.01, 5.0)):
        a = np.full((1, T, 1), aval)
        b = np.full((1, T, 1), bval)
        _, H = oracle.linear_scan_fwd_h0(a, b, np.array([[h0]]))
        t = np.arange(1, T + 1, dtype=np.float64)
        np.testing.assert_allclose(H[0, :, 0], aval ** t * h0 + bval * (1 - aval ** t) / (1 - aval), rtol=1e-11)


def test_h0_linear_resume():
    """Scanning [0, T) equals scanning [0, T1) and resuming [T1, T) from the
    last state: the semantics that carries state across calls."""
    r = rng(171)
    a = r.uniform(0.5, 1.0, size=(2, 90, 3))
    b = r.standard_normal((2, 90, 3))
    h0 = r.standard_normal((2, 3))
    A, H = oracle.linear_scan_fwd_h0(a, b, h0)
    for T1 in (1, 37, 89):
        A1, H1 = oracle.linear_scan_fwd_h0(a[:, :T1], b[:, :T1], h0)
        A2, H2 = oracle.linear_scan_fwd_h0(a[:, T1:], b[:, T1:], H1[:, -1])
        np.testing.assert_allclose(H[:, T1:], H2, rtol=1e-12, atol=1e-12)
        np.testing.assert_allclose(A[:, T1:], A2 * A1[:, -1:], rtol=1e-13)


def _loss_linear_h0(a, b, h0, gA, gH):
    A, H = oracle.linear_scan_fwd_h0(a, b, h0)
    return float(np.sum(gA * A) + np.sum(gH * H))


def test_h0_linear_bwd_finite_differences():
    r = rng(172)
    eps = 1e-6
    for T in (1, 2, 6):
        a = r.uniform(-1.2, 1.2, size=(1, T, 2))
        b = r.standard_normal((1, T, 2))
        h0 = r.standard_normal((1, 2))
        gA, gH = r.standard_normal((1, T, 2)), r.standard_normal((1, T, 2))
        A, H = oracle.linear_scan_fwd_h0(a, b, h0)
        da, db, dh0 = oracle.linear_scan_bwd_h0(a, A, H, h0, gA, gH)
        for x, g in ((a, da), (b, db), (h0, dh0)):
            for idx in np.ndindex(x.shape):
                xp, xm = x.copy(), x.copy()
                xp[idx] += eps
                xm[idx] -= eps
                args_p = [xp if y is x else y for y in (a, b, h0)]
                args_m = [xm if y is x else y for y in (a, b, h0)]
                fd = (_loss_linear_h0(*args_p, gA, gH) - _loss_linear_h0(*args_m, gA, gH)) / (2 * eps)
                assert abs(fd - g[idx]) <= 1e-7 * max(1.0, abs(fd)), (T, idx, fd, g[idx])


def test_h0_linear_bwd_zero_state_agrees():
    """With h0 = None the gradient equals lrs_oracle_linear_bwd's, and dh0 is
    sum_t gH_t A_t (a numpy sum, a formula of its own)."""
    r = rng(173)
    a = r.uniform(0.5, 0.999, size=(2, 200, 3))
    b = r.standard_normal((2, 200, 3))
    gA, gH = r.standard_normal(a.shape), r.standard_normal(a.shape)
    A, Bc = oracle.linear_scan_fwd(a, b)
    da0, db0 = oracle.linear_scan_bwd(a, A, Bc, gA, gH)
    da, db, dh0 = oracle.linear_scan_bwd_h0(a, A, Bc, None, gA, gH)
    np.testing.assert_array_equal(da, da0)
    np.testing.assert_array_equal(db, db0)
    np.testing.assert_allclose(dh0, np.sum(gH * A, axis=1), rtol=1e-11)


def test_h0_affine_is_the_composed_state():
    """H from H0 equals Abar @ H0 + Bbar of the zero-state scan (numpy matmul of
    independent oracle outputs)."""
    r = rng(174)
    from workloads import affine_inputs_diag
    x = affine_inputs_diag(2, 120, 3, 4, 5, seed=175)
    H0 = r.standard_normal((2, 3, 4, 5))
    Abar, H = oracle.affine_scan_fwd_h0(x["A"], x["Bm"], H0)
    Abar0, Bbar = oracle.affine_scan_fwd(x["A"], x["Bm"])
    np.testing.assert_array_equal(Abar, Abar0)
    np.testing.assert_allclose(H, np.matmul(Abar0, H0[:, None]) + Bbar, rtol=1e-11, atol=1e-12)


def test_h0_affine_resume():
    r = rng(176)
    from workloads import affine_inputs_rotation
    x = affine_inputs_rotation(1, 60, 2, 3, 4, seed=177)
    H0 = r.standard_normal((1, 2, 3, 4))
    Abar, H = oracle.affine_scan_fwd_h0(x["A"], x["Bm"], H0)
    for T1 in (1, 25):
        Ab1, H1 = oracle.affine_scan_fwd_h0(x["A"][:, :T1], x["Bm"][:, :T1], H0)
        Ab2, H2 = oracle.affine_scan_fwd_h0(x["A"][:, T1:], x["Bm"][:, T1:], H1[:, -1])
        np.testing.assert_allclose(H[:, T1:], H2, rtol=1e-11, atol=1e-12)
        np.testing.assert_allclose(Abar[:, T1:], np.matmul(Ab2, Ab1[:, -1:]), rtol=1e-11, atol=1e-12)


def _loss_affine_h0(A, Bm, H0, gAbar, gH):
    Abar, H = oracle.affine_scan_fwd_h0(A, Bm, H0)
    return float(np.sum(gAbar * Abar) + np.sum(gH * H))


def test_h0_affine_bwd_finite_differences():
    r = rng(178)
    eps = 1e-6
    for T, k, v in ((1, 2, 3), (4, 3, 2)):
        A = r.uniform(-0.9, 0.9, size=(1, T, 1, k, k))
        Bm = r.standard_normal((1, T, 1, k, v))
        H0 = r.standard_normal((1, 1, k, v))
        gAbar, gH = r.standard_normal(A.shape), r.standard_normal(Bm.shape)
        Abar, H = oracle.affine_scan_fwd_h0(A, Bm, H0)
        dA, dB, dH0 = oracle.affine_scan_bwd_h0(A, Abar, H, H0, gAbar, gH)
        for x, g in ((A, dA), (Bm, dB), (H0, dH0)):
            for idx in np.ndindex(x.shape):
                xp, xm = x.copy(), x.copy()
                xp[idx] += eps
                xm[idx] -= eps
                args_p = [xp if y is x else y for y in (A, Bm, H0)]
                args_m = [xm if y is x else y for y in (A, Bm, H0)]
                fd = (_loss_affine_h0(*args_p, gAbar, gH) - _loss_affine_h0(*args_m, gAbar, gH)) / (2 * eps)
                assert abs(fd - g[idx]) <= 1e-7 * max(1.0, abs(fd)), (T, k, v, idx, fd, g[idx])


def test_h0_affine_bwd_zero_state_agrees():
    """H0 = None gives lrs_oracle_affine_bwd's gradient; dH0 = sum_t Abar_t^T gH_t
    (numpy, a formula of its own: H_t depends on H0 through Abar_t H0)."""
    from workloads import affine_inputs_diag
    x = affine_inputs_diag(1, 80, 2, 3, 4, seed=179, grads=True)
    Abar, Bbar = oracle.affine_scan_fwd(x["A"], x["Bm"])
    dA0, dB0 = oracle.affine_scan_bwd(x["A"], Abar, Bbar, x["gAbar"], x["gBbar"])
    dA, dB, dH0 = oracle.affine_scan_bwd_h0(x["A"], Abar, Bbar, None, x["gAbar"], x["gBbar"])
    np.testing.assert_array_equal(dA, dA0)
    np.testing.assert_array_equal(dB, dB0)
    want = np.sum(np.matmul(np.swapaxes(Abar, -1, -2), x["gBbar"]), axis=1)
    np.testing.assert_allclose(dH0, want, rtol=1e-10, atol=1e-12)


def test_oracle_threads_reported():
    assert oracle.num_threads() >= 1
