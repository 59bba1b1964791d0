"""Seeded synthetic inputs for the five scan workloads.

This module only draws random numbers and shapes them.  It holds none of the
scans' arithmetic, imports neither the oracle nor the HIP library, and is shared
by both sides (tests, smoke check, benchmark) so that they see identical inputs.

Every array is drawn in fp64 from ``numpy.random.Generator(PCG64(seed))``.  The
caller casts it to the device dtype (fp32 or bf16, round-to-nearest-even) and, for
the oracle, widens that cast value back to fp64, so both sides start from the
same numbers.

Workloads (the recurrence h_t = a_t h_{t-1} + b_t and its k x k form, as the
minGRU "Triton kernels" page defines the ops):

  1. linear_fwd_small   k=1 fp32,  B=1, T=1024, D=64;    a~U(0.5,0.999), b~N(0,1)
  2. log_fwd            log fp32,  B=4, T=4096, D=512;   log_coeffs=-softplus(N(0,1)),
                        log_values[:,0]=log h0, h0~U(0.1,1); log_values[:,1:]=
                        log(sigmoid(N(0,1)) * U(0.1,1))
  3. linear_fwd_bwd     k=1 bf16,  B=8, T=8192, D=4096;  a~U(0.9,0.9999), b,gA,gBc~N(0,1)
  4. affine_fwd_k4      k x k fp32, B=2, T=2048, n=64, k=4, v=16; A_t=0.95*Q_t with
                        Q_t Haar-random orthogonal; Bm~N(0, 0.1^2)
  5. affine_fwd_bwd_k8  k x k fp32, B=4, T=4096, n=32, k=8, v=32; A_t=diag(U(0.8,0.99))
                        + off-diagonal N(0, 0.01^2); Bm~N(0,0.1^2); gAbar,gBbar~N(0,1)

"N(0, s)" is read as standard deviation s.
"""
from __future__ import annotations

import numpy as np

WORKLOADS = {
    1: dict(name="linear_fwd_small", op="linear", dtype="f32", B=1, T=1024, D=64),
    2: dict(name="log_fwd", op="log", dtype="f32", B=4, T=4096, D=512),
    3: dict(name="linear_fwd_bwd", op="linear", dtype="bf16", B=8, T=8192, D=4096),
    4: dict(name="affine_fwd_k4", op="affine", dtype="f32", B=2, T=2048, n=64, k=4, v=16),
    5: dict(name="affine_fwd_bwd_k8", op="affine", dtype="f32", B=4, T=4096, n=32, k=8, v=32),
    # the log-space scan's forward and its adjoint at the workload-2 size
    6: dict(name="log_fwd_bwd", op="log", dtype="f32", B=4, T=4096, D=512),
}


def rng(seed: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(seed))


def linear_inputs(B, T, D, seed, a_lo=0.5, a_hi=0.999, grads=False):
    """a ~ U(a_lo, a_hi), b ~ N(0,1); with grads, also gA, gBc ~ N(0,1).  All (B,T,D)."""
    g = rng(seed)
    out = {"a": g.uniform(a_lo, a_hi, size=(B, T, D)),
           "b": g.standard_normal(size=(B, T, D))}
    if grads:
        out["gA"] = g.standard_normal(size=(B, T, D))
        out["gBc"] = g.standard_normal(size=(B, T, D))
    return out


def log_inputs(B, T, D, seed, grads=False):
    """log_coeffs (B,T,D) = -softplus(x), x~N(0,1), taken as -logaddexp(0, x);
    log_values (B,T+1,D): slot 0 = log h0 with h0~U(0.1,1) per (b,d);
    slots 1..T = log(sigmoid(y) * u), y~N(0,1), u~U(0.1,1).
    grads: also an upstream gradient g = dL/dh (B,T,D) ~ N(0,1)."""
    g = rng(seed)
    x = g.standard_normal(size=(B, T, D))
    log_coeffs = -np.logaddexp(0.0, x)
    h0 = g.uniform(0.1, 1.0, size=(B, 1, D))
    y = g.standard_normal(size=(B, T, D))
    u = g.uniform(0.1, 1.0, size=(B, T, D))
    # log(sigmoid(y)) = -logaddexp(0, -y)
    lv_rest = -np.logaddexp(0.0, -y) + np.log(u)
    log_values = np.concatenate([np.log(h0), lv_rest], axis=1)
    out = {"log_coeffs": log_coeffs, "log_values": log_values}
    if grads:
        out["g"] = g.standard_normal(size=(B, T, D))
    return out


def haar_orthogonal(g: np.random.Generator, shape, k):
    """Haar-distributed k x k orthogonal matrices: QR of a N(0,1) matrix with the
    signs of diag(R) folded into Q."""
    Z = g.standard_normal(size=tuple(shape) + (k, k))
    Q, R = np.linalg.qr(Z)
    d = np.sign(np.diagonal(R, axis1=-2, axis2=-1))
    d[d == 0] = 1.0
    return Q * d[..., None, :]


def affine_inputs_rotation(B, T, n, k, v, seed, rho=0.95):
    """A_t = rho * Q_t (Haar orthogonal), Bm ~ N(0, 0.1^2)."""
    g = rng(seed)
    A = rho * haar_orthogonal(g, (B, T, n), k)
    Bm = 0.1 * g.standard_normal(size=(B, T, n, k, v))
    return {"A": A, "Bm": Bm}


def affine_inputs_diag(B, T, n, k, v, seed, grads=False):
    """A_t = diag(U(0.8,0.99)) + off-diagonal N(0, 0.01^2); Bm ~ N(0, 0.1^2);
    with grads, gAbar (B,T,n,k,k) and gBbar (B,T,n,k,v) ~ N(0,1)."""
    g = rng(seed)
    off = 0.01 * g.standard_normal(size=(B, T, n, k, k))
    diag = g.uniform(0.8, 0.99, size=(B, T, n, k))
    eye = np.eye(k, dtype=bool)
    A = np.where(eye, 0.0, off)
    A[..., np.arange(k), np.arange(k)] = diag
    Bm = 0.1 * g.standard_normal(size=(B, T, n, k, v))
    out = {"A": A, "Bm": Bm}
    if grads:
        out["gAbar"] = g.standard_normal(size=(B, T, n, k, k))
        out["gBbar"] = g.standard_normal(size=(B, T, n, k, v))
    return out


def workload_inputs(wid: int, seed: int | None = None, **shape):
    """Inputs of workload ``wid`` (1..6) at its own sizes, or at sizes overridden by
    keyword (B, T, D or B, T, n, k, v), with the workload's distributions."""
    w = dict(WORKLOADS[wid])
    w.update(shape)
    s = wid if seed is None else seed
    if wid == 1:
        return linear_inputs(w["B"], w["T"], w["D"], s)
    if wid == 2:
        return log_inputs(w["B"], w["T"], w["D"], s)
    if wid == 3:
        return linear_inputs(w["B"], w["T"], w["D"], s, 0.9, 0.9999, grads=True)
    if wid == 4:
        return affine_inputs_rotation(w["B"], w["T"], w["n"], w["k"], w["v"], s)
    if wid == 5:
        return affine_inputs_diag(w["B"], w["T"], w["n"], w["k"], w["v"], s, grads=True)
    if wid == 6:
        return log_inputs(w["B"], w["T"], w["D"], s, grads=True)
    raise KeyError(wid)
