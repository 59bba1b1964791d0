"""Shared helpers for the GPU parity tests: quantise seeded inputs once, hand the
same values to the HIP path (on the GPU) and to the oracle (widened to fp64),
and measure the error the way the tolerances are stated.

Error readings (the pages give only "max relative error"):
  * channel and log scans: e = max_i |g_i - r_i| / (s_i + 2^-100), where s_i is
    the oracle run on the absolute values of every input -- the sum of the
    magnitudes of all terms that make up output i.  For A and for the log
    output every term is positive, so s_i = |r_i| and e is the plain relative
    error; for Bc, da, db it is the error relative to the summation's own
    magnitude, the only relative error a signed sum can promise.
  * k x k scans: per (b, t, head) block, max |G - R| / (max |R| + 2^-100).
  * any non-finite GPU value where the oracle is finite is an infinite error.
  * 2^-100 only matters where the true value underflows fp32 (running
    products of hundreds of factors below one).
Tolerances: 1e-5 for fp32 storage, 2e-2 for bf16 storage with fp32 arithmetic,
and 2.5e-3 for fp16 storage with fp32 arithmetic: the bf16 bar scaled by the
ratio of the two formats' unit roundoffs (2^-11 / 2^-8).  With fp16 storage the
denominator is at least 2^-14, fp16's smallest normal: below it the format
keeps only an absolute precision of 2^-25 (its subnormal grid), so outputs
there are compared to that grid rather than to their own magnitude.
"""
import numpy as np
import torch

TOL = {torch.float32: 1e-5, torch.bfloat16: 2e-2, torch.float16: 2.5e-3}
TINY = 2.0 ** -100
# Smallest error denominator per storage type (see above).
FLOOR = {torch.float32: TINY, torch.bfloat16: TINY, torch.float16: 2.0 ** -14}


def quantise(x: np.ndarray, dtype):
    """(device tensor, the same values widened to fp64 as numpy)."""
    t = torch.from_numpy(np.ascontiguousarray(x)).to(dtype)
    return t.cuda(), t.double().numpy()


def to_np(t: torch.Tensor) -> np.ndarray:
    return t.detach().double().cpu().numpy()


def scaled_err(g: np.ndarray, r: np.ndarray, s: np.ndarray, floor: float = TINY) -> float:
    g = np.asarray(g, dtype=np.float64)
    if np.any(~np.isfinite(g) & np.isfinite(r)):
        return float("inf")
    den = np.maximum(np.abs(s) + TINY, floor)
    return float(np.max(np.abs(g - r) / den)) if g.size else 0.0


def block_err(G: np.ndarray, R: np.ndarray) -> float:
    G = np.asarray(G, dtype=np.float64)
    if np.any(~np.isfinite(G) & np.isfinite(R)):
        return float("inf")
    num = np.max(np.abs(G - R), axis=(-2, -1))
    den = np.max(np.abs(R), axis=(-2, -1)) + TINY
    return float(np.max(num / den)) if G.size else 0.0


def timeouts(ws: torch.Tensor) -> int:
    """Word 1 of a workspace: cross-workgroup waits that hit their spin limit."""
    return int(ws[4:8].cpu().view(torch.int32).item())
