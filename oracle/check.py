"""Pass rules for a computed D against the oracle (test infrastructure only).

* Random inputs, fp32 output: ``|D - D_ref| <= 2^-12 * S + 1e-6`` per element,
  ``S = sum_k |a*b|``, and D finite.  ``2^-12 = K * 2^-24`` at K = 4096 is the
  classical worst-case bound of a sequential fp32 sum.
* Integer-valued inputs: ``D == D_ref`` exactly (every partial sum is an
  integer below 2^24, so any summation order gives the same fp32 value).
* bf16 output: the same kernel with fp32 output meets the rule above, and the
  bf16 result equals the round-to-nearest-even of that fp32 result bit for
  bit; against the oracle alone the bound gains the bf16 half-ulp,
  ``2^-8 * |D_ref|``.

Block Freivalds: ``D[:, J] @ x_J`` against ``A @ (B_J^T x_J) + C[:, J] @ x_J``
for column blocks J, in float64, with the bound summed from the per-element
tolerances (exact in integer mode).  It checks every element of a large D at
once in O((M + N) K N / w) work and catches any wrong block or tile that
sampled checks could miss.
"""
from __future__ import annotations

import numpy as np

TOL_REL = 2.0 ** -12
TOL_ABS = 1e-6


def tolerance(S):
    return TOL_REL * np.asarray(S, dtype=np.float64) + TOL_ABS


def within_tolerance(D, D_ref, S, extra_rel=0.0):
    """Boolean mask: finite and ``|D - D_ref| <= 2^-12 S + 1e-6 (+ extra_rel |D_ref|)``."""
    D = np.asarray(D, dtype=np.float64)
    D_ref = np.asarray(D_ref, dtype=np.float64)
    bound = tolerance(S) + extra_rel * np.abs(D_ref)
    return np.isfinite(D) & (np.abs(D - D_ref) <= bound)


def report(D, D_ref, S, extra_rel=0.0):
    """Summary dict: count, failures, worst error relative to its bound."""
    D = np.asarray(D, dtype=np.float64)
    D_ref = np.asarray(D_ref, dtype=np.float64)
    bound = tolerance(S) + extra_rel * np.abs(D_ref)
    err = np.abs(D - D_ref)
    ok = np.isfinite(D) & (err <= bound)
    ratio = np.where(np.isfinite(err), err / bound, np.inf)
    return {"n": int(D.size), "fail": int((~ok).sum()),
            "max_err_over_bound": float(ratio.max()) if D.size else 0.0,
            "max_abs_err": float(np.nanmax(err)) if D.size else 0.0}


def freivalds_blocks(D, a, b, c=None, block=64, seed=12345, integer=False):
    """Block-Freivalds check of a whole D (float64 operands from ``operands_f64``).

    ``D``: (M, N) result under test; ``a``: (M, K); ``b``: (N, K); ``c``: (M, N)
    or None.  Returns ``(ok, worst_ratio)`` with ``worst_ratio`` the largest
    ``|lhs - rhs| / bound`` over all (row, block) pairs (0 is exact).
    """
    D = np.asarray(D, dtype=np.float64)
    M, N = D.shape
    rng = np.random.default_rng(seed)
    x = rng.choice(np.array([-1.0, 1.0]), size=N)
    nb = (N + block - 1) // block
    # X: (N, nb) block-diagonal spread of x
    X = np.zeros((N, nb))
    X[np.arange(N), np.arange(N) // block] = x
    lhs = D @ X
    rhs = a @ (b.T @ X)
    if c is not None:
        rhs = rhs + np.asarray(c, dtype=np.float64) @ X
    diff = np.abs(lhs - rhs)
    if integer:
        ok = bool(np.all(diff == 0)) and bool(np.all(np.isfinite(D)))
        return ok, float(diff.max()) if diff.size else 0.0
    absX = np.abs(X)
    Ssum = np.abs(a) @ (np.abs(b).T @ absX)            # sum_n |x_n| S_mn per block
    bound = TOL_REL * Ssum + TOL_ABS * absX.sum(axis=0)[None, :]
    # slack for the float64 evaluation of both sides
    mag = np.abs(D) @ absX + Ssum
    if c is not None:
        mag = mag + np.abs(np.asarray(c, dtype=np.float64)) @ absX
    bound = bound + 1e-12 * mag
    ratio = diff / bound
    ok = bool(np.all(ratio <= 1.0)) and bool(np.all(np.isfinite(D)))
    return ok, float(ratio.max()) if ratio.size else 0.0
