"""Threshold calibration, fp64 (oracle; test infrastructure only).

The pages: lambda = a / L ([xllm] 核心公式, threshold calibration), and a calibration model
lambda * L = alpha * exp(beta * s) for a target sparsity s ([xllm] 核心公式, calibration model;
[gist-de] Kalibrierung), fitted from one forward pass over a sample ([xllm] 模型组件,
calibration module).

Readings where the pages are silent:
  * Sparsity at a threshold is the fraction of critical values below ln(lambda): a live
    tile-block is skipped iff its critical value c < ln(lambda) (closed form of the rule).
  * Quantile inversion: with the N critical values sorted ascending, k = ceil(s * N), ln(lambda)
    is the midpoint of the k-th and (k+1)-th values (1-based).  It is capped at 0 (lambda <= 1);
    s = 0 gives lambda = 0 (dense).
  * The fit is ordinary least squares of y = ln(lambda * L) on x = s, i.e. ln(alpha) + beta * s.
"""

from __future__ import annotations

import math

import numpy as np


def achieved_sparsity(crit, ln_lam: float) -> float:
    """Fraction of critical values strictly below ln(lambda); nan entries (not live) ignored."""
    c = np.asarray(crit, dtype=np.float64).ravel()
    c = c[~np.isnan(c)]
    if c.size == 0:
        return 0.0
    return float(np.count_nonzero(c < ln_lam)) / c.size


def quantile_ln_lambda(crit, s: float) -> float:
    """ln(lambda) such that a fraction s of the critical values lies below it (midpoint rule)."""
    if not (0.0 <= s <= 1.0):
        raise ValueError("s must lie in [0, 1]")
    c = np.sort(np.asarray(crit, dtype=np.float64).ravel()[~np.isnan(np.asarray(crit, dtype=np.float64).ravel())])
    N = c.size
    if N == 0:
        raise ValueError("no critical values")
    k = math.ceil(s * N)
    if k <= 0:
        return -math.inf
    lo = c[k - 1]
    hi = c[k] if k < N else math.inf
    if lo == math.inf:
        return 0.0
    mid = hi if lo == hi else (lo + hi) / 2.0 if math.isfinite(hi) else lo + 1.0
    return min(0.0, mid)


def fit_alpha_beta(L, s, lam):
    """OLS fit of ln(lambda * L) = ln(alpha) + beta * s.  Returns (alpha, beta, rmse of ln(lambda*L))."""
    L = np.asarray(L, dtype=np.float64)
    s = np.asarray(s, dtype=np.float64)
    lam = np.asarray(lam, dtype=np.float64)
    if L.size < 2 or np.any(lam <= 0) or np.any(L <= 0):
        raise ValueError("need >= 2 points with lambda > 0 and L > 0")
    y = np.log(lam * L)
    xm, ym = s.mean(), y.mean()
    sxx = ((s - xm) ** 2).sum()
    if sxx == 0:
        raise ValueError("all target sparsities equal; beta is not identifiable")
    beta = ((s - xm) * (y - ym)).sum() / sxx
    ln_alpha = ym - beta * xm
    resid = y - (ln_alpha + beta * s)
    return math.exp(ln_alpha), beta, math.sqrt((resid ** 2).mean())


def lambda_for(alpha: float, beta: float, s: float, L: float) -> float:
    """Deployed threshold lambda(L, s) = alpha * exp(beta * s) / L, capped at 1."""
    return min(1.0, alpha * math.exp(beta * s) / L)
