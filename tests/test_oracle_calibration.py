"""Pins for the oracle's calibration helpers (lambda * L = alpha * exp(beta * s))."""

import math

import numpy as np
import pytest

import oracle


def test_fit_recovers_known_alpha_beta_exactly():
    alpha, beta = 3.7, 4.2
    Ls, ss, lams = [], [], []
    for L in [4096, 8192, 16384, 32768, 65536, 131072]:
        for s in [0.3, 0.5, 0.7]:
            Ls.append(L)
            ss.append(s)
            lams.append(alpha * math.exp(beta * s) / L)
    a, b, rmse = oracle.fit_alpha_beta(Ls, ss, lams)
    assert abs(a - alpha) < 1e-10 and abs(b - beta) < 1e-12 and rmse < 1e-12
    assert abs(oracle.lambda_for(a, b, 0.5, 8192) - alpha * math.exp(beta * 0.5) / 8192) < 1e-15


def test_fit_is_least_squares():
    """Perturbing the fitted line in any direction increases the squared residual."""
    rng = np.random.default_rng(0)
    s = rng.uniform(0.2, 0.8, 30)
    L = rng.choice([4096, 8192, 65536], 30)
    lam = np.exp(0.5 + 3.0 * s + 0.1 * rng.standard_normal(30)) / L
    a, b, rmse = oracle.fit_alpha_beta(L, s, lam)
    y = np.log(lam * L)

    def sse(la, bb):
        return float(((y - la - bb * s) ** 2).sum())
    best = sse(math.log(a), b)
    assert abs(math.sqrt(best / 30) - rmse) < 1e-12
    for d in [(1e-3, 0), (-1e-3, 0), (0, 1e-3), (0, -1e-3)]:
        assert sse(math.log(a) + d[0], b + d[1]) > best


@pytest.mark.parametrize("N", [7, 100, 1001])
def test_quantile_hits_target_within_one_over_n(N):
    rng = np.random.default_rng(N)
    c = -np.abs(rng.standard_normal(N)) * 5.0
    c[: max(1, N // 10)] = np.inf            # first blocks of splits
    c = np.concatenate([c, [np.nan, np.nan]])  # not-live entries are ignored
    for s in [0.0, 0.1, 0.3, 0.5, 0.7, 0.85]:
        ln_lam = oracle.quantile_ln_lambda(c, s)
        got = oracle.achieved_sparsity(c, ln_lam)
        assert ln_lam <= 0.0
        assert abs(got - s) <= 1.0 / N + 1e-12, (s, got)
    # a target above what lambda <= 1 can reach is capped at ln(lambda) = 0
    ln_lam = oracle.quantile_ln_lambda(c, 0.99)
    assert ln_lam == 0.0
    assert oracle.achieved_sparsity(c, ln_lam) <= 0.99


def test_quantile_zero_is_dense():
    assert oracle.quantile_ln_lambda([-1.0, -2.0, np.inf], 0.0) == -math.inf
