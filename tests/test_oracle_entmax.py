"""Pins of the oracle's exact alpha-entmax against mathematics it does not share code with.

* closed forms derived by hand (tests/golden/entmax_closed_form.txt);
* brute force over every support for tiny inputs (optimality conditions);
* the variational definition (maximise p.z + Tsallis entropy over the simplex),
  solved by a generic constrained optimiser;
* sparsemax (alpha = 2) as the Euclidean projection onto the simplex;
* the softmax limit alpha -> 1;
* invariants: sum to one, non-negative, support <=> u > tau, tau bracket,
  translation invariance, permutation equivariance, one candidate -> p = 1.
"""

import os

import numpy as np
import pytest
from scipy.optimize import minimize

from oracle.entmax import (
    entmax,
    entmax_backward,
    entmax_threshold,
    entmax_threshold_bruteforce,
    entmax_threshold_rows,
)

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "entmax_closed_form.txt")
ALPHAS = [1.25, 1.333, 1.5, 2.0, 3.0]


def _golden_rows():
    rows = []
    with open(GOLDEN) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            a, z, t, p, _ = [x.strip() for x in line.split("|")]
            rows.append((float(a), [float(v) for v in z.split(",")], float(t), [float(v) for v in p.split(",")]))
    return rows


@pytest.mark.parametrize("alpha,z,tau,p", _golden_rows())
def test_golden_closed_forms(alpha, z, tau, p):
    assert entmax_threshold(z, alpha) == pytest.approx(tau, abs=1e-12)
    np.testing.assert_allclose(entmax(z, alpha), p, atol=1e-12)
    np.testing.assert_allclose(entmax_threshold_rows(np.array([z]), alpha), [tau], atol=1e-12)


@pytest.mark.parametrize("alpha", ALPHAS)
@pytest.mark.parametrize("n", [1, 2, 3, 5, 8, 10])
def test_bruteforce_support(alpha, n):
    rng = np.random.default_rng(100 + n)
    for scale in (0.3, 1.0, 4.0):
        z = rng.normal(size=n) * scale
        t_bf = entmax_threshold_bruteforce(z, alpha)
        assert entmax_threshold(z, alpha) == pytest.approx(t_bf, abs=1e-9)
        assert entmax_threshold_rows(z[None, :], alpha)[0] == pytest.approx(t_bf, abs=1e-9)


def _tsallis_argmax(z, alpha):
    """argmax_{p in simplex} p.z + (sum p - p^alpha) / (alpha (alpha - 1)), generic SLSQP."""
    n = len(z)

    def neg(p):
        p = np.clip(p, 0.0, None)
        return -(p @ z + np.sum(p - p**alpha) / (alpha * (alpha - 1.0)))

    res = minimize(
        neg,
        np.full(n, 1.0 / n),
        method="SLSQP",
        bounds=[(0.0, 1.0)] * n,
        constraints=[{"type": "eq", "fun": lambda p: np.sum(p) - 1.0}],
        options={"ftol": 1e-14, "maxiter": 500},
    )
    assert res.success
    return res.x


@pytest.mark.parametrize("alpha", [1.5, 2.0, 1.333])
def test_variational_definition(alpha):
    rng = np.random.default_rng(7)
    for _ in range(5):
        z = rng.normal(size=6) * 1.5
        np.testing.assert_allclose(entmax(z, alpha), _tsallis_argmax(z, alpha), atol=2e-5)


def test_sparsemax_is_simplex_projection():
    rng = np.random.default_rng(11)
    for _ in range(10):
        z = rng.normal(size=7)
        res = minimize(
            lambda p: np.sum((p - z) ** 2),
            np.full(7, 1 / 7),
            method="SLSQP",
            bounds=[(0.0, None)] * 7,
            constraints=[{"type": "eq", "fun": lambda p: np.sum(p) - 1.0}],
            options={"ftol": 1e-15, "maxiter": 500},
        )
        np.testing.assert_allclose(entmax(z, 2.0), res.x, atol=1e-6)


def test_softmax_limit():
    rng = np.random.default_rng(3)
    z = rng.normal(size=32)
    sm = np.exp(z - z.max())
    sm /= sm.sum()
    errs = [np.abs(entmax(z, a) - sm).sum() for a in (1.1, 1.01, 1.001)]
    assert errs[0] > errs[1] > errs[2]
    assert errs[2] < 5e-3


@pytest.mark.parametrize("alpha", ALPHAS)
def test_invariants(alpha):
    rng = np.random.default_rng(5)
    for n in (1, 4, 33, 300):
        z = rng.normal(size=n) * 2.0
        p = entmax(z, alpha)
        tau = entmax_threshold(z, alpha)
        u = (alpha - 1.0) * z
        assert p.sum() == pytest.approx(1.0, abs=1e-10)
        assert np.all(p >= 0)
        assert np.array_equal(p > 0, u > tau)
        # bracket: p <= 1 gives tau >= max u - 1; the largest p >= 1/n gives
        # tau <= max u - n^-(alpha-1)
        assert tau >= u.max() - 1.0 - 1e-12
        assert tau <= u.max() - n ** (-(alpha - 1.0)) + 1e-12
        np.testing.assert_allclose(entmax(z + 3.7, alpha), p, atol=1e-10)
        perm = rng.permutation(n)
        np.testing.assert_allclose(entmax(z[perm], alpha), p[perm], atol=1e-12)
    np.testing.assert_allclose(entmax([0.42], alpha), [1.0], atol=1e-12)


def test_rows_masking_and_empty_rows():
    Z = np.array([[0.5, -np.inf, 0.1], [-np.inf, -np.inf, -np.inf], [2.0, 2.0, -np.inf]])
    t = entmax_threshold_rows(Z, 1.5)
    assert t[0] == pytest.approx(entmax_threshold([0.5, 0.1], 1.5), abs=1e-12)
    assert np.isinf(t[1]) and t[1] > 0
    assert t[2] == pytest.approx(entmax_threshold([2.0, 2.0], 1.5), abs=1e-12)


@pytest.mark.parametrize("alpha", [1.5, 2.0])
def test_rows_match_single_row(alpha):
    rng = np.random.default_rng(9)
    Z = rng.normal(size=(50, 40)) * 2
    Z[rng.random(Z.shape) < 0.3] = -np.inf
    t_rows = entmax_threshold_rows(Z, alpha)
    for r in range(Z.shape[0]):
        assert t_rows[r] == pytest.approx(entmax_threshold(Z[r], alpha), abs=1e-12)


def test_alpha_controls_sparsity():
    """AdaSplash README, "Adaptive Sparsity Control": alpha 2 sparser than 1.333."""
    rng = np.random.default_rng(2)
    z = rng.normal(size=200)
    nnz = [np.count_nonzero(entmax(z, a)) for a in (1.333, 1.5, 2.0)]
    assert nnz[0] > nnz[1] > nnz[2]


@pytest.mark.parametrize("alpha", ALPHAS)
def test_backward_matches_finite_differences(alpha):
    """The closed-form vector-Jacobian product against central differences of the
    exact forward (a different computation: the sort-based threshold), at points
    whose support does not change within the step."""
    rng = np.random.default_rng(17)
    checked = 0
    for _ in range(40):
        z = rng.normal(size=9) * 1.5
        y = entmax(z, alpha)
        tau = entmax_threshold(z, alpha)
        if np.min(np.abs((alpha - 1.0) * z - tau)) < 1e-3:
            continue  # too close to a support change for differences
        dy = rng.normal(size=9)
        h = 1e-6
        fd = np.array([(entmax(z + h * e, alpha) - entmax(z - h * e, alpha)) @ dy / (2 * h) for e in np.eye(9)])
        np.testing.assert_allclose(entmax_backward(y, dy, alpha), fd, atol=2e-6)
        checked += 1
    assert checked >= 20


def test_backward_softmax_limit_and_invariants():
    rng = np.random.default_rng(19)
    z = rng.normal(size=24)
    dy = rng.normal(size=24)
    # alpha -> 1: the softmax Jacobian diag(p) - p p^T
    sm = np.exp(z - z.max())
    sm /= sm.sum()
    vjp_sm = sm * dy - sm * float(sm @ dy)
    errs = [np.abs(entmax_backward(entmax(z, a), dy, a) - vjp_sm).max() for a in (1.1, 1.01, 1.001)]
    assert errs[0] > errs[1] > errs[2] and errs[2] < 5e-3
    for alpha in ALPHAS:
        y = entmax(z, alpha)
        dz = entmax_backward(y, dy, alpha)
        assert abs(dz.sum()) < 1e-12  # shifting z leaves y unchanged
        assert np.all(dz[y == 0] == 0)  # off the support nothing moves
        assert np.allclose(entmax_backward(y, np.full(24, 0.7), alpha), 0.0, atol=1e-12)
    assert np.all(entmax_backward(np.zeros(5), rng.normal(size=5), 1.5) == 0)

