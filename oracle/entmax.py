"""Exact alpha-entmax thresholds in float64 (CPU oracle; test infrastructure only).

The AdaSplash README ("Usage", "Triton Entmax (Optimized Entmax Activation)")
names a row-wise entmax with an ``alpha`` argument (default 1.5) and says its
threshold is found iteratively (Halley's method plus bisection); the section
"Adaptive Sparsity Control" says alpha = 2 is sparser and alpha = 1.333 denser.
The mapping itself is not written on the page. The oracle uses the published
definition (Peters, Niculae & Martins, ACL 2019):

    u   = (alpha - 1) * z
    p_i = max(u_i - tau, 0) ** (1 / (alpha - 1))

with tau the unique value for which the p_i sum to one. The result is unique, so
the oracle computes it exactly (up to float64 rounding) instead of iterating:

1. sort u in decreasing order, s_1 >= s_2 >= ... >= s_n;
2. the support size k* is the number of k with g(s_k) < 1, where
   g(tau) = sum_j max(s_j - tau, 0) ** beta is decreasing in tau, so
   tau < s_k  <=>  g(s_k) < 1;
3. on that support, solve sum_{j<=k*} (s_j - tau) ** beta = 1 for
   tau in [s_{k*+1}, s_{k*}):
     * alpha = 2 (sparsemax, Martins & Astudillo 2016):  tau = (sum s_j - 1) / k*
     * alpha = 1.5 (beta = 2): the smaller root of the quadratic
       k tau^2 - 2 tau S1 + S2 - 1 = 0, i.e. tau = M - sqrt(M^2 - S2/k + 1/k)
     * any other alpha > 1: float64 bisection (the function is monotone).

Candidates equal to -inf are "not a candidate"; a row with no candidate gets
tau = +inf.
"""

from __future__ import annotations

import itertools

import numpy as np

__all__ = [
    "entmax_threshold",
    "entmax_threshold_rows",
    "entmax",
    "entmax_backward",
    "entmax_threshold_bruteforce",
]

_BISECT_STEPS = 200


def _power(x: np.ndarray, beta: float) -> np.ndarray:
    """max(x, 0) ** beta, evaluated in the log domain for large beta (alpha -> 1)."""
    x = np.asarray(x, dtype=np.float64)
    out = np.zeros_like(x)
    pos = x > 0
    if beta == 1.0:
        out[pos] = x[pos]
    elif beta == 2.0:
        out[pos] = x[pos] * x[pos]
    else:
        out[pos] = np.exp(beta * np.log(x[pos]))
    return out


def _solve_on_support(top: np.ndarray, alpha: float, lo: float, hi: float) -> float:
    """tau with sum_j (top_j - tau) ** beta = 1, tau in [lo, hi]; top sorted desc."""
    k = top.size
    if alpha == 2.0:
        return (float(np.sum(top)) - 1.0) / k
    if alpha == 1.5:
        mean = float(np.mean(top))
        mean_sq = float(np.mean(top * top))
        disc = mean * mean - mean_sq + 1.0 / k
        return mean - np.sqrt(max(disc, 0.0))
    beta = 1.0 / (alpha - 1.0)
    for _ in range(_BISECT_STEPS):
        mid = 0.5 * (lo + hi)
        if float(np.sum(_power(top - mid, beta))) >= 1.0:
            lo = mid
        else:
            hi = mid
    return 0.5 * (lo + hi)


def entmax_threshold(z, alpha: float) -> float:
    """Exact tau (in u = (alpha-1) z units) for one row of scores ``z``.

    Entries equal to -inf are not candidates. Returns +inf if there is none.
    """
    if not alpha > 1.0:
        raise ValueError("alpha must be > 1")
    z = np.asarray(z, dtype=np.float64).ravel()
    cand = z[np.isfinite(z)]
    if cand.size == 0:
        return float("inf")
    beta = 1.0 / (alpha - 1.0)
    s = np.sort((alpha - 1.0) * cand)[::-1]
    # Only entries above max(u) - 1 can be in the support: p <= 1 forces
    # tau >= max(u) - 1. Dropping the rest changes nothing (exact pruning).
    s = s[s > s[0] - 1.0]
    # g(s_k) = sum_{j<k} (s_j - s_k) ** beta; tau < s_k  <=>  g(s_k) < 1
    g = np.array([float(np.sum(_power(s[:k] - s[k], beta))) for k in range(s.size)])
    kstar = int(np.count_nonzero(g < 1.0))
    top = s[:kstar]
    hi = float(s[kstar - 1])
    lo = float(s[kstar]) if kstar < s.size else float(s[0]) - 1.0
    lo = max(lo, float(s[0]) - 1.0)
    return float(_solve_on_support(top, alpha, lo, hi))


def entmax_threshold_rows(Z, alpha: float) -> np.ndarray:
    """Row-wise exact tau for a 2-D array of scores (-inf = not a candidate).

    Same mathematics as :func:`entmax_threshold`, vectorised over rows for the
    closed-form cases alpha = 1.5 and alpha = 2; other alpha values are handled
    row by row.
    """
    if not alpha > 1.0:
        raise ValueError("alpha must be > 1")
    Z = np.asarray(Z, dtype=np.float64)
    if Z.ndim != 2:
        raise ValueError("Z must be 2-D")
    rows, n = Z.shape
    tau = np.full(rows, np.inf)
    if n == 0 or rows == 0:
        return tau
    if alpha not in (1.5, 2.0):
        for r in range(rows):
            tau[r] = entmax_threshold(Z[r], alpha)
        return tau
    U = (alpha - 1.0) * Z
    rowmax = np.max(U, axis=1)
    has = np.isfinite(rowmax)
    if not np.any(has):
        return tau
    U = U[has]
    mx = rowmax[has][:, None]
    # exact pruning: entries at or below max - 1 are never in the support
    U = np.where(U > mx - 1.0, U, -np.inf)
    s = -np.sort(-U, axis=1)  # descending, -inf last
    valid = np.isfinite(s)
    s0 = np.where(valid, s, 0.0)
    k = np.arange(1, n + 1, dtype=np.float64)[None, :]
    c1 = np.cumsum(s0, axis=1)
    if alpha == 2.0:
        # g(s_k) = sum_{j<k} (s_j - s_k) = c1_{k-1} - (k-1) s_k
        g = (c1 - s0) - (k - 1.0) * s0
    else:
        c2 = np.cumsum(s0 * s0, axis=1)
        # g(s_k) = sum_{j<k} (s_j - s_k)^2
        g = (c2 - s0 * s0) - 2.0 * s0 * (c1 - s0) + (k - 1.0) * s0 * s0
    kstar = np.count_nonzero((g < 1.0) & valid, axis=1)  # >= 1 for rows with a candidate
    idx = kstar - 1
    r = np.arange(U.shape[0])
    S1 = c1[r, idx]
    kk = kstar.astype(np.float64)
    if alpha == 2.0:
        t = (S1 - 1.0) / kk
    else:
        S2 = np.cumsum(s0 * s0, axis=1)[r, idx]
        mean = S1 / kk
        disc = mean * mean - S2 / kk + 1.0 / kk
        t = mean - np.sqrt(np.maximum(disc, 0.0))
    tau[has] = t
    return tau


def entmax(z, alpha: float) -> np.ndarray:
    """alpha-entmax probabilities of a 1-D score vector (-inf entries get 0)."""
    z = np.asarray(z, dtype=np.float64).ravel()
    tau = entmax_threshold(z, alpha)
    if not np.isfinite(tau):
        return np.zeros_like(z)
    u = np.where(np.isfinite(z), (alpha - 1.0) * z, -np.inf)
    return _power(u - tau, 1.0 / (alpha - 1.0))


def entmax_backward(y, dy, alpha: float) -> np.ndarray:
    """Vector-Jacobian product of alpha-entmax at its output ``y`` (1-D) for the
    cotangent ``dy``: the gradient with respect to the scores z.

    The AdaSplash README ("Usage", AdaSplash with Block Masking) runs its kernels
    forward and backward; the Jacobian itself is the published one (Peters,
    Niculae & Martins 2019): differentiating sum_i (u_i - tau)^beta = 1 with
    u = (alpha - 1) z gives, with g_i = y_i^(2 - alpha) on the support and 0 off
    it,
        d y / d z = diag(g) - g g^T / sum(g),
    a symmetric matrix, so dz = g * dy - g * (g . dy) / sum(g). A row without a
    support (no finite score) gets dz = 0.
    """
    y = np.asarray(y, dtype=np.float64).ravel()
    dy = np.asarray(dy, dtype=np.float64).ravel()
    if y.shape != dy.shape:
        raise ValueError("y and dy must have the same length")
    g = np.where(y > 0.0, _power(y, 2.0 - alpha), 0.0)
    sg = float(np.sum(g))
    if sg <= 0.0:
        return np.zeros_like(y)
    return g * dy - g * (float(np.dot(g, dy)) / sg)


def entmax_threshold_bruteforce(z, alpha: float) -> float:
    """tau by enumerating every candidate support (for tiny n only).

    For each non-empty subset S, solve sum_{i in S} (u_i - tau) ** beta = 1 with
    tau below min_S u (bisection in float64), then keep the subset that satisfies
    the optimality conditions: u_i > tau inside S and u_j <= tau outside S.
    Exactly one subset does (ties aside), which is what makes entmax well defined.
    """
    z = np.asarray(z, dtype=np.float64).ravel()
    n = z.size
    if n > 12:
        raise ValueError("brute force is for n <= 12")
    u = (alpha - 1.0) * z
    beta = 1.0 / (alpha - 1.0)
    found = []
    for size in range(1, n + 1):
        for subset in itertools.combinations(range(n), size):
            us = u[list(subset)]
            lo, hi = float(np.max(us)) - 1.0, float(np.min(us))
            if float(np.sum(_power(us - hi, beta))) > 1.0:
                continue  # no root below min_S u
            for _ in range(_BISECT_STEPS):
                mid = 0.5 * (lo + hi)
                if float(np.sum(_power(us - mid, beta))) >= 1.0:
                    lo = mid
                else:
                    hi = mid
            tau = 0.5 * (lo + hi)
            inside = np.all(us > tau - 1e-12)
            rest = np.delete(u, list(subset))
            outside = np.all(rest <= tau + 1e-12)
            if inside and outside:
                found.append(tau)
    if not found:
        raise RuntimeError("no self-consistent support found")
    return float(found[0])
