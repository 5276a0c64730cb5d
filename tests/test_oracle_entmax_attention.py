"""Pins of the dense alpha-entmax attention oracle.

* alpha = 2: each row's weights are the Euclidean projection of the scores onto
  the simplex (solved here by a generic constrained optimiser);
* causal row 0 sees one key: output v_0 and tau = (alpha - 1) s_00 - 1;
* alpha -> 1 approaches softmax attention (torch SDPA, float64, CPU);
* varlen: a sequence alone equals the same sequence inside a padded batch, and
  padded rows are zero with tau = 0;
* the block mask equals "any non-zero weight" per 64 x 64 tile, recomputed here
  by reshaping the weight matrix into tiles.
"""

import numpy as np
import pytest
import torch
from scipy.optimize import minimize

from oracle.entmax_attention import entmax_attention, entmax_attention_rows


def _rand(shape, seed, scale=1.0):
    return np.random.default_rng(seed).normal(size=shape) * scale


def test_sparsemax_rows_are_simplex_projections():
    N, d = 12, 8
    Q, K, V = _rand((1, 1, N, d), 1), _rand((1, 1, N, d), 2), _rand((1, 1, N, d), 3)
    O, tau, _ = entmax_attention(Q, K, V, alpha=2.0, causal=False)
    S = Q[0, 0] @ K[0, 0].T / np.sqrt(d)
    for i in range(N):
        res = minimize(
            lambda p: np.sum((p - S[i]) ** 2),
            np.full(N, 1.0 / N),
            method="SLSQP",
            bounds=[(0.0, None)] * N,
            constraints=[{"type": "eq", "fun": lambda p: np.sum(p) - 1.0}],
            options={"ftol": 1e-15, "maxiter": 500},
        )
        np.testing.assert_allclose(O[0, 0, i], res.x @ V[0, 0], atol=1e-5)


@pytest.mark.parametrize("alpha", [1.5, 2.0, 1.333])
def test_causal_first_row(alpha):
    N, d = 16, 8
    Q, K, V = _rand((1, 2, N, d), 4), _rand((1, 2, N, d), 5), _rand((1, 2, N, d), 6)
    O, tau, _ = entmax_attention(Q, K, V, alpha=alpha, causal=True)
    for h in range(2):
        np.testing.assert_allclose(O[0, h, 0], V[0, h, 0], atol=1e-12)
        s00 = Q[0, h, 0] @ K[0, h, 0] / np.sqrt(d)
        assert tau[0, h, 0] == pytest.approx((alpha - 1.0) * s00 - 1.0, abs=1e-12)


@pytest.mark.parametrize("causal", [True, False])
def test_softmax_limit(causal):
    N, d = 20, 8
    Q, K, V = _rand((1, 1, N, d), 7), _rand((1, 1, N, d), 8), _rand((1, 1, N, d), 9)
    ref = torch.nn.functional.scaled_dot_product_attention(
        *(torch.from_numpy(x) for x in (Q, K, V)), is_causal=causal
    ).numpy()
    errs = [np.abs(entmax_attention(Q, K, V, a, causal)[0] - ref).max() for a in (1.1, 1.01, 1.001)]
    assert errs[0] > errs[1] > errs[2]
    assert errs[2] < 5e-3 and errs[1] > 5 * errs[2]  # error shrinks like (alpha - 1)


@pytest.mark.parametrize("causal", [True, False])
def test_varlen_isolation(causal):
    B, H, N, d = 3, 2, 150, 8
    Q, K, V = _rand((B, H, N, d), 10), _rand((B, H, N, d), 11), _rand((B, H, N, d), 12)
    lens = np.array([34, 150, 77])
    O, tau, mask = entmax_attention(Q, K, V, 1.5, causal, varlen=lens)
    for b in range(B):
        L = lens[b]
        Ob, tb, mb = entmax_attention(Q[b : b + 1, :, :L], K[b : b + 1, :, :L], V[b : b + 1, :, :L], 1.5, causal)
        np.testing.assert_allclose(O[b, :, :L], Ob[0], atol=1e-13)
        np.testing.assert_allclose(tau[b, :, :L], tb[0], atol=1e-13)
        assert np.all(O[b, :, L:] == 0) and np.all(tau[b, :, L:] == 0)
        nT = -(-L // 64)
        assert np.array_equal(mask[b, :, :nT, : mb.shape[-1]], mb[0])
        assert np.all(mask[b, :, nT:] == 0)


@pytest.mark.parametrize("alpha,causal", [(2.0, False), (1.5, True)])
def test_block_mask_is_tile_any(alpha, causal):
    N, d = 200, 16
    Q, K, V = _rand((1, 1, N, d), 13, 2.0), _rand((1, 1, N, d), 14, 2.0), _rand((1, 1, N, d), 15)
    _, _, mask = entmax_attention(Q, K, V, alpha, causal)
    _, _, P = entmax_attention_rows(Q[0, 0], np.arange(N), K[0, 0], V[0, 0], N, alpha, causal)
    nT = -(-N // 64)
    Pp = np.zeros((nT * 64, nT * 64))
    Pp[:N, :N] = P
    tiles = (Pp.reshape(nT, 64, nT, 64) > 0).any(axis=(1, 3))
    for I in range(nT):
        for J in range(nT):
            assert bool(mask[0, 0, I, J // 32] >> (J % 32) & 1) == tiles[I, J]
    # alpha = 2 with scaled inputs is sparse: some tiles must be skippable
    if alpha == 2.0:
        assert not tiles.all()


def test_rows_sum_to_one_support():
    N, d = 64, 8
    Q, K = _rand((N, d), 16, 2.0), _rand((N, d), 17, 2.0)
    for alpha in (1.5, 2.0):
        _, tau, P = entmax_attention_rows(Q, np.arange(N), K, np.eye(N, d), N, alpha, False)
        np.testing.assert_allclose(P.sum(axis=1), 1.0, atol=1e-12)
        U = (alpha - 1) * (Q @ K.T) / np.sqrt(d)
        assert np.array_equal(P > 0, U > tau[:, None])


# ---- backward (gradients of sum(O * dO)) ----

from oracle.entmax_attention import entmax_attention_backward  # noqa: E402


def _fd_grads(Q, K, V, dO, alpha, causal, varlen, eps=1e-6):
    """Central differences of sum(O * dO) through the forward oracle."""
    def loss(q, k, v):
        return float(np.sum(entmax_attention(q, k, v, alpha, causal, varlen=varlen)[0] * dO))

    out = []
    for which in range(3):
        args = [Q.copy(), K.copy(), V.copy()]
        g = np.zeros_like(args[which])
        for idx in np.ndindex(*g.shape):
            a_p = [x.copy() for x in args]
            a_m = [x.copy() for x in args]
            a_p[which][idx] += eps
            a_m[which][idx] -= eps
            g[idx] = (loss(*a_p) - loss(*a_m)) / (2 * eps)
        out.append(g)
    return out


@pytest.mark.parametrize(
    "alpha,causal,varlen",
    [(1.5, True, None), (2.0, False, None), (1.25, True, None), (1.5, False, [5, 9]), (2.0, True, [9, 3])],
)
def test_backward_matches_finite_differences(alpha, causal, varlen):
    B = 1 if varlen is None else len(varlen)
    N, d = 9, 4
    Q, K, V = _rand((B, 1, N, d), 30, 1.5), _rand((B, 1, N, d), 31, 1.5), _rand((B, 1, N, d), 32)
    dO = _rand((B, 1, N, d), 33)
    lens = None if varlen is None else np.array(varlen)
    dQ, dK, dV = entmax_attention_backward(Q, K, V, dO, alpha, causal, varlen=lens)
    fQ, fK, fV = _fd_grads(Q, K, V, dO, alpha, causal, lens)
    np.testing.assert_allclose(dQ, fQ, atol=1e-6)
    np.testing.assert_allclose(dK, fK, atol=1e-6)
    np.testing.assert_allclose(dV, fV, atol=1e-6)
    # sparse weights leave some gradient entries exactly zero only off the support;
    # the check above must not pass trivially
    assert np.abs(dQ).max() > 1e-3 and np.abs(dK).max() > 1e-3


@pytest.mark.parametrize("alpha,causal", [(1.5, True), (2.0, False), (1.333, True)])
def test_backward_invariants(alpha, causal):
    """Shift invariance of entmax makes every row of dS sum to 0, so the key
    gradients of one (b, h) sum to 0; each row's weights sum to 1, so the value
    gradients sum to the sum of dO over the valid rows. Causal row 0 has a single
    key, hence a zero Jacobian and dQ_0 = 0."""
    B, H, N, d = 2, 2, 70, 8
    Q, K, V = _rand((B, H, N, d), 40, 2.0), _rand((B, H, N, d), 41, 2.0), _rand((B, H, N, d), 42)
    dO = _rand((B, H, N, d), 43)
    lens = np.array([70, 37])
    dQ, dK, dV = entmax_attention_backward(Q, K, V, dO, alpha, causal, varlen=lens)
    for b in range(B):
        L = lens[b]
        np.testing.assert_allclose(dK[b].sum(axis=1), 0.0, atol=1e-10)
        np.testing.assert_allclose(dV[b].sum(axis=1), dO[b, :, :L].sum(axis=1), atol=1e-10)
        assert np.all(dQ[b, :, L:] == 0) and np.all(dK[b, :, L:] == 0) and np.all(dV[b, :, L:] == 0)
        if causal:
            assert np.all(dQ[b, :, 0] == 0)


@pytest.mark.parametrize("causal", [True, False])
def test_backward_softmax_limit(causal):
    """alpha -> 1: the gradients approach those of softmax attention (torch autograd
    through SDPA, float64 on the CPU), with the error shrinking with alpha - 1."""
    N, d = 16, 8
    Q, K, V = _rand((1, 1, N, d), 50), _rand((1, 1, N, d), 51), _rand((1, 1, N, d), 52)
    dO = _rand((1, 1, N, d), 53)
    tq, tk, tv = (torch.from_numpy(x).requires_grad_(True) for x in (Q, K, V))
    out = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, is_causal=causal)
    out.backward(torch.from_numpy(dO))
    ref = [t.grad.numpy() for t in (tq, tk, tv)]
    errs = []
    for a in (1.1, 1.01, 1.001):
        g = entmax_attention_backward(Q, K, V, dO, a, causal)
        errs.append(max(np.abs(x - r).max() for x, r in zip(g, ref)))
    assert errs[0] > errs[1] > errs[2]
    assert errs[2] < 1e-2 and errs[1] > 5 * errs[2]
