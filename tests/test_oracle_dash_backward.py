"""Pins of the oracle's DashAttention backward (``oracle.dash_backward``), CPU only.

The backward is pinned to things other than itself:

* central differences of the forward oracle's L = sum(O * dO) (``dash_prefill``)
  for Q, K, V and head_cls, at points where no routing score lies near its
  row's threshold (the support, and with it L, is then smooth), for alpha 1.5
  and 2, causal and non-causal, with and without the own-chunk estimate;
* scaling_factor = 0: the prior is uniform over every candidate, the forward is
  dense (causal) softmax attention, and the gradients are those of
  torch.nn.functional.scaled_dot_product_attention (float64 autograd), with a
  zero head_cls gradient;
* GQA: the gradients with g query heads per KV head equal those of MHA over the
  KV heads repeated g times, summed over each group.

A sign error in the softmax or entmax Jacobian, a missing 1/sqrt(d) or
scaling_factor, a dropped summary or estimate term, or a transposed product
each fails one of them (checked by planting each in a copy of the oracle).
"""

import numpy as np
import pytest
import torch

import oracle
from oracle.dash import DashParams, dash_backward, dash_prefill, route_row, chunk_summaries


def _inputs(B, Hq, Hkv, N, d, seed, scale=1.0):
    rng = np.random.default_rng(seed)
    Q = rng.standard_normal((B, Hq, N, d)) * scale
    K = rng.standard_normal((B, Hkv, N, d)) * scale
    V = rng.standard_normal((B, Hkv, N, d))
    cls = rng.standard_normal((Hkv, d))
    dO = rng.standard_normal((B, Hq, N, d))
    return Q, K, V, cls, dO


def _loss(Q, K, V, cls, dO, p):
    O, _, _ = dash_prefill(Q, K, V, cls, p)
    return float(np.sum(O * dO))


def _margin(Q, K, cls, p):
    """Smallest |u - tau| over every routing candidate of every row."""
    B, Hq, N, d = Q.shape
    Hkv = K.shape[1]
    g = Hq // Hkv
    m = np.inf
    for b in range(B):
        for h in range(Hq):
            hk = h // g
            summ = chunk_summaries(K[b, hk], cls[hk], p.chunk_size, N)
            Z, tau, _, _ = route_row(Q[b, h], np.arange(N), K[b, hk], cls[hk], N, p, summ)
            U = (p.alpha - 1.0) * Z
            fin = np.isfinite(U) & np.isfinite(tau)[:, None]
            if fin.any():
                m = min(m, float(np.min(np.abs(U[fin] - np.broadcast_to(tau[:, None], U.shape)[fin]))))
    return m


CASES = [
    (1.5, True, True, 3),
    (1.5, True, False, 4),
    (1.5, False, True, 5),
    (2.0, True, True, 6),
    (2.0, True, False, 7),
    (2.0, False, True, 8),
]


@pytest.mark.parametrize("alpha,causal,est,seed", CASES)
def test_backward_matches_central_differences(alpha, causal, est, seed):
    p = DashParams(chunk_size=8, alpha=alpha, scaling_factor=1.5, causal=causal, estimate_diagonal=est)
    Q, K, V, cls, dO = _inputs(1, 2, 1, 37, 8, seed, scale=1.5)
    assert _margin(Q, K, cls, p) > 5e-5, "a routing score lies too close to its threshold for finite differences"
    grads = dash_backward(Q, K, V, cls, dO, p)
    rng = np.random.default_rng(seed + 100)
    eps = 1e-6
    for name, x, gx in zip("QKVc", (Q, K, V, cls), grads):
        flat = x.reshape(-1)
        for idx in rng.choice(flat.size, size=min(12, flat.size), replace=False):
            old = flat[idx]
            flat[idx] = old + eps
            lp = _loss(Q, K, V, cls, dO, p)
            flat[idx] = old - eps
            lm = _loss(Q, K, V, cls, dO, p)
            flat[idx] = old
            fd = (lp - lm) / (2 * eps)
            an = gx.reshape(-1)[idx]
            assert abs(fd - an) <= 1e-5 * max(1.0, abs(fd)), f"d{name}[{idx}]: analytic {an:.8f} vs central {fd:.8f}"


@pytest.mark.parametrize("causal,est", [(True, True), (True, False), (False, True)])
def test_zero_scaling_gradients_are_sdpa_gradients(causal, est):
    p = DashParams(chunk_size=8, alpha=1.5, scaling_factor=0.0, causal=causal, estimate_diagonal=est)
    Q, K, V, cls, dO = _inputs(1, 2, 2, 40, 8, 11)
    dQ, dK, dV, dcls = dash_backward(Q, K, V, cls, dO, p)
    if causal and not est:
        # the own chunk keeps weight 1 while every past chunk gets 1/n: not dense; skip the SDPA identity
        pytest.skip("estimate_diagonal off gives the own chunk weight 1, not the uniform prior")
    q, k, v = (torch.tensor(x, requires_grad=True) for x in (Q, K, V))
    o = torch.nn.functional.scaled_dot_product_attention(q, k, v, is_causal=causal)
    o.backward(torch.tensor(dO))
    np.testing.assert_allclose(dQ, q.grad.numpy(), atol=1e-10, rtol=1e-9)
    np.testing.assert_allclose(dK, k.grad.numpy(), atol=1e-10, rtol=1e-9)
    np.testing.assert_allclose(dV, v.grad.numpy(), atol=1e-10, rtol=1e-9)
    assert np.all(dcls == 0.0)


def test_gqa_gradients_are_summed_mha_gradients():
    p = DashParams(chunk_size=8, alpha=1.5, scaling_factor=1.0, causal=True, estimate_diagonal=True)
    Q, K, V, cls, dO = _inputs(1, 4, 2, 30, 8, 21)
    gq = dash_backward(Q, K, V, cls, dO, p)
    Kr, Vr, clsr = np.repeat(K, 2, axis=1), np.repeat(V, 2, axis=1), np.repeat(cls, 2, axis=0)
    mq = dash_backward(Q, Kr, Vr, clsr, dO, p)
    np.testing.assert_allclose(gq[0], mq[0], atol=1e-12)
    np.testing.assert_allclose(gq[1], mq[1].reshape(1, 2, 2, 30, 8).sum(axis=2), atol=1e-12)
    np.testing.assert_allclose(gq[2], mq[2].reshape(1, 2, 2, 30, 8).sum(axis=2), atol=1e-12)
    np.testing.assert_allclose(gq[3], mq[3].reshape(2, 2, 8).sum(axis=1), atol=1e-12)
