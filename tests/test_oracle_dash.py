"""Pins of the DashAttention oracle against results it does not compute itself.

* head_cls = 0 turns the summary into the plain mean of the chunk's keys; a
  chunk of identical keys summarises to that key;
* scaling_factor = 0 makes every routing score equal, so the prior is uniform
  over the candidates and the attention equals dense softmax attention
  (torch's scaled_dot_product_attention, float64 on the CPU), causal or not;
* one chunk covering the whole sequence leaves a single candidate: dense causal;
* without estimate_diagonal, rows of the first chunk attend only their own
  chunk with weight 1: dense causal attention over that chunk;
* chunk-constant keys and values reduce the token softmax to a closed-form
  mixture over chunks, weighted by (tokens seen) * prior * exp(score);
* GQA equals MHA over repeated KV heads; decode of token t equals prefill row t.
"""

import numpy as np
import pytest
import torch

from oracle import entmax
from oracle.dash import DashParams, chunk_summary, chunk_summaries, dash_decode, dash_prefill, route_row


def _sdpa(Q, K, V, causal):
    q, k, v = (torch.from_numpy(np.ascontiguousarray(x)).to(torch.float64) for x in (Q, K, V))
    return torch.nn.functional.scaled_dot_product_attention(q, k, v, is_causal=causal).numpy()


def _rand(shape, seed):
    return np.random.default_rng(seed).normal(size=shape)


def test_summary_zero_cls_is_mean():
    keys = _rand((64, 16), 0)
    np.testing.assert_allclose(chunk_summary(keys, np.zeros(16)), keys.mean(axis=0), atol=1e-14)


def test_summary_identical_keys():
    key = _rand(16, 1)
    np.testing.assert_allclose(chunk_summary(np.tile(key, (64, 1)), _rand(16, 2)), key, atol=1e-14)


def test_summary_picks_dominant_key():
    keys = _rand((8, 16), 3)
    cls = keys[5] * 50.0  # softmax weight concentrates on the key most aligned with cls
    np.testing.assert_allclose(chunk_summary(keys, cls), keys[5], atol=1e-6)


def test_partial_tail_summary():
    keys = _rand((100, 8), 4)
    cls = _rand(8, 5)
    s = chunk_summaries(keys, cls, 32, 100)
    assert s.shape == (4, 8)
    np.testing.assert_allclose(s[3], chunk_summary(keys[96:100], cls), atol=1e-14)


@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("N,C", [(96, 16), (100, 16), (64, 64)])
def test_zero_scaling_is_dense_attention(causal, N, C):
    B, Hq, Hkv, d = 1, 2, 1, 16
    Q, K, V = _rand((B, Hq, N, d), 10), _rand((B, Hkv, N, d), 11), _rand((B, Hkv, N, d), 12)
    cls = _rand((Hkv, d), 13)
    p = DashParams(chunk_size=C, alpha=1.5, scaling_factor=0.0, causal=causal, estimate_diagonal=True)
    O, tau, bits = dash_prefill(Q, K, V, cls, p)
    ref = _sdpa(Q, np.repeat(K, Hq, axis=1), np.repeat(V, Hq, axis=1), causal)
    np.testing.assert_allclose(O, ref, atol=1e-12)
    # uniform prior: every candidate routed
    n_c = -(-N // C)
    for i in (0, N // 2, N - 1):
        active = [c for c in range(n_c) if bits[0, 0, i, c // 32] >> (c % 32) & 1]
        want = list(range(i // C + 1)) if causal else list(range(n_c))
        assert active == want


def test_single_chunk_is_dense_causal():
    B, Hq, Hkv, N, d = 1, 1, 1, 48, 8
    Q, K, V = _rand((B, Hq, N, d), 20), _rand((B, Hkv, N, d), 21), _rand((B, Hkv, N, d), 22)
    p = DashParams(chunk_size=64, alpha=1.5, scaling_factor=1.0, causal=True, estimate_diagonal=True)
    O, tau, _ = dash_prefill(Q, K, V, _rand((Hkv, d), 23), p)
    np.testing.assert_allclose(O, _sdpa(Q, K, V, True), atol=1e-12)
    # a single candidate has p = 1, so tau = u - 1
    np.testing.assert_array_less(np.abs(tau[0, 0] - (0.5 * _diag_scores(Q, K, p) - 1.0)), 1e-12)


def _diag_scores(Q, K, p):
    cls = _rand((1, Q.shape[-1]), 23)[0]
    out = []
    for i in range(Q.shape[2]):
        s = chunk_summary(K[0, 0, : i + 1], cls)
        out.append(Q[0, 0, i] @ s / np.sqrt(Q.shape[-1]))
    return np.array(out)


def test_first_chunk_without_estimate_is_local_causal():
    B, Hq, Hkv, N, d, C = 1, 1, 1, 64, 8, 16
    Q, K, V = _rand((B, Hq, N, d), 30), _rand((B, Hkv, N, d), 31), _rand((B, Hkv, N, d), 32)
    p = DashParams(chunk_size=C, alpha=1.5, causal=True, estimate_diagonal=False)
    O, tau, bits = dash_prefill(Q, K, V, _rand((Hkv, d), 33), p)
    ref = _sdpa(Q[:, :, :C], K[:, :, :C], V[:, :, :C], True)
    np.testing.assert_allclose(O[:, :, :C], ref, atol=1e-12)
    assert np.all(np.isinf(tau[0, 0, :C]))
    assert np.all(bits[0, 0, :C, 0] == 1)
    # later rows always have their own chunk active
    for i in range(C, N):
        assert bits[0, 0, i, 0] >> (i // C) & 1


@pytest.mark.parametrize("causal,est", [(True, True), (True, False), (False, True)])
def test_chunk_constant_mixture(causal, est):
    """Keys and values constant per chunk: the token softmax collapses to a chunk mixture.

    With k_j = kc[c(j)] and v_j = vc[c(j)], every summary is kc[c] and the output
    of row i is sum_c n_c w_c exp(z_c) vc[c] / sum_c n_c w_c exp(z_c), where n_c
    is the number of visible tokens of chunk c and z_c = <q_i, kc[c]>/sqrt(d).
    """
    C, n_chunks, d, alpha = 8, 6, 4, 1.5
    N = C * n_chunks - 3  # ragged tail
    rng = np.random.default_rng(40)
    kc = rng.normal(size=(n_chunks, d)) * 1.5
    vc = rng.normal(size=(n_chunks, d))
    K = kc[np.arange(N) // C][None, None]
    V = vc[np.arange(N) // C][None, None]
    Q = rng.normal(size=(1, 1, N, d)) * 2.0
    cls = rng.normal(size=(1, d))
    p = DashParams(chunk_size=C, alpha=alpha, scaling_factor=1.0, causal=causal, estimate_diagonal=est)
    O, tau, _ = dash_prefill(Q, K, V, cls, p)
    for i in range(N):
        q = Q[0, 0, i]
        ci = i // C
        if causal:
            cands = list(range(ci + (1 if est else 0)))
        else:
            cands = list(range(n_chunks))
        z = np.array([q @ kc[c] / np.sqrt(d) for c in cands])
        w = {c: 0.0 for c in range(n_chunks)}
        if cands:
            for c, pc in zip(cands, entmax(z, alpha)):
                w[c] = pc
        if causal and not est:
            w[ci] = 1.0
        num = np.zeros(d)
        den = 0.0
        for c in range(n_chunks):
            if w[c] <= 0:
                continue
            lo, hi = c * C, min(N, (c + 1) * C)
            if causal:
                hi = min(hi, i + 1)
            n_vis = max(0, hi - lo)
            e = n_vis * w[c] * np.exp(q @ kc[c] / np.sqrt(d))
            num += e * vc[c]
            den += e
        np.testing.assert_allclose(O[0, 0, i], num / den, atol=1e-12)


def test_gqa_equals_repeated_mha():
    B, Hq, Hkv, N, d, C = 2, 4, 2, 40, 8, 8
    Q, K, V = _rand((B, Hq, N, d), 50), _rand((B, Hkv, N, d), 51), _rand((B, Hkv, N, d), 52)
    cls = _rand((Hkv, d), 53)
    p = DashParams(chunk_size=C)
    O1, t1, b1 = dash_prefill(Q, K, V, cls, p)
    O2, t2, b2 = dash_prefill(Q, np.repeat(K, 2, axis=1), np.repeat(V, 2, axis=1), np.repeat(cls, 2, axis=0), p)
    np.testing.assert_allclose(O1, O2, atol=1e-14)
    np.testing.assert_allclose(t1, t2, atol=1e-14)
    assert np.array_equal(b1, b2)


@pytest.mark.parametrize("est", [True, False])
def test_decode_equals_prefill_row(est):
    B, Hq, Hkv, d, C = 2, 4, 2, 8, 8
    Lmax = 50
    Q, K, V = _rand((B, Hq, Lmax, d), 60), _rand((B, Hkv, Lmax, d), 61), _rand((B, Hkv, Lmax, d), 62)
    cls = _rand((Hkv, d), 63)
    p = DashParams(chunk_size=C, estimate_diagonal=est)
    seqlens = np.array([33, 48])  # positions 32 (chunk start) and 47 (chunk end)
    q = np.stack([Q[b, :, seqlens[b] - 1] for b in range(B)])
    O, tau, bits = dash_decode(q, K, V, cls, seqlens, p)
    for b in range(B):
        n = seqlens[b]
        Op, tp, bp = dash_prefill(Q[b : b + 1, :, :n], K[b : b + 1, :, :n], V[b : b + 1, :, :n], cls, p)
        np.testing.assert_allclose(O[b], Op[0, :, n - 1], atol=1e-14)
        np.testing.assert_allclose(tau[b], tp[0, :, n - 1], atol=1e-14)
        for h in range(Hq):
            assert np.array_equal(bits[b][h], bp[0, h, n - 1])


def test_route_prior_is_entmax_of_scores():
    rng = np.random.default_rng(70)
    d, C, N = 8, 4, 40
    K = rng.normal(size=(N, d))
    cls = rng.normal(size=d)
    q = rng.normal(size=(1, d))
    p = DashParams(chunk_size=C, alpha=1.5, scaling_factor=2.0)
    Z, tau, prior, logw = route_row(q, np.array([N - 1]), K, cls, N, p)
    summ = chunk_summaries(K, cls, C, N)
    z = [2.0 * q[0] @ summ[c] / np.sqrt(d) for c in range(N // C - 1)]
    z.append(2.0 * q[0] @ chunk_summary(K[(N - 1) // C * C : N], cls) / np.sqrt(d))
    np.testing.assert_allclose(prior[0], entmax(np.array(z), 1.5), atol=1e-12)
    assert prior[0].sum() == pytest.approx(1.0, abs=1e-12)


# ---- summary backward (gradients of <s, ds> with respect to the keys and head_cls)

from oracle.dash import chunk_summary_backward  # noqa: E402


@pytest.mark.parametrize("n,d,scale", [(7, 4, 1.0), (12, 6, 3.0), (1, 5, 1.0)])
def test_summary_backward_matches_finite_differences(n, d, scale):
    rng = np.random.default_rng(60 + n)
    k, cls, ds = rng.normal(size=(n, d)), rng.normal(size=d) * scale, rng.normal(size=d)
    dk, dcls = chunk_summary_backward(k, cls, ds)
    eps = 1e-6
    fk = np.zeros_like(k)
    for idx in np.ndindex(*k.shape):
        kp, km = k.copy(), k.copy()
        kp[idx] += eps
        km[idx] -= eps
        fk[idx] = (chunk_summary(kp, cls) - chunk_summary(km, cls)) @ ds / (2 * eps)
    fc = np.zeros_like(cls)
    for i in range(d):
        cp, cm = cls.copy(), cls.copy()
        cp[i] += eps
        cm[i] -= eps
        fc[i] = (chunk_summary(k, cp) - chunk_summary(k, cm)) @ ds / (2 * eps)
    np.testing.assert_allclose(dk, fk, atol=1e-7)
    np.testing.assert_allclose(dcls, fc, atol=1e-7)


def test_summary_backward_zero_cls_is_covariance():
    """head_cls = 0 gives mean pooling: dk_j = ds / n, and dcls is the (biased)
    covariance of the keys applied to ds, over sqrt(d)."""
    rng = np.random.default_rng(70)
    n, d = 9, 5
    k, ds = rng.normal(size=(n, d)), rng.normal(size=d)
    dk, dcls = chunk_summary_backward(k, np.zeros(d), ds)
    np.testing.assert_allclose(dk, np.tile(ds / n, (n, 1)), atol=1e-14)
    kc = k - k.mean(axis=0)
    np.testing.assert_allclose(dcls, (kc.T @ kc / n) @ ds / np.sqrt(d), atol=1e-13)


def test_summary_backward_identical_keys():
    """Identical keys: the weights cannot move the summary, so dcls = 0 and each
    key takes its weight's share of ds."""
    rng = np.random.default_rng(71)
    d = 6
    v = rng.normal(size=d)
    k = np.tile(v, (5, 1))
    ds = rng.normal(size=d) + 1.0
    dk, dcls = chunk_summary_backward(k, rng.normal(size=d), ds)
    np.testing.assert_allclose(dcls, 0.0, atol=1e-13)
    np.testing.assert_allclose(dk, np.tile(ds / 5, (5, 1)), atol=1e-14)
