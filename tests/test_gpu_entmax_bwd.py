"""GPU parity of the dense alpha-entmax attention backward (entmax_attn_backward)
against the float64 CPU oracle (chain rule through the entmax Jacobian), through
the C ABI: float32 gradients within 1e-4, bfloat16 within 2e-2 + 2^-8 |ref|
(the gradients are rounded to bfloat16 once, a relative error up to 2^-9);
varlen, causal and non-causal, head_dim 64/128, the three power
specialisations (alpha 1.5, 2, other), with and without the forward's block
mask, torch autograd, and the full varlen workload through sampled dQ rows and
two identities that hold at any size.

At alpha = 2 the Jacobian weight g is 1 on the support and 0 off it, so an entry
whose u - tau is within rounding of 0 may be in the support on one side and not
on the other, changing its row's gradient by O(1); the small cases assert that
no entry is within 1e-5 of tau, and the sampled rows of the full workload skip
such rows (continuous g at alpha 1.5 and 1.333 needs no such rule).
"""

import numpy as np
import pytest
import torch

import oracle
from adaptive_sparse_long_amd import api
from adaptive_sparse_long_amd.workloads import WORKLOADS, cotangent, dense_entmax_inputs

from _helpers import TOL_BF16, TOL_F32, f64

pytestmark = pytest.mark.gpu

NEAR = 1e-5


def _tol(dtype, ref):
    return TOL_F32 if dtype == torch.float32 else TOL_BF16 + 2.0 ** -8 * np.abs(ref)


def _close(gpu, ref, dtype, where):
    err = np.abs(gpu - ref)
    bad = err > _tol(dtype, ref)
    assert np.all(np.isfinite(gpu)), f"{where}: non-finite"
    assert not bad.any(), f"{where}: {int(bad.sum())} entries off, max err {err.max():.3e} at {np.unravel_index(np.argmax(err), err.shape)}"


def _near_tau(q, k, L, alpha, causal):
    """Oracle's u - tau for rows [0, L) of one (b, h), -inf where not allowed."""
    d = q.shape[1]
    s = q[:L] @ k[:L].T / np.sqrt(d)
    if causal:
        s = np.where(np.arange(L)[None, :] <= np.arange(L)[:, None], s, -np.inf)
    _, tau, _ = oracle.entmax_attention_rows(q[:L], np.arange(L), k, np.zeros_like(k), L, alpha, causal)
    return (alpha - 1.0) * s - tau[:, None]


def check_backward(Q, K, V, dO, alpha, causal, varlen=None, where=""):
    O, tau, mask = api.entmax_attn(Q, K, V, alpha=alpha, causal=causal, varlen=varlen)
    dQ, dK, dV = api.entmax_attn_backward(Q, K, V, dO, tau, mask, alpha=alpha, causal=causal, varlen=varlen)
    torch.cuda.synchronize()
    B, H, N, d = Q.shape
    lens = varlen.cpu().numpy() if varlen is not None else None
    if alpha == 2.0:
        for b in range(B):
            L = N if lens is None else int(lens[b])
            for h in range(H):
                t = _near_tau(f64(Q[b, h]), f64(K[b, h]), L, alpha, causal)
                assert not (np.abs(t) < NEAR).any(), f"{where}: ill-conditioned case (entry within {NEAR} of tau)"
    rQ, rK, rV = oracle.entmax_attention_backward(f64(Q), f64(K), f64(V), f64(dO), alpha, causal, varlen=lens)
    _close(f64(dQ), rQ, Q.dtype, where + " dQ")
    _close(f64(dK), rK, Q.dtype, where + " dK")
    _close(f64(dV), rV, Q.dtype, where + " dV")
    return dQ, dK, dV, tau, mask


def test_backward_dense_entmax_128_f32():
    w = WORKLOADS["dense_entmax_128"]
    q, k, v, _ = dense_entmax_inputs(w.B, w.Hq, w.N, w.d, w.seed, dtype="f32", device="cuda")
    dO = cotangent(q.shape, w.seed + 500, dtype="f32", device="cuda")
    check_backward(q, k, v, dO, w.alpha, w.causal, where="f32 128")


@pytest.mark.parametrize(
    "B,H,N,d,alpha,causal,lens,scale,dtype",
    [
        (2, 2, 300, 64, 2.0, False, [300, 170], 2.0, "bf16"),
        (1, 2, 200, 128, 1.5, True, None, 1.0, "bf16"),
        (2, 1, 160, 64, 1.333, True, [160, 33], 1.0, "bf16"),
        (1, 1, 230, 128, 2.0, True, None, 1.0, "bf16"),
        (2, 2, 190, 128, 2.0, False, [190, 1], 1.0, "f32"),
        (1, 1, 256, 64, 1.333, False, None, 1.0, "f32"),
    ],
)
def test_backward_small(B, H, N, d, alpha, causal, lens, scale, dtype):
    q, k, v, _ = dense_entmax_inputs(B, H, N, d, 900 + N, dtype=dtype, scale=scale, device="cuda")
    dO = cotangent(q.shape, 1900 + N, dtype=dtype, device="cuda")
    varlen = torch.tensor(lens, dtype=torch.int32, device="cuda") if lens else None
    check_backward(q, k, v, dO, alpha, causal, varlen, where=f"{dtype} N{N} d{d} a{alpha} causal={causal}")


@pytest.mark.parametrize("dtype,alpha", [("bf16", 2.0), ("f32", 1.5)])
def test_backward_mask_skipping_is_exact(dtype, alpha):
    """Skipping the tiles the forward's mask clears gives bit-identical gradients
    to visiting every tile (block_mask NULL), and a repeat call is bit-identical."""
    q, k, v, _ = dense_entmax_inputs(2, 2, 333, 64, 17, dtype=dtype, scale=2.0, device="cuda")
    dO = cotangent(q.shape, 18, dtype=dtype, device="cuda")
    varlen = torch.tensor([333, 150], dtype=torch.int32, device="cuda")
    _, tau, mask = api.entmax_attn(q, k, v, alpha=alpha, causal=False, varlen=varlen)
    a = api.entmax_attn_backward(q, k, v, dO, tau, mask, alpha=alpha, causal=False, varlen=varlen)
    b = api.entmax_attn_backward(q, k, v, dO, tau, None, alpha=alpha, causal=False, varlen=varlen)
    c = api.entmax_attn_backward(q, k, v, dO, tau, mask, alpha=alpha, causal=False, varlen=varlen)
    torch.cuda.synchronize()
    assert all(torch.equal(x, y) for x, y in zip(a, b))
    assert all(torch.equal(x, y) for x, y in zip(a, c))
    assert not bool((mask != 0).all()), "the case should leave some tiles empty"


def test_backward_autograd():
    """torch autograd through api.entmax_attn_fn runs the same backward."""
    q, k, v, _ = dense_entmax_inputs(1, 2, 150, 64, 23, dtype="bf16", device="cuda")
    dO = cotangent(q.shape, 24, dtype="bf16", device="cuda")
    qs, ks, vs = (t.clone().requires_grad_(True) for t in (q, k, v))
    out = api.entmax_attn_fn(qs, ks, vs, alpha=1.5, causal=True)
    out.backward(dO)
    _, tau, mask = api.entmax_attn(q, k, v, alpha=1.5, causal=True)
    ref = api.entmax_attn_backward(q, k, v, dO, tau, mask, alpha=1.5, causal=True)
    torch.cuda.synchronize()
    for t, r in zip((qs, ks, vs), ref):
        assert torch.equal(t.grad, r)


def test_backward_varlen_workload():
    """The full varlen workload (8 x 16 heads, lengths in [512, 8192], d 64,
    bf16, alpha 2, non-causal): sampled dQ rows against the oracle row by row,
    and per (b, h) sum_j dK_j = 0 (shift invariance of entmax) and
    sum_j dV_j = sum_i dO_i (each row's weights sum to 1), each within the
    rounding of its bfloat16 terms (2^-8 of the sum of magnitudes) plus 2e-2."""
    w = WORKLOADS["varlen_entmax"]
    q, k, v, lens = dense_entmax_inputs(w.B, w.Hq, w.N, w.d, w.seed, dtype=w.dtype, scale=w.scale,
                                        varlen_range=w.varlen_range, device="cuda")
    dO = cotangent(q.shape, w.seed + 500, dtype=w.dtype, device="cuda")
    _, tau, mask = api.entmax_attn(q, k, v, alpha=w.alpha, causal=w.causal, varlen=lens)
    dQ, dK, dV = api.entmax_attn_backward(q, k, v, dO, tau, mask, alpha=w.alpha, causal=w.causal, varlen=lens)
    torch.cuda.synchronize()
    lens_ = lens.cpu().numpy()
    rng = np.random.default_rng(w.seed + 1)
    d = w.d
    checked = 0
    for b in range(w.B):
        L = int(lens_[b])
        for h in (0, 9):
            qb, kb, vb, ob = f64(q[b, h, :L]), f64(k[b, h, :L]), f64(v[b, h, :L]), f64(dO[b, h, :L])
            for i in np.unique(np.concatenate([[0, L - 1], rng.integers(0, L, 6)])):
                _, tr, P = oracle.entmax_attention_rows(qb[i : i + 1], np.array([i]), kb, vb, L, w.alpha, w.causal)
                s = qb[i] @ kb.T / np.sqrt(d)
                if np.any(np.abs((w.alpha - 1.0) * s - tr[0]) < NEAR):
                    continue
                ds = oracle.entmax_backward(P[0], ob[i] @ vb.T, w.alpha)
                ref = ds @ kb / np.sqrt(d)
                _close(f64(dQ[b, h, i]), ref, q.dtype, f"varlen dQ b{b} h{h} row {i}")
                checked += 1
        for h in range(w.Hq):
            gk, gv = dK[b, h, :L].double(), dV[b, h, :L].double()
            sk = gk.sum(0).abs()
            assert bool((sk <= 2.0 ** -8 * gk.abs().sum(0) + TOL_BF16).all()), f"sum dK b{b} h{h}: {float(sk.max()):.3e}"
            sv = (gv.sum(0) - dO[b, h, :L].double().sum(0)).abs()
            assert bool((sv <= 2.0 ** -8 * gv.abs().sum(0) + TOL_BF16).all()), f"sum dV b{b} h{h}: {float(sv.max()):.3e}"
            assert bool((dQ[b, h, L:] == 0).all() and (dK[b, h, L:] == 0).all() and (dV[b, h, L:] == 0).all())
    assert checked >= 100


def test_backward_maximum_length():
    """Nmax = 65536 (1024 tiles, the largest the library takes): the mask column of
    a key tile spans all 32 words of its bitmap. One head, alpha = 2, non-causal,
    length 65536 - 37 (a ragged last tile); sampled dQ rows against the oracle row
    by row (rows with an entry within 1e-5 of tau skipped) and the two identities
    per head."""
    N, d, L = 65536, 64, 65536 - 37
    q, k, v, _ = dense_entmax_inputs(1, 1, N, d, 4242, dtype="bf16", scale=2.0, device="cuda")
    dO = cotangent(q.shape, 4243, dtype="bf16", device="cuda")
    lens = torch.tensor([L], dtype=torch.int32, device="cuda")
    _, tau, mask = api.entmax_attn(q, k, v, alpha=2.0, causal=False, varlen=lens)
    dQ, dK, dV = api.entmax_attn_backward(q, k, v, dO, tau, mask, alpha=2.0, causal=False, varlen=lens)
    torch.cuda.synchronize()
    qb, kb, vb, ob = f64(q[0, 0, :L]), f64(k[0, 0, :L]), f64(v[0, 0, :L]), f64(dO[0, 0, :L])
    checked = 0
    for i in [0, 1, 4095, 40000, L - 1] + list(np.random.default_rng(5).integers(0, L, 5)):
        _, tr, P = oracle.entmax_attention_rows(qb[i : i + 1], np.array([i]), kb, vb, L, 2.0, False)
        s = qb[i] @ kb.T / np.sqrt(d)
        if np.any(np.abs(s - tr[0]) < NEAR):
            continue
        ref = oracle.entmax_backward(P[0], ob[i] @ vb.T, 2.0) @ kb / np.sqrt(d)
        _close(f64(dQ[0, 0, i]), ref, q.dtype, f"N=65536 dQ row {i}")
        checked += 1
    assert checked >= 6
    gk, gv = dK[0, 0, :L].double(), dV[0, 0, :L].double()
    assert bool((gk.sum(0).abs() <= 2.0 ** -8 * gk.abs().sum(0) + TOL_BF16).all())
    assert bool(((gv.sum(0) - dO[0, 0, :L].double().sum(0)).abs() <= 2.0 ** -8 * gv.abs().sum(0) + TOL_BF16).all())
    assert bool((dQ[0, 0, L:] == 0).all() and (dK[0, 0, L:] == 0).all() and (dV[0, 0, L:] == 0).all())


def test_backward_autograd_varlen_f32():
    """torch autograd through api.entmax_attn_fn with varlen and causal masking,
    float32, against the oracle's gradients."""
    q, k, v, _ = dense_entmax_inputs(2, 1, 140, 64, 25, dtype="f32", device="cuda")
    dO = cotangent(q.shape, 26, dtype="f32", device="cuda")
    lens = torch.tensor([140, 77], dtype=torch.int32, device="cuda")
    qs, ks, vs = (t.clone().requires_grad_(True) for t in (q, k, v))
    out = api.entmax_attn_fn(qs, ks, vs, alpha=1.5, causal=True, varlen=lens)
    out.backward(dO)
    torch.cuda.synchronize()
    refs = oracle.entmax_attention_backward(f64(q), f64(k), f64(v), f64(dO), 1.5, True, varlen=np.array([140, 77]))
    for t, r, name in zip((qs, ks, vs), refs, ("dQ", "dK", "dV")):
        _close(f64(t.grad), r, torch.float32, f"autograd varlen {name}")
