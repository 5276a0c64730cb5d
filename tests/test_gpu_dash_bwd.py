"""GPU parity of the DashAttention prefill backward (dash_sparse_attn_prefill_backward)
against the float64 oracle's ``dash_backward``, through the C ABI.

Cases cover the own chunk attended with weight 1 and routed with its prefix
estimate, non-causal routing, alpha 1.5 / 2 / 1.333, GQA, a scaling factor,
ragged last chunks and sequences of one chunk or less. The bf16 gradients are
held to 2e-2 + 2^-8 |reference| (the bf16 result carries 2^-9 of its own
magnitude as rounding); dcls (float32) to 1e-4 + 2^-14 max|reference| -- it
sums one term per (row, routed chunk) and per summarised key over every row and
head of its KV head in float32, and the routing weights it depends on are
recomputed from the forward's float32 tau (within 1e-4 of the exact one).
"""

import numpy as np
import pytest
import torch

import oracle
from adaptive_sparse_long_amd import api
from adaptive_sparse_long_amd.workloads import cotangent, routed_prefill_inputs

from _helpers import f64

pytestmark = pytest.mark.gpu
C = 64


def _bf16_tol(ref):
    return 2e-2 + 2.0 ** -8 * np.abs(ref)


def _check(name, got, ref, tol):
    err = np.abs(got - ref)
    bad = err > tol
    assert not bad.any(), f"{name}: {int(bad.sum())} entries off, max err {float(err.max()):.3e} at {np.unravel_index(np.argmax(err - tol), err.shape)}"


def _run(B, Hq, Hkv, N, p: api.Params, seed, planted="chunks", d=128):
    Q, K, V, cls = routed_prefill_inputs(B, Hq, Hkv, N, d, seed, planted=planted, device="cuda")
    dO = cotangent((B, Hq, N, d), seed + 1, dtype="bf16", device="cuda")
    O, tau, bits, S, _ = api.prefill(Q, K, V, cls, p, with_bits=True)
    dQ, dK, dV, dcls = api.prefill_backward(Q, K, V, cls, S, dO, tau, bits, p)
    torch.cuda.synchronize()
    op = oracle.DashParams(chunk_size=C, alpha=p.alpha, scaling_factor=p.scaling_factor, causal=p.causal,
                           estimate_diagonal=p.estimate_diagonal)
    ref = oracle.dash_backward(f64(Q), f64(K), f64(V), f64(cls), f64(dO), op)
    for name, got, r in zip(("dQ", "dK", "dV"), (dQ, dK, dV), ref[:3]):
        _check(f"{name} N={N} {p}", f64(got), r, _bf16_tol(r))
    _check(f"dcls N={N} {p}", f64(dcls), ref[3], 1e-4 + 2.0 ** -14 * float(np.abs(ref[3]).max()))
    return dQ, dK, dV, dcls


@pytest.mark.parametrize(
    "B,Hq,Hkv,N,p,planted",
    [
        (1, 4, 1, 300, api.Params(estimate_diagonal=False), "needles"),
        (1, 4, 2, 260, api.Params(estimate_diagonal=True), "chunks"),
        (2, 2, 1, 200, api.Params(causal=False), "chunks"),
        (1, 2, 1, 330, api.Params(alpha=2.0), "chunks"),
        (1, 2, 2, 270, api.Params(alpha=1.333, scaling_factor=2.0), None),
        (1, 2, 1, 64, api.Params(), None),
        (1, 2, 1, 37, api.Params(estimate_diagonal=False), None),
        (1, 8, 2, 520, api.Params(estimate_diagonal=False), "needles"),
    ],
)
def test_prefill_backward_small(B, Hq, Hkv, N, p, planted):
    _run(B, Hq, Hkv, N, p, seed=100 + N, planted=planted)


@pytest.mark.parametrize(
    "B,Hq,Hkv,N,p,planted",
    [
        (1, 4, 2, 260, api.Params(estimate_diagonal=True), "chunks"),
        (1, 4, 1, 300, api.Params(estimate_diagonal=False), "needles"),
        (2, 2, 1, 200, api.Params(causal=False), "chunks"),
        (1, 2, 1, 330, api.Params(alpha=2.0), "chunks"),
    ],
)
def test_prefill_backward_head_dim_64(B, Hq, Hkv, N, p, planted):
    """The DashAttention backward at head_dim 64 against the oracle."""
    _run(B, Hq, Hkv, N, p, seed=300 + N, planted=planted, d=64)


@pytest.mark.parametrize(
    "B,Hq,Hkv,N,p",
    [
        (1, 2, 1, 1, api.Params()),
        (1, 2, 1, 2, api.Params(estimate_diagonal=False)),
        (1, 2, 2, 65, api.Params()),
        (1, 2, 1, 129, api.Params(causal=False)),
    ],
)
def test_prefill_backward_tiny_edges(B, Hq, Hkv, N, p):
    """The backward at tiny and ragged lengths around the chunk and tile sizes."""
    _run(B, Hq, Hkv, N, p, seed=400 + N, planted=None)


def test_prefill_backward_deterministic():
    Q, K, V, cls = routed_prefill_inputs(1, 4, 1, 400, 128, 5, planted="chunks", device="cuda")
    dO = cotangent((1, 4, 400, 128), 6, dtype="bf16", device="cuda")
    p = api.Params()
    O, tau, bits, S, _ = api.prefill(Q, K, V, cls, p)
    g1 = api.prefill_backward(Q, K, V, cls, S, dO, tau, bits, p)
    g2 = api.prefill_backward(Q, K, V, cls, S, dO, tau, bits, p)
    for a, b in zip(g1, g2):
        assert torch.equal(a, b)


def test_dash_attn_fn_autograd():
    """torch autograd through the whole prefill (dash_attn_fn) gives the oracle's gradients."""
    p = api.Params(estimate_diagonal=False)
    Q, K, V, cls = routed_prefill_inputs(1, 2, 1, 200, 128, 9, planted="needles", device="cuda")
    dO = cotangent((1, 2, 200, 128), 10, dtype="bf16", device="cuda")
    q, k, v, c = (t.clone().requires_grad_(True) for t in (Q, K, V, cls))
    out = api.dash_attn_fn(q, k, v, c, p)
    out.backward(dO)
    op = oracle.DashParams(chunk_size=C, alpha=p.alpha, causal=True, estimate_diagonal=False)
    ref = oracle.dash_backward(f64(Q), f64(K), f64(V), f64(cls), f64(dO), op)
    for name, t, r in zip(("dQ", "dK", "dV"), (q, k, v), ref[:3]):
        _check(f"autograd {name}", f64(t.grad), r, _bf16_tol(r))
    # head_cls's gradient comes back in head_cls's dtype (bf16)
    _check("autograd dcls", f64(c.grad), ref[3], _bf16_tol(ref[3]))
