"""GPU parity of the chunk-summary backward (dash_summarize_backward) against
the float64 CPU oracle (oracle.chunk_summary_backward), through the C ABI: dK
rows of the listed chunks and dcls (summed over batch entries and chunks) within
1e-4 absolute (float32 outputs of bf16 keys), rows outside the listed chunks
untouched (zero), a ragged last chunk, a sub-range of chunks, and the 32K
prefill workload's keys at full size (every KV head, dK on sampled chunks).
"""

import numpy as np
import pytest
import torch

import oracle
from adaptive_sparse_long_amd import api
from adaptive_sparse_long_amd.workloads import WORKLOADS, cotangent, routed_prefill_inputs

from _helpers import TOL_F32, assert_close, f64

pytestmark = pytest.mark.gpu
C = 64


def _reference(K, cls, dS, n_tokens, c0, c1, chunks=None):
    B, Hkv, Lmax, d = K.shape
    dK = np.zeros((B, Hkv, Lmax, d))
    dcls = np.zeros((Hkv, d))
    n_terms, term_max = 0, 0.0
    for b in range(B):
        for h in range(Hkv):
            for c in range(c0, c1):
                t0, t1 = c * C, min((c + 1) * C, n_tokens)
                if t1 <= t0:
                    continue
                dk, dc = oracle.chunk_summary_backward(K[b, h, t0:t1], cls[h], dS[b, h, c])
                dcls[h] += dc
                n_terms += 1 if h == 0 else 0
                term_max = max(term_max, float(np.abs(dc).max()))
                if chunks is None or c in chunks:
                    dK[b, h, t0:t1] = dk
    _reference.last_terms = (n_terms, term_max)
    return dK, dcls


def dcls_tol(n_terms, term_max):
    """dcls is a float32 sum of n per-chunk terms (each within float32 rounding of
    its exact value): its error grows with n times the largest term. The bar is
    1e-4 plus n * 2^-22 (four float32 ulps) times that largest term."""
    return TOL_F32 + n_terms * 2.0 ** -22 * term_max


@pytest.mark.parametrize("B,Hkv,Lmax,n_tokens,c0,c1,cls_scale", [
    (2, 2, 320, 300, 0, 5, 1.0),   # ragged last chunk (44 tokens)
    (1, 3, 256, 256, 1, 3, 3.0),   # sub-range of chunks, peaked pooling weights
    (3, 1, 128, 65, 0, 2, 0.0),    # head_cls = 0 (mean pooling), one-token last chunk
])
def test_summarize_backward_small(B, Hkv, Lmax, n_tokens, c0, c1, cls_scale):
    gen = torch.Generator(device="cuda")
    gen.manual_seed(500 + Lmax + c1)
    K = torch.randn(B, Hkv, Lmax, 128, generator=gen, device="cuda").to(torch.bfloat16)
    cls = (torch.randn(Hkv, 128, generator=gen, device="cuda") * cls_scale).to(torch.bfloat16)
    s_cap = c1 + 1
    dS = cotangent((B, Hkv, s_cap, 128), 600 + Lmax, dtype="f32", device="cuda")
    p = api.Params()
    dK, dcls = api.summarize_backward(K, cls, dS, n_tokens=n_tokens, chunk_begin=c0, chunk_end=c1, params=p)
    torch.cuda.synchronize()
    rK, rc = _reference(f64(K), f64(cls), f64(dS), n_tokens, c0, c1)
    assert_close(f64(dK), rK, TOL_F32, "dK")
    assert_close(f64(dcls), rc, TOL_F32, "dcls")
    assert bool((dK[:, :, : c0 * C] == 0).all()) and bool((dK[:, :, min(c1 * C, Lmax):] == 0).all())


@pytest.mark.parametrize("B,Hkv,Lmax,n_tokens,c0,c1", [(2, 2, 320, 300, 0, 5), (1, 1, 128, 65, 0, 2)])
def test_summarize_backward_head_dim_64(B, Hkv, Lmax, n_tokens, c0, c1):
    gen = torch.Generator(device="cuda")
    gen.manual_seed(700 + Lmax)
    K = torch.randn(B, Hkv, Lmax, 64, generator=gen, device="cuda").to(torch.bfloat16)
    cls = torch.randn(Hkv, 64, generator=gen, device="cuda").to(torch.bfloat16)
    dS = cotangent((B, Hkv, c1 + 1, 64), 800 + Lmax, dtype="f32", device="cuda")
    dK, dcls = api.summarize_backward(K, cls, dS, n_tokens=n_tokens, chunk_begin=c0, chunk_end=c1,
                                      params=api.Params())
    torch.cuda.synchronize()
    rK, rc = _reference(f64(K), f64(cls), f64(dS), n_tokens, c0, c1)
    assert_close(f64(dK), rK, TOL_F32, "dK d64")
    assert_close(f64(dcls), rc, TOL_F32, "dcls d64")


def test_summarize_backward_deterministic_and_empty_range():
    gen = torch.Generator(device="cuda")
    gen.manual_seed(7)
    K = torch.randn(2, 2, 512, 128, generator=gen, device="cuda").to(torch.bfloat16)
    cls = torch.randn(2, 128, generator=gen, device="cuda").to(torch.bfloat16)
    dS = cotangent((2, 2, 8, 128), 8, dtype="f32", device="cuda")
    a = api.summarize_backward(K, cls, dS)
    b = api.summarize_backward(K, cls, dS)
    torch.cuda.synchronize()
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])
    dK, dcls = api.summarize_backward(K, cls, dS, chunk_begin=3, chunk_end=3)
    torch.cuda.synchronize()
    assert bool((dK == 0).all()) and bool((dcls == 0).all())


def test_summarize_backward_32k_workload():
    """The 32K prefill workload's keys and head_cls (8 KV heads, 512 chunks, d 128):
    dcls of every head in full, dK on sampled chunks."""
    w = WORKLOADS["routed_prefill_32k"]
    _, K, _, cls = routed_prefill_inputs(w.B, w.Hq, w.Hkv, w.N, w.d, w.seed, planted=w.planted, device="cuda")
    n_c = w.N // C
    dS = cotangent((w.B, w.Hkv, n_c, w.d), w.seed + 700, dtype="f32", device="cuda")
    dK, dcls = api.summarize_backward(K, cls, dS)
    torch.cuda.synchronize()
    rng = np.random.default_rng(w.seed)
    sample = set(int(c) for c in np.concatenate([[0, n_c - 1], rng.integers(0, n_c, 6)]))
    rK, rc = _reference(f64(K), f64(cls), f64(dS), w.N, 0, n_c, chunks=sample)
    # dcls adds 512 chunk terms per head (up to ~10 each with the x4 needle keys)
    n_terms, term_max = _reference.last_terms
    assert_close(f64(dcls), rc, dcls_tol(n_terms, term_max), f"dcls (sum of {n_terms} chunk terms)")
    for c in sorted(sample):
        assert_close(f64(dK[:, :, c * C : (c + 1) * C]), rK[:, :, c * C : (c + 1) * C], TOL_F32, f"dK chunk {c}")


def test_summarize_backward_decode_cache():
    """The 128K decode cache at batch 16 (8 KV heads, 2048 chunks per sequence):
    dcls of two heads in full (32768 chunk terms each), dK on sampled chunks."""
    w = WORKLOADS["decode_128k"]
    gen = torch.Generator(device="cuda")
    gen.manual_seed(w.seed)
    K = torch.randn(w.B, w.Hkv, w.N, w.d, generator=gen, device="cuda").to(torch.bfloat16)
    cls = torch.randn(w.Hkv, w.d, generator=gen, device="cuda").to(torch.bfloat16)
    n_c = w.N // C
    dS = cotangent((w.B, w.Hkv, n_c, w.d), w.seed + 700, dtype="f32", device="cuda")
    dK, dcls = api.summarize_backward(K, cls, dS)
    torch.cuda.synchronize()
    for h in (0, 7):
        Kh, dSh, ch = f64(K[:, h]), f64(dS[:, h]), f64(cls[h])
        ref = np.zeros(w.d)
        term_max = 0.0
        for b in range(w.B):
            for c in range(n_c):
                dc = oracle.chunk_summary_backward(Kh[b, c * C : (c + 1) * C], ch, dSh[b, c])[1]
                ref += dc
                term_max = max(term_max, float(np.abs(dc).max()))
        # 32768 chunk terms added in float32
        assert_close(f64(dcls[h]), ref, dcls_tol(w.B * n_c, term_max), f"dcls head {h}")
    rng = np.random.default_rng(w.seed)
    for _ in range(8):
        b, h, c = int(rng.integers(0, w.B)), int(rng.integers(0, w.Hkv)), int(rng.integers(0, n_c))
        dk_ref, _ = oracle.chunk_summary_backward(f64(K[b, h, c * C : (c + 1) * C]), f64(cls[h]), f64(dS[b, h, c]))
        assert_close(f64(dK[b, h, c * C : (c + 1) * C]), dk_ref, TOL_F32, f"dK b{b} h{h} c{c}")
