"""GPU test of dash_decode_step_noalloc (the decode step for callers that cannot
allocate), through the C ABI: on two calls in a row -- the second with a
smaller batch and cache, so stale scratch contents from the first would show --
its outputs must equal those of dash_route (decode mode) + dash_sparse_attn_decode
with a caller workspace, bit for bit (the same kernels run), and meet the
oracle's bar; sizes beyond the static scratch are refused before any launch."""

import numpy as np
import pytest
import torch

import oracle
from adaptive_sparse_long_amd import _lib, api
from adaptive_sparse_long_amd.workloads import decode_inputs

from _helpers import TOL_BF16, assert_close, f64, tau_close

pytestmark = pytest.mark.gpu
C = 64


def _case(B, Hq, Hkv, L, Lmax, seed, lens, d=128):
    q, Kc, Vc, cls, _ = decode_inputs(B, Hq, Hkv, L, d, seed, device="cuda", Lmax=Lmax)
    seqlens = torch.tensor(lens, dtype=torch.int32, device="cuda")
    S = torch.zeros(B, Hkv, -(-Lmax // C), d, dtype=torch.float32, device="cuda")
    p = api.Params()
    api.summarize(Kc, cls, S, seqlens=seqlens, chunk_begin=0, chunk_end=Lmax // C, params=p)
    return q, Kc, Vc, cls, S, seqlens, p


def test_noalloc_decode_matches_workspace_path_twice():
    cases = [
        (4, 8, 2, 3000, 3072, 11, [3001, 2049, 64, 1500]),
        (2, 8, 2, 900, 1024, 12, [901, 640]),  # smaller than the first call
    ]
    for B, Hq, Hkv, L, Lmax, seed, lens in cases:
        q, Kc, Vc, cls, S, seqlens, p = _case(B, Hq, Hkv, L, Lmax, seed, lens)
        ref_O, ref_tau, ref_bits, _ = api.decode_step(q, Kc, Vc, cls, S, seqlens, p)
        O, tau, bits = api.decode_step_noalloc(q, Kc, Vc, cls, S, seqlens, p)
        torch.cuda.synchronize()
        assert torch.equal(O, ref_O), f"B={B}: O differs from the workspace path"
        assert torch.equal(tau, ref_tau), f"B={B}: tau differs from the workspace path"
        assert torch.equal(bits, ref_bits), f"B={B}: routed chunks differ from the workspace path"
        # and the oracle's bar on one (b, kv head) group per call
        op = oracle.DashParams(chunk_size=C, alpha=p.alpha, causal=True, estimate_diagonal=p.estimate_diagonal)
        b, hk = B - 1, Hkv - 1
        n = lens[b]
        g = Hq // Hkv
        keys, vals, clsv = f64(Kc[b, hk, :n]), f64(Vc[b, hk, :n]), f64(cls[hk])
        summ = oracle.chunk_summaries(keys, clsv, C, n)
        for h in range(hk * g, (hk + 1) * g):
            o_ref, t_ref, _ = oracle.dash_rows(f64(q[b, h]), np.array([n - 1]), keys, vals, clsv, n, op, summ)
            tau_close(f64(tau[b, h, :1]), t_ref, f"noalloc b{b} h{h}")
            assert_close(f64(O[b, h, 0]), o_ref[0], TOL_BF16, f"noalloc O b{b} h{h}")


def test_noalloc_decode_head_dim_64():
    """head_dim 64 through the allocation-free step: equal to the workspace path."""
    q, Kc, Vc, cls, S, seqlens, p = _case(2, 8, 2, 900, 1024, 13, [901, 700], d=64)
    ref_O, ref_tau, ref_bits, _ = api.decode_step(q, Kc, Vc, cls, S, seqlens, p)
    O, tau, bits = api.decode_step_noalloc(q, Kc, Vc, cls, S, seqlens, p)
    torch.cuda.synchronize()
    assert torch.equal(O, ref_O) and torch.equal(tau, ref_tau) and torch.equal(bits, ref_bits)


def test_noalloc_refuses_sizes_beyond_the_scratch():
    lib = _lib.load()
    cap = int(lib.dash_decode_noalloc_max_bytes())
    p = api.Params()
    # batch 64 at 262144 cached tokens needs far more than the scratch holds
    need = api.workspace_size(64, 32, 8, 1, 262144, 128, True, p)
    assert need > cap
    dummy = torch.zeros(16, dtype=torch.int32, device="cuda")
    ptr = dummy.data_ptr()
    st = lib.dash_decode_step_noalloc(ptr, ptr, ptr, ptr, ptr, _lib.DASH_BF16, 64, 32, 8, ptr, 262144, 128,
                                      262144 // C, p.c(), ptr, ptr, None, 0, None)
    assert st == 3  # DASH_ERR_WORKSPACE, before any launch
