"""The C ABI library loads without a GPU, exports every symbol the header
declares, and rejects bad arguments on the host before any HIP call.

Only argument combinations that fail validation are passed here (plus the pure
host helpers), so nothing is launched: these tests need no GPU.
"""

import ctypes

import pytest

from adaptive_sparse_long_amd import _lib

OK, INVALID, UNSUPPORTED, WORKSPACE = 0, 1, 2, 3
FAKE = ctypes.c_void_p(0x1000)  # never dereferenced: every call below fails validation first
NULL = ctypes.c_void_p(0)


@pytest.fixture(scope="module")
def lib():
    return _lib.load()


def test_header_symbols_exported(lib):
    names = _lib.header_symbols()
    assert set(names) == {
        "dash_default_params", "dash_status_string", "dash_summarize", "dash_workspace_size",
        "dash_route", "dash_sparse_attn_prefill", "dash_sparse_attn_decode", "entmax_attn",
        "entmax_rows", "entmax_rows_backward", "entmax_attn_backward", "dash_summarize_backward",
        "dash_decode_step_noalloc", "dash_decode_noalloc_max_bytes",
        "dash_sparse_attn_prefill_backward", "dash_backward_workspace_size",
        "dash_prefill_workspace_size", "dash_prefill_counters",
    }
    for n in names:
        assert hasattr(lib, n), n


def test_default_params_and_status_strings(lib):
    p = _lib.DashParams()
    lib.dash_default_params(ctypes.byref(p))
    assert (p.chunk_size, p.alpha, p.n_iter, p.scaling_factor, p.causal, p.estimate_diagonal) == (64, 1.5, 10, 1.0, 1, 1)
    assert lib.dash_status_string(0) == b"ok"
    assert lib.dash_status_string(3) == b"workspace too small"
    assert lib.dash_status_string(99) == b"unknown status"


def _p(**kw):
    return _lib.params(**kw)


def test_workspace_size(lib):
    p = _p()
    assert lib.dash_workspace_size(1, 32, 8, 4096, 4096, 128, 0, p) > 0
    assert lib.dash_workspace_size(16, 32, 8, 1, 131073, 128, 1, p) > 0
    assert lib.dash_workspace_size(1, 6, 4, 128, 128, 128, 0, p) == 0  # Hq % Hkv
    assert lib.dash_workspace_size(1, 4, 4, 200, 100, 128, 0, p) == 0  # Nq > Lmax
    assert lib.dash_workspace_size(1, 4, 4, 100, 100, 128, 0, _p(chunk_size=32)) == 0
    # causal tiles are packed in a triangle: smaller than the rectangle
    assert lib.dash_workspace_size(1, 4, 4, 4096, 4096, 128, 0, p) < lib.dash_workspace_size(
        1, 4, 4, 4096, 4096, 128, 0, _p(causal=False))


def test_prefill_workspace_pool(lib):
    """The prefill workspace is a fixed part plus the partial-result pool
    (2 d + 36 bytes per pair, rounded to 256-byte arrays); the default pool is
    16 pairs per row up to 8K tokens and 5 from 32K on, which keeps the 32K
    workload (B 1, 32 query heads, 8 KV heads, d 128) under 2 GB."""
    p = _p()
    base = lib.dash_prefill_workspace_size(1, 32, 8, 32768, 32768, 128, p, 0)
    assert base > 0
    assert lib.dash_prefill_workspace_size(1, 32, 8, 32768, 32768, 128, p, -1) == 0
    assert lib.dash_prefill_workspace_size(1, 32, 8, 32768, 32768, 128, p, 1 << 33) == 0
    assert lib.dash_prefill_workspace_size(1, 6, 4, 128, 128, 128, p, 0) == 0  # Hq % Hkv
    for pairs in (1000, 10 ** 6):
        grown = lib.dash_prefill_workspace_size(1, 32, 8, 32768, 32768, 128, p, pairs) - base
        assert pairs * 292 <= grown <= pairs * 292 + 5 * 256 + 8 * (pairs // 768 + 1) + 256
    rows32 = 32 * 32768
    assert lib.dash_workspace_size(1, 32, 8, 32768, 32768, 128, 0, p) == lib.dash_prefill_workspace_size(
        1, 32, 8, 32768, 32768, 128, p, 5 * rows32)
    assert lib.dash_workspace_size(1, 32, 8, 32768, 32768, 128, 0, p) < 2 * 2 ** 30
    # head_dim 64 runs the 128-wide layouts: the same workspace
    assert lib.dash_workspace_size(1, 32, 8, 4096, 4096, 64, 0, p) == lib.dash_workspace_size(1, 32, 8, 4096, 4096, 128, 0, p)
    assert lib.dash_workspace_size(2, 8, 2, 1, 8193, 64, 1, p) == lib.dash_workspace_size(2, 8, 2, 1, 8193, 128, 1, p)
    assert lib.dash_workspace_size(1, 32, 8, 4096, 4096, 128, 0, p) == lib.dash_prefill_workspace_size(
        1, 32, 8, 4096, 4096, 128, p, 16 * 32 * 4096)
    assert lib.dash_workspace_size(1, 32, 8, 16384, 16384, 128, 0, p) == lib.dash_prefill_workspace_size(
        1, 32, 8, 16384, 16384, 128, p, 8 * 32 * 16384)


def _summ(lib, K=FAKE, cls=FAKE, S=FAKE, dt=1, B=1, Hkv=1, Lmax=128, d=128, n=128, seqlens=NULL, c0=0, c1=2, cap=2, p=None):
    return lib.dash_summarize(K, cls, S, dt, B, Hkv, Lmax, d, n, seqlens, c0, c1, cap, p or _p(), NULL)


def test_summarize_validation(lib):
    assert _summ(lib, K=NULL) == INVALID
    assert _summ(lib, B=0) == INVALID
    assert _summ(lib, c1=3, cap=2) == INVALID       # chunk_end beyond the cache
    assert _summ(lib, n=0) == INVALID
    assert _summ(lib, n=200, Lmax=128) == INVALID
    assert _summ(lib, d=96) == UNSUPPORTED   # head_dim 64 and 128 only
    assert _summ(lib, dt=0) == UNSUPPORTED
    assert _summ(lib, dt=7) == INVALID
    assert _summ(lib, p=_p(chunk_size=32)) == UNSUPPORTED
    assert _summ(lib, c0=1, c1=1) == OK             # empty range: nothing to do, nothing launched


def _route(lib, Q=FAKE, K=FAKE, cls=FAKE, S=FAKE, dt=1, B=1, Hq=4, Hkv=1, Nq=256, Lmax=256, d=128, cap=4,
           seqlens=NULL, p=None, tau=FAKE, bits=NULL, words=1, ws=FAKE, ws_bytes=0):
    return lib.dash_route(Q, K, cls, S, dt, B, Hq, Hkv, Nq, Lmax, d, cap, seqlens, p or _p(), tau, bits, words,
                          ws, ws_bytes, NULL)


def test_route_validation(lib):
    assert _route(lib, Q=NULL) == INVALID
    assert _route(lib, tau=NULL) == INVALID
    assert _route(lib, Hq=6, Hkv=4) == INVALID
    assert _route(lib, p=_p(alpha=1.0)) == INVALID
    assert _route(lib, p=_p(alpha=float("nan"))) == INVALID
    assert _route(lib, p=_p(n_iter=0)) == INVALID
    assert _route(lib, d=96) == UNSUPPORTED
    assert _route(lib, d=64, ws_bytes=16) == WORKSPACE  # head_dim 64 passes the checks
    assert _route(lib, dt=0) == UNSUPPORTED
    assert _route(lib, p=_p(chunk_size=128)) == UNSUPPORTED
    assert _route(lib, Nq=300, Lmax=256) == INVALID
    assert _route(lib, Nq=140000, Lmax=140000, cap=2200) == UNSUPPORTED  # > 2048 chunk slots in prefill
    assert _route(lib, cap=2) == INVALID                             # summary cache too small
    assert _route(lib, bits=FAKE, words=0) == INVALID
    assert _route(lib, ws_bytes=16) == WORKSPACE
    # decode mode
    assert _route(lib, seqlens=FAKE, Nq=2) == INVALID
    assert _route(lib, seqlens=FAKE, Nq=1, p=_p(causal=False)) == INVALID
    assert _route(lib, seqlens=FAKE, Nq=1, Hq=12, Hkv=4) == UNSUPPORTED  # g = 3
    assert _route(lib, seqlens=FAKE, Nq=1, Lmax=300000, cap=5000) == UNSUPPORTED
    assert _route(lib, seqlens=FAKE, Nq=1, ws_bytes=16) == WORKSPACE


def test_attention_validation(lib):
    p = _p()
    f = lib.dash_sparse_attn_prefill
    assert f(NULL, FAKE, FAKE, 1, 1, 4, 1, 256, 256, 128, p, FAKE, FAKE, 0, NULL) == INVALID
    assert f(FAKE, FAKE, FAKE, 1, 1, 4, 1, 256, 128, 128, p, FAKE, FAKE, 0, NULL) == INVALID
    assert f(FAKE, FAKE, FAKE, 1, 1, 4, 1, 256, 256, 96, p, FAKE, FAKE, 0, NULL) == UNSUPPORTED
    assert f(FAKE, FAKE, FAKE, 1, 1, 4, 1, 256, 256, 64, p, FAKE, FAKE, 8, NULL) == WORKSPACE
    assert f(FAKE, FAKE, FAKE, 1, 1, 4, 1, 256, 256, 128, p, FAKE, FAKE, 8, NULL) == WORKSPACE
    g = lib.dash_sparse_attn_decode
    assert g(FAKE, FAKE, FAKE, 1, 1, 4, 1, NULL, 256, 128, p, FAKE, FAKE, 0, NULL) == INVALID
    assert g(FAKE, FAKE, FAKE, 1, 1, 4, 1, FAKE, 256, 128, _p(causal=False), FAKE, FAKE, 0, NULL) == INVALID
    assert g(FAKE, FAKE, FAKE, 1, 1, 48, 1, FAKE, 256, 128, p, FAKE, FAKE, 0, NULL) == UNSUPPORTED
    assert g(FAKE, FAKE, FAKE, 1, 1, 4, 1, FAKE, 256, 128, p, FAKE, FAKE, 8, NULL) == WORKSPACE
    assert g(FAKE, FAKE, FAKE, 1, 1, 4, 1, FAKE, 256, 96, p, FAKE, FAKE, 0, NULL) == UNSUPPORTED
    assert g(FAKE, FAKE, FAKE, 1, 1, 4, 1, FAKE, 256, 64, p, FAKE, FAKE, 8, NULL) == WORKSPACE
    e = lib.entmax_attn
    assert e(NULL, FAKE, FAKE, 1, 1, 1, 128, 64, NULL, 1.5, 10, 1, FAKE, FAKE, NULL, NULL) == INVALID
    assert e(FAKE, FAKE, FAKE, 1, 1, 1, 128, 64, NULL, 1.0, 10, 1, FAKE, FAKE, NULL, NULL) == INVALID
    assert e(FAKE, FAKE, FAKE, 1, 1, 1, 128, 64, NULL, 1.5, 0, 1, FAKE, FAKE, NULL, NULL) == INVALID
    assert e(FAKE, FAKE, FAKE, 1, 1, 1, 128, 64, NULL, 1.5, 10, 2, FAKE, FAKE, NULL, NULL) == INVALID
    assert e(FAKE, FAKE, FAKE, 1, 1, 1, 128, 96, NULL, 1.5, 10, 1, FAKE, FAKE, NULL, NULL) == UNSUPPORTED
    assert e(FAKE, FAKE, FAKE, 1, 1, 1, 70000, 64, NULL, 1.5, 10, 1, FAKE, FAKE, NULL, NULL) == UNSUPPORTED


def test_entmax_rows_validation(lib):
    r = lib.entmax_rows
    assert r(NULL, FAKE, 0, 4, 16, 1.5, 10, NULL, NULL) == INVALID
    assert r(FAKE, NULL, 0, 4, 16, 1.5, 10, NULL, NULL) == INVALID
    assert r(FAKE, FAKE, 0, 0, 16, 1.5, 10, NULL, NULL) == INVALID
    assert r(FAKE, FAKE, 0, 4, 0, 1.5, 10, NULL, NULL) == INVALID
    assert r(FAKE, FAKE, 0, 4, 16, 1.0, 10, NULL, NULL) == INVALID
    assert r(FAKE, FAKE, 0, 4, 16, float("inf"), 10, NULL, NULL) == INVALID
    assert r(FAKE, FAKE, 0, 4, 16, 1.5, 0, NULL, NULL) == INVALID
    assert r(FAKE, FAKE, 7, 4, 16, 1.5, 10, NULL, NULL) == INVALID
    assert r(FAKE, FAKE, 0, 4, 32769, 1.5, 10, NULL, NULL) == UNSUPPORTED
    b = lib.entmax_rows_backward
    assert b(NULL, FAKE, FAKE, 0, 4, 16, 1.5, NULL) == INVALID
    assert b(FAKE, NULL, FAKE, 0, 4, 16, 1.5, NULL) == INVALID
    assert b(FAKE, FAKE, NULL, 0, 4, 16, 1.5, NULL) == INVALID
    assert b(FAKE, FAKE, FAKE, 0, 0, 16, 1.5, NULL) == INVALID
    assert b(FAKE, FAKE, FAKE, 0, 4, 16, 0.5, NULL) == INVALID
    assert b(FAKE, FAKE, FAKE, 3, 4, 16, 1.5, NULL) == INVALID
    assert b(FAKE, FAKE, FAKE, 0, 4, 40000, 1.5, NULL) == UNSUPPORTED


def test_entmax_attn_backward_validation(lib):
    e = lib.entmax_attn_backward
    F5 = [FAKE] * 5
    # Q K V dO tau mask dt B H N d varlen alpha causal dQ dK dV coef stream
    assert e(NULL, *F5[1:], NULL, 1, 1, 1, 128, 64, NULL, 1.5, 1, FAKE, FAKE, FAKE, FAKE, NULL) == INVALID
    assert e(*F5[:4], NULL, NULL, 1, 1, 1, 128, 64, NULL, 1.5, 1, FAKE, FAKE, FAKE, FAKE, NULL) == INVALID
    assert e(*F5, NULL, 1, 1, 1, 128, 64, NULL, 1.5, 1, FAKE, FAKE, FAKE, NULL, NULL) == INVALID
    assert e(*F5, NULL, 1, 1, 1, 128, 64, NULL, 1.5, 1, NULL, FAKE, FAKE, FAKE, NULL) == INVALID
    assert e(*F5, NULL, 1, 0, 1, 128, 64, NULL, 1.5, 1, FAKE, FAKE, FAKE, FAKE, NULL) == INVALID
    assert e(*F5, NULL, 1, 1, 1, 128, 64, NULL, 1.0, 1, FAKE, FAKE, FAKE, FAKE, NULL) == INVALID
    assert e(*F5, NULL, 1, 1, 1, 128, 64, NULL, float("nan"), 1, FAKE, FAKE, FAKE, FAKE, NULL) == INVALID
    assert e(*F5, NULL, 1, 1, 1, 128, 64, NULL, 1.5, 3, FAKE, FAKE, FAKE, FAKE, NULL) == INVALID
    assert e(*F5, NULL, 5, 1, 1, 128, 64, NULL, 1.5, 1, FAKE, FAKE, FAKE, FAKE, NULL) == INVALID
    assert e(*F5, NULL, 1, 1, 1, 128, 96, NULL, 1.5, 1, FAKE, FAKE, FAKE, FAKE, NULL) == UNSUPPORTED
    assert e(*F5, NULL, 1, 1, 1, 70000, 64, NULL, 1.5, 1, FAKE, FAKE, FAKE, FAKE, NULL) == UNSUPPORTED


def test_summarize_backward_validation(lib):
    f = lib.dash_summarize_backward
    p = _lib.params()
    F3 = [FAKE] * 3
    # K cls dS dt B Hkv Lmax d n_tokens c0 c1 s_cap params dK dcls parts stream
    assert f(NULL, FAKE, FAKE, 1, 1, 2, 256, 128, 256, 0, 4, 4, p, *F3, NULL) == INVALID
    assert f(*F3, 1, 1, 2, 256, 128, 256, 0, 4, 4, p, FAKE, NULL, FAKE, NULL) == INVALID
    assert f(*F3, 1, 1, 2, 256, 128, 256, 0, 4, 4, p, FAKE, FAKE, NULL, NULL) == INVALID
    assert f(*F3, 1, 0, 2, 256, 128, 256, 0, 4, 4, p, *F3, NULL) == INVALID
    assert f(*F3, 1, 1, 2, 256, 128, 300, 0, 4, 4, p, *F3, NULL) == INVALID
    assert f(*F3, 1, 1, 2, 256, 128, 256, 3, 2, 4, p, *F3, NULL) == INVALID
    assert f(*F3, 1, 1, 2, 256, 128, 256, 0, 5, 4, p, *F3, NULL) == INVALID
    assert f(*F3, 1, 1, 2, 256, 128, 256, 0, 6, 8, p, *F3, NULL) == INVALID
    assert f(*F3, 0, 1, 2, 256, 128, 256, 0, 4, 4, p, *F3, NULL) == UNSUPPORTED
    assert f(*F3, 1, 1, 2, 256, 96, 256, 0, 4, 4, p, *F3, NULL) == UNSUPPORTED
    assert f(*F3, 1, 1, 2, 256, 128, 256, 0, 4, 4, _lib.params(chunk_size=32), *F3, NULL) == UNSUPPORTED


def test_decode_noalloc_validation(lib):
    """The allocation-free decode step checks its arguments on the host: NULL
    pointers, bad sizes and sizes beyond its static scratch are refused before
    any HIP call (so this runs without a GPU)."""
    cap = int(lib.dash_decode_noalloc_max_bytes())
    assert cap == 64 << 20
    p = _p()
    P = ctypes.c_void_p(16)  # never dereferenced: every case fails on the host
    # NULL q
    assert lib.dash_decode_step_noalloc(None, P, P, P, P, 1, 16, 32, 8, P, 131073, 128, 2048, p, P, P, None, 0, None) == 1
    # Hq not a multiple of Hkv
    assert lib.dash_decode_step_noalloc(P, P, P, P, P, 1, 16, 30, 8, P, 131073, 128, 2048, p, P, P, None, 0, None) == 1
    # the 128K batch-16 decode fits the scratch ...
    assert lib.dash_workspace_size(16, 32, 8, 1, 131073, 128, 1, p) <= cap
    # ... batch 64 at 256K does not
    assert lib.dash_workspace_size(64, 32, 8, 1, 262145, 128, 1, p) > cap
    assert lib.dash_decode_step_noalloc(P, P, P, P, P, 1, 64, 32, 8, P, 262145, 128, 4096, p, P, P, None, 0, None) == 3
    # non-causal decode is refused
    assert lib.dash_decode_step_noalloc(P, P, P, P, P, 1, 2, 8, 2, P, 1024, 128, 16, _p(causal=False), P, P, None, 0,
                                        None) == 1


def test_backward_head_dim(lib):
    """The backward entry points take head_dim 64 and 128 and refuse others on
    the host (no launch)."""
    p = _p()
    f = lib.dash_sparse_attn_prefill_backward
    F8 = [FAKE] * 8
    # Q K V cls S dO tau bits words dt B Hq Hkv N Lmax d s_cap params dQ dK dV dcls ws ws_bytes stream
    assert f(*F8, 8, 1, 1, 4, 1, 256, 256, 96, 4, p, FAKE, FAKE, FAKE, FAKE, FAKE, 1 << 30, NULL) == UNSUPPORTED
    assert f(*F8, 8, 1, 1, 4, 1, 256, 256, 64, 4, p, FAKE, FAKE, FAKE, FAKE, FAKE, 16, NULL) == WORKSPACE
    g = lib.dash_summarize_backward
    F3 = [FAKE] * 3
    assert g(*F3, 1, 1, 2, 256, 96, 256, 0, 4, 4, p, *F3, NULL) == UNSUPPORTED
