"""Python binding of libdash.so over torch tensors.

torch provides device memory and the current HIP stream; every step of the
computation runs in the library's kernels. Each function checks that tensors
are contiguous, on the GPU and of the expected dtype, allocates the outputs,
and passes raw pointers to the C entry point of the same name (include/dash.h).

Method (DashAttention README page, "How it works"): ``summarize`` builds one
key summary per chunk with head_cls, ``route`` runs alpha-entmax chunk routing,
``sparse_attn_prefill`` / ``sparse_attn_decode`` run the prior-induced sparse
softmax over the routed chunks. ``entmax_attn`` is the dense alpha-entmax
attention with block skipping of the AdaSplash README page, and ``entmax``
its row-wise entmax activation ("Usage": Triton Entmax).
"""

from __future__ import annotations

import ctypes
from dataclasses import dataclass

import torch

from . import _lib

__all__ = [
    "Params",
    "summarize",
    "workspace_size",
    "prefill_workspace_size",
    "prefill_counters",
    "route",
    "sparse_attn_prefill",
    "sparse_attn_decode",
    "entmax_attn",
    "entmax",
    "entmax_backward",
    "entmax_fn",
    "prefill",
    "decode_step",
    "decode_step_noalloc",
    "prefill_backward",
    "dash_attn_fn",
]

CHUNK = 64


@dataclass(frozen=True)
class Params:
    """The wrapper arguments of "Core API" plus the entmax alpha / iteration count."""

    chunk_size: int = 64
    alpha: float = 1.5
    n_iter: int = 10
    scaling_factor: float = 1.0
    causal: bool = True
    estimate_diagonal: bool = True

    def c(self) -> _lib.DashParams:
        return _lib.params(self.chunk_size, self.alpha, self.n_iter, self.scaling_factor, self.causal, self.estimate_diagonal)


def _p(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else ctypes.c_void_p(0)


def _stream(dev):
    return ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)


def _need(t: torch.Tensor, name: str, dtype=None, dim=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must live on the GPU (the library has no CPU path)")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if dim is not None and t.dim() != dim:
        raise ValueError(f"{name} must have {dim} dimensions")


def _dt(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return _lib.DASH_BF16
    if t.dtype == torch.float32:
        return _lib.DASH_F32
    raise ValueError(f"unsupported dtype {t.dtype}")


def summarize(K, head_cls, S, n_tokens=None, seqlens=None, chunk_begin=0, chunk_end=None, params: Params = Params()):
    """Chunk summaries S[b, h, c] for c in [chunk_begin, chunk_end) ("How it works" 1)."""
    lib = _lib.load()
    _need(K, "K", dim=4)
    _need(head_cls, "head_cls", K.dtype, 2)
    _need(S, "S", torch.float32, 4)
    B, Hkv, Lmax, d = K.shape
    if seqlens is not None:
        _need(seqlens, "seqlens", torch.int32, 1)
    n_tokens = Lmax if n_tokens is None else int(n_tokens)
    if chunk_end is None:
        chunk_end = -(-n_tokens // CHUNK)
    st = lib.dash_summarize(_p(K), _p(head_cls), _p(S), _dt(K), B, Hkv, Lmax, d, n_tokens, _p(seqlens),
                            int(chunk_begin), int(chunk_end), S.shape[2], params.c(), _stream(K.device))
    _lib.check(st, "dash_summarize")
    return S


def summarize_backward(K, head_cls, dS, n_tokens=None, chunk_begin=0, chunk_end=None, params: Params = Params(),
                       out=None):
    """Gradients (dK float32 [B, Hkv, Lmax, d], dcls float32 [Hkv, d]) of the chunk
    summaries over tokens [0, n_tokens) for their cotangent dS (float32
    [B, Hkv, s_cap, d]); dK rows outside the chunks [chunk_begin, chunk_end) are 0.
    ``out`` = (dK, dcls, partials) reuses caller buffers (dK rows outside the
    chunks are then left as they are)."""
    lib = _lib.load()
    _need(K, "K", dim=4)
    _need(head_cls, "head_cls", K.dtype, 2)
    _need(dS, "dS", torch.float32, 4)
    B, Hkv, Lmax, d = K.shape
    n_tokens = Lmax if n_tokens is None else int(n_tokens)
    if chunk_end is None:
        chunk_end = -(-n_tokens // CHUNK)
    if out is None:
        dK = torch.zeros(B, Hkv, Lmax, d, dtype=torch.float32, device=K.device)
        dcls = torch.empty(Hkv, d, dtype=torch.float32, device=K.device)
        parts = torch.empty(B, Hkv, max(int(chunk_end) - int(chunk_begin), 1), d, dtype=torch.float32,
                            device=K.device)
    else:
        dK, dcls, parts = out
        _need(dK, "dK", torch.float32, 4)
        _need(dcls, "dcls", torch.float32, 2)
        _need(parts, "partials", torch.float32)
        if tuple(dK.shape) != (B, Hkv, Lmax, d) or tuple(dcls.shape) != (Hkv, d):
            raise ValueError("dK must be [B, Hkv, Lmax, d] and dcls [Hkv, d]")
        if parts.numel() < B * Hkv * max(int(chunk_end) - int(chunk_begin), 1) * d:
            raise ValueError("partials must hold B * Hkv * (chunk_end - chunk_begin) * d floats")
    st = lib.dash_summarize_backward(_p(K), _p(head_cls), _p(dS), _dt(K), B, Hkv, Lmax, d, n_tokens,
                                     int(chunk_begin), int(chunk_end), dS.shape[2], params.c(), _p(dK),
                                     _p(dcls), _p(parts), _stream(K.device))
    _lib.check(st, "dash_summarize_backward")
    return dK, dcls


def workspace_size(B, Hq, Hkv, Nq, Lmax, d, decode: bool, params: Params = Params()) -> int:
    return int(_lib.load().dash_workspace_size(B, Hq, Hkv, Nq, Lmax, d, int(decode), params.c()))


def prefill_workspace_size(B, Hq, Hkv, Nq, Lmax, d, params: Params = Params(), pool_pairs: int = 0) -> int:
    """Prefill workspace bytes with a partial-result pool of exactly pool_pairs
    (row, routed past chunk) pairs; tiles that find the pool full are attended
    row-major, so any pool size gives the same result up to rounding."""
    return int(_lib.load().dash_prefill_workspace_size(B, Hq, Hkv, Nq, Lmax, d, params.c(), int(pool_pairs)))


def prefill_counters(workspace, B, Hq, Hkv, N, d, params: Params = Params(), device=None) -> dict:
    """Counters of the last prefill routing in `workspace` (synchronises the
    stream): pool pairs used, pool capacity, tiles left to the general routing
    kernel, tiles attended row-major."""
    out = (ctypes.c_longlong * 4)()
    st = _lib.load().dash_prefill_counters(_p(workspace), workspace.numel(), B, Hq, Hkv, N, d, params.c(),
                                           ctypes.cast(out, ctypes.c_void_p), _stream(device or workspace.device))
    _lib.check(st, "dash_prefill_counters")
    return {"pool_pairs": out[0], "pool_capacity": out[1], "general_route_tiles": out[2], "row_major_tiles": out[3]}


def route(Q, K, head_cls, S, params: Params = Params(), seqlens=None, with_bits=True, workspace=None):
    """Chunk routing ("How it works" 2). Returns (tau, active_bits or None, workspace)."""
    lib = _lib.load()
    _need(Q, "Q", dim=4)
    _need(K, "K", Q.dtype, 4)
    _need(head_cls, "head_cls", Q.dtype, 2)
    _need(S, "S", torch.float32, 4)
    B, Hq, Nq, d = Q.shape
    Hkv, Lmax = K.shape[1], K.shape[2]
    decode = seqlens is not None
    if decode:
        _need(seqlens, "seqlens", torch.int32, 1)
    n_slots = -(-(Lmax if decode else Nq) // CHUNK)
    words = -(-n_slots // 32)
    if workspace is None:
        ws_bytes = workspace_size(B, Hq, Hkv, Nq, Lmax, d, decode, params)
        workspace = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=Q.device)
    else:
        # prefill: anything from the pool-free part up (the rest is the pool)
        least = (workspace_size(B, Hq, Hkv, Nq, Lmax, d, True, params) if decode
                 else prefill_workspace_size(B, Hq, Hkv, Nq, Lmax, d, params, 0))
        if workspace.numel() < least:
            raise ValueError(f"workspace holds {workspace.numel()} bytes, these sizes need at least {least}")
    tau = torch.empty(B, Hq, Nq, dtype=torch.float32, device=Q.device)
    bits = torch.empty(B, Hq, Nq, words, dtype=torch.int32, device=Q.device) if with_bits else None
    st = lib.dash_route(_p(Q), _p(K), _p(head_cls), _p(S), _dt(Q), B, Hq, Hkv, Nq, Lmax, d, S.shape[2],
                        _p(seqlens), params.c(), _p(tau), _p(bits), words, _p(workspace),
                        workspace.numel(), _stream(Q.device))
    _lib.check(st, "dash_route")
    return tau, bits, workspace


def sparse_attn_prefill(Q, K, V, workspace, params: Params = Params(), out=None):
    """Prior-induced sparse softmax over the routed chunks ("How it works" 3)."""
    lib = _lib.load()
    _need(Q, "Q", dim=4)
    _need(K, "K", Q.dtype, 4)
    _need(V, "V", Q.dtype, 4)
    B, Hq, N, d = Q.shape
    Hkv, Lmax = K.shape[1], K.shape[2]
    out = torch.empty_like(Q) if out is None else out
    st = lib.dash_sparse_attn_prefill(_p(Q), _p(K), _p(V), _dt(Q), B, Hq, Hkv, N, Lmax, d, params.c(),
                                      _p(out), _p(workspace), workspace.numel(), _stream(Q.device))
    _lib.check(st, "dash_sparse_attn_prefill")
    return out


def sparse_attn_decode(q, Kc, Vc, seqlens, workspace, params: Params = Params(), out=None):
    """Sparse attention of one new token per sequence over the routed cache chunks."""
    lib = _lib.load()
    _need(q, "q", dim=4)
    _need(Kc, "Kc", q.dtype, 4)
    _need(Vc, "Vc", q.dtype, 4)
    _need(seqlens, "seqlens", torch.int32, 1)
    B, Hq, _, d = q.shape
    Hkv, Lmax = Kc.shape[1], Kc.shape[2]
    out = torch.empty_like(q) if out is None else out
    st = lib.dash_sparse_attn_decode(_p(q), _p(Kc), _p(Vc), _dt(q), B, Hq, Hkv, _p(seqlens), Lmax, d,
                                     params.c(), _p(out), _p(workspace), workspace.numel(), _stream(q.device))
    _lib.check(st, "dash_sparse_attn_decode")
    return out


def prefill_backward(Q, K, V, head_cls, S, dO, tau, bits, params: Params = Params(), workspace=None):
    """Gradients (dQ, dK, dV, dcls) of :func:`prefill` for the cotangent ``dO`` of
    its output, from the forward's inputs, its summaries ``S`` and its ``tau`` and
    routed-chunk ``bits`` (``dash_sparse_attn_prefill_backward``). dcls is
    float32; the rest have the inputs' dtype."""
    lib = _lib.load()
    _need(Q, "Q", dim=4)
    for name, t in (("K", K), ("V", V), ("dO", dO)):
        _need(t, name, Q.dtype, 4)
    _need(head_cls, "head_cls", Q.dtype, 2)
    _need(S, "S", torch.float32, 4)
    _need(tau, "tau", torch.float32, 3)
    _need(bits, "bits", torch.int32, 4)
    B, Hq, N, d = Q.shape
    Hkv, Lmax = K.shape[1], K.shape[2]
    if dO.shape != Q.shape or V.shape != K.shape:
        raise ValueError("dO must have Q's shape, V K's shape")
    need = int(lib.dash_backward_workspace_size(B, Hq, Hkv, N, Lmax, d, params.c()))
    if workspace is None or workspace.numel() < need:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=Q.device)
    dQ = torch.empty_like(Q)
    dK = torch.zeros_like(K)
    dV = torch.zeros_like(V)
    dcls = torch.empty(Hkv, d, dtype=torch.float32, device=Q.device)
    st = lib.dash_sparse_attn_prefill_backward(
        _p(Q), _p(K), _p(V), _p(head_cls), _p(S), _p(dO), _p(tau), _p(bits), bits.shape[-1], _dt(Q), B, Hq,
        Hkv, N, Lmax, d, S.shape[2], params.c(), _p(dQ), _p(dK), _p(dV), _p(dcls), _p(workspace), workspace.numel(),
        _stream(Q.device))
    _lib.check(st, "dash_sparse_attn_prefill_backward")
    return dQ, dK, dV, dcls


class _DashPrefillFn(torch.autograd.Function):
    @staticmethod
    def forward(ctx, Q, K, V, head_cls, params):
        O, tau, bits, S, _ = prefill(Q, K, V, head_cls, params, with_bits=True)
        ctx.save_for_backward(Q, K, V, head_cls, S, tau, bits)
        ctx.params = params
        return O

    @staticmethod
    def backward(ctx, dO):
        Q, K, V, head_cls, S, tau, bits = ctx.saved_tensors
        dQ, dK, dV, dcls = prefill_backward(Q, K, V, head_cls, S, dO.contiguous().to(Q.dtype), tau, bits, ctx.params)
        return dQ, dK, dV, dcls.to(head_cls.dtype), None


def dash_attn_fn(Q, K, V, head_cls, params: Params = Params()):
    """The whole prefill (summaries, routing, sparse attention) with a backward
    (torch autograd) through all three stages: gradients into Q, K, V and head_cls
    run in ``dash_sparse_attn_prefill_backward``."""
    return _DashPrefillFn.apply(Q, K, V, head_cls, params)


def decode_step_noalloc(q, Kc, Vc, head_cls, S, seqlens, params: Params = Params(), with_bits=True, out=None):
    """One decode step (routing against the summary cache, then attention over the
    routed chunks) through ``dash_decode_step_noalloc``: the library's own static
    scratch replaces the workspace, so the call allocates no device memory apart
    from the outputs made here when ``out`` is None. ``out`` = (O, tau, bits or
    None) reuses caller tensors. Calls that overlap on one GPU race for the
    scratch. Returns (O, tau, bits). Appending completed chunks stays with the
    caller (``summarize`` with ``seqlens``)."""
    lib = _lib.load()
    _need(q, "q", dim=4)
    _need(Kc, "Kc", q.dtype, 4)
    _need(Vc, "Vc", q.dtype, 4)
    _need(head_cls, "head_cls", q.dtype, 2)
    _need(S, "S", torch.float32, 4)
    _need(seqlens, "seqlens", torch.int32, 1)
    B, Hq, _, d = q.shape
    Hkv, Lmax = Kc.shape[1], Kc.shape[2]
    words = -(-(-(-Lmax // CHUNK)) // 32)
    if out is None:
        O = torch.empty_like(q)
        tau = torch.empty(B, Hq, 1, dtype=torch.float32, device=q.device)
        bits = torch.empty(B, Hq, 1, words, dtype=torch.int32, device=q.device) if with_bits else None
    else:
        O, tau, bits = out
    st = lib.dash_decode_step_noalloc(_p(q), _p(Kc), _p(Vc), _p(head_cls), _p(S), _dt(q), B, Hq, Hkv, _p(seqlens),
                                      Lmax, d, S.shape[2], params.c(), _p(O), _p(tau), _p(bits), words,
                                      _stream(q.device))
    _lib.check(st, "dash_decode_step_noalloc")
    return O, tau, bits


def entmax_attn(Q, K, V, alpha=1.5, n_iter=10, causal=True, varlen=None, with_mask=True):
    """Dense alpha-entmax attention with a per-tile block mask (AdaSplash "Usage")."""
    lib = _lib.load()
    _need(Q, "Q", dim=4)
    _need(K, "K", Q.dtype, 4)
    _need(V, "V", Q.dtype, 4)
    B, H, N, d = Q.shape
    if varlen is not None:
        _need(varlen, "varlen", torch.int32, 1)
    nT = -(-N // 64)
    out = torch.empty_like(Q)
    tau = torch.empty(B, H, N, dtype=torch.float32, device=Q.device)
    mask = torch.empty(B, H, nT, -(-nT // 32), dtype=torch.int32, device=Q.device) if with_mask else None
    st = lib.entmax_attn(_p(Q), _p(K), _p(V), _dt(Q), B, H, N, d, _p(varlen), float(alpha), int(n_iter),
                         int(bool(causal)), _p(out), _p(tau), _p(mask), _stream(Q.device))
    _lib.check(st, "entmax_attn")
    return out, tau, mask


def entmax_attn_backward(Q, K, V, dO, tau, mask=None, alpha=1.5, causal=True, varlen=None):
    """Gradients (dQ, dK, dV) of :func:`entmax_attn` for the cotangent ``dO``, from
    the forward's inputs, its ``tau`` and (optionally) its block ``mask``."""
    lib = _lib.load()
    _need(Q, "Q", dim=4)
    for name, t in (("K", K), ("V", V), ("dO", dO)):
        _need(t, name, Q.dtype, 4)
        if t.shape != Q.shape:
            raise ValueError(f"{name} must have the shape of Q")
    B, H, N, d = Q.shape
    _need(tau, "tau", torch.float32, 3)
    if tuple(tau.shape) != (B, H, N):
        raise ValueError("tau must be [B, H, N]")
    if mask is not None:
        nT = -(-N // 64)
        _need(mask, "mask", torch.int32, 4)
        if tuple(mask.shape) != (B, H, nT, -(-nT // 32)):
            raise ValueError("mask must be [B, H, ceil(N/64), ceil(ceil(N/64)/32)]")
    if varlen is not None:
        _need(varlen, "varlen", torch.int32, 1)
    dQ, dK, dV = torch.empty_like(Q), torch.empty_like(K), torch.empty_like(V)
    coef = torch.empty(B, H, N, dtype=torch.float32, device=Q.device)
    st = lib.entmax_attn_backward(_p(Q), _p(K), _p(V), _p(dO), _p(tau), _p(mask), _dt(Q), B, H, N, d,
                                  _p(varlen), float(alpha), int(bool(causal)), _p(dQ), _p(dK), _p(dV),
                                  _p(coef), _stream(Q.device))
    _lib.check(st, "entmax_attn_backward")
    return dQ, dK, dV


class _EntmaxAttnFn(torch.autograd.Function):
    @staticmethod
    def forward(ctx, Q, K, V, alpha, n_iter, causal, varlen):
        out, tau, mask = entmax_attn(Q, K, V, alpha=alpha, n_iter=n_iter, causal=causal, varlen=varlen)
        ctx.save_for_backward(Q, K, V, tau, mask, varlen)
        ctx.alpha, ctx.causal = alpha, causal
        return out

    @staticmethod
    def backward(ctx, dO):
        Q, K, V, tau, mask, varlen = ctx.saved_tensors
        dQ, dK, dV = entmax_attn_backward(Q, K, V, dO.contiguous().to(Q.dtype), tau, mask, ctx.alpha, ctx.causal, varlen)
        return dQ, dK, dV, None, None, None, None


def entmax_attn_fn(Q, K, V, alpha=1.5, n_iter=10, causal=True, varlen=None):
    """:func:`entmax_attn` with a backward (torch autograd): the gradients run in
    ``entmax_attn_backward``, skipping the tiles the forward's block mask clears."""
    return _EntmaxAttnFn.apply(Q, K, V, alpha, n_iter, causal, varlen)


def entmax(x, alpha=1.5, n_iter=10, return_tau=False, out=None):
    """Row-wise alpha-entmax over the last dimension (AdaSplash "Usage": Triton Entmax).

    ``x`` is a contiguous float32 or bfloat16 GPU tensor; ``out`` (same shape
    and dtype) may be ``x`` itself. Returns the probabilities, and tau per row
    (float32, u units) when ``return_tau``."""
    lib = _lib.load()
    _need(x, "x")
    if x.dim() < 1 or x.shape[-1] == 0:
        raise ValueError("x needs a non-empty last dimension")
    n = x.shape[-1]
    rows = x.numel() // n
    y = torch.empty_like(x) if out is None else out
    if out is not None:
        _need(out, "out", x.dtype)
        if out.shape != x.shape:
            raise ValueError("out must have the shape of x")
    tau = torch.empty(x.shape[:-1], dtype=torch.float32, device=x.device) if return_tau else None
    st = lib.entmax_rows(_p(x), _p(y), _dt(x), rows, n, float(alpha), int(n_iter), _p(tau), _stream(x.device))
    _lib.check(st, "entmax_rows")
    return (y, tau) if return_tau else y


def entmax_backward(y, dy, alpha=1.5, out=None):
    """Gradient of :func:`entmax` with respect to its scores, from its output ``y``
    and the cotangent ``dy`` (same shape and dtype); ``out`` may be ``dy``."""
    lib = _lib.load()
    _need(y, "y")
    _need(dy, "dy", y.dtype)
    if dy.shape != y.shape or y.dim() < 1 or y.shape[-1] == 0:
        raise ValueError("y and dy must have one shape with a non-empty last dimension")
    n = y.shape[-1]
    dx = torch.empty_like(y) if out is None else out
    if out is not None:
        _need(out, "out", y.dtype)
        if out.shape != y.shape:
            raise ValueError("out must have the shape of y")
    st = lib.entmax_rows_backward(_p(y), _p(dy), _p(dx), _dt(y), y.numel() // n, n, float(alpha), _stream(y.device))
    _lib.check(st, "entmax_rows_backward")
    return dx


class _EntmaxFn(torch.autograd.Function):
    @staticmethod
    def forward(ctx, x, alpha, n_iter):
        y = entmax(x, alpha=alpha, n_iter=n_iter)
        ctx.save_for_backward(y)
        ctx.alpha = alpha
        return y

    @staticmethod
    def backward(ctx, dy):
        (y,) = ctx.saved_tensors
        return entmax_backward(y, dy.contiguous().to(y.dtype), alpha=ctx.alpha), None, None


def entmax_fn(x, alpha=1.5, n_iter=10):
    """:func:`entmax` with a backward (torch autograd): the gradient runs in
    ``entmax_rows_backward``."""
    return _EntmaxFn.apply(x, alpha, n_iter)


def prefill(Q, K, V, head_cls, params: Params = Params(), with_bits=True, workspace=None, S=None):
    """Whole prefill: summaries of every chunk, routing, sparse attention.

    Returns (O, tau, active_bits, S, workspace); S is the float32 summary cache."""
    B, Hkv, N, d = K.shape
    n_c = -(-N // CHUNK)
    if S is None:
        S = torch.empty(B, Hkv, n_c, d, dtype=torch.float32, device=K.device)
    summarize(K, head_cls, S, n_tokens=N, chunk_begin=0, chunk_end=n_c if not params.causal else N // CHUNK,
              params=params)
    tau, bits, workspace = route(Q, K, head_cls, S, params, with_bits=with_bits, workspace=workspace)
    O = sparse_attn_prefill(Q, K, V, workspace, params)
    return O, tau, bits, S, workspace


def decode_step(q, Kc, Vc, head_cls, S, seqlens, params: Params = Params(), lengths=None, with_bits=True,
                workspace=None):
    """One decode step for new tokens already written at position seqlens[b] - 1.

    Routes against the summary cache, attends over the routed chunks, then
    appends the summary of every chunk this token completed. ``lengths`` holds
    the same lengths on the host (ints); it only selects which chunk indices to
    append. Without it the lengths are copied from ``seqlens`` to the host (one
    stream synchronisation), so no completed chunk is ever left out of the cache.
    Returns (O, tau, bits, workspace).
    """
    tau, bits, workspace = route(q, Kc, head_cls, S, params, seqlens=seqlens, with_bits=with_bits, workspace=workspace)
    O = sparse_attn_decode(q, Kc, Vc, seqlens, workspace, params)
    if lengths is None:
        lengths = seqlens.tolist()
    done = sorted({int(n) // CHUNK - 1 for n in lengths if int(n) % CHUNK == 0})
    for c in done:
        summarize(Kc, head_cls, S, seqlens=seqlens, chunk_begin=c, chunk_end=c + 1, params=params)
    return O, tau, bits, workspace
