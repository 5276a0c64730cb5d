"""Seeded synthetic inputs for the five workloads (no attention arithmetic here).

Both the HIP library's tests/benchmark and the CPU oracle receive tensors made by
these functions; this module only draws random numbers and plants the structures
each workload describes. Shapes follow the DashAttention README ("Usage": q/k/v
in [batch, heads, seq_len, head_dim], head_cls in [kv_heads, head_dim]) and the
AdaSplash README ("Usage" and "Key Features": q/k/v in the same layout, per-batch
lengths in ``varlen``).

Numbers are drawn as float32 N(0, 1) with ``torch.Generator(device)`` seeded by
the workload's seed, then rounded to bfloat16 (round to nearest even) unless the
workload is float32. The same seed on different devices gives different (but
equally valid) draws; every check hands the very same tensors to both sides.
"""

from __future__ import annotations

from dataclasses import dataclass, field
from typing import Optional

import torch

__all__ = [
    "Workload",
    "WORKLOADS",
    "dense_entmax_inputs",
    "routed_prefill_inputs",
    "decode_inputs",
]


@dataclass(frozen=True)
class Workload:
    name: str
    seed: int
    kind: str  # "entmax", "prefill", "decode"
    B: int
    Hq: int
    Hkv: int
    N: int
    d: int
    dtype: str  # "f32" or "bf16"
    alpha: float
    causal: bool = True
    chunk_size: int = 64
    estimate_diagonal: bool = True
    planted: Optional[str] = None  # "chunks", "needles" or None
    scale: float = 1.0
    varlen_range: Optional[tuple] = None
    extra: dict = field(default_factory=dict)


WORKLOADS = {
    "dense_entmax_128": Workload(
        "dense_entmax_128", 1001, "entmax", 1, 1, 1, 128, 64, "f32", 1.5, causal=True
    ),
    "routed_prefill_4k": Workload(
        "routed_prefill_4k", 1002, "prefill", 1, 32, 8, 4096, 128, "bf16", 1.5,
        causal=True, estimate_diagonal=True, planted="chunks",
    ),
    "routed_prefill_32k": Workload(
        "routed_prefill_32k", 1003, "prefill", 1, 32, 8, 32768, 128, "bf16", 1.5,
        causal=True, estimate_diagonal=False, planted="needles",
    ),
    # the 32K recipe at longer contexts (beyond the 32K headline, for the length ceiling)
    "routed_prefill_64k": Workload(
        "routed_prefill_64k", 1008, "prefill", 1, 32, 8, 65536, 128, "bf16", 1.5,
        causal=True, estimate_diagonal=False, planted="needles",
    ),
    "routed_prefill_128k": Workload(
        "routed_prefill_128k", 1009, "prefill", 1, 32, 8, 131072, 128, "bf16", 1.5,
        causal=True, estimate_diagonal=False, planted="needles",
    ),
    "decode_128k": Workload(
        "decode_128k", 1004, "decode", 16, 32, 8, 131072, 128, "bf16", 1.5,
        causal=True, estimate_diagonal=True,
    ),
    "varlen_entmax": Workload(
        "varlen_entmax", 1005, "entmax", 8, 16, 16, 8192, 64, "bf16", 2.0,
        causal=False, scale=2.0, varlen_range=(512, 8192),
    ),
    # row-wise entmax: B rows of N entries (Hq, Hkv, d unused)
    "entmax_rows_64k_1024": Workload(
        "entmax_rows_64k_1024", 1006, "entmax_rows", 65536, 1, 1, 1024, 1, "f32", 1.5, scale=2.0,
    ),
    "entmax_rows_128x256": Workload(
        "entmax_rows_128x256", 1007, "entmax_rows", 128, 1, 1, 256, 1, "f32", 1.5,
    ),
}


def _gen(seed: int, device) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return g


def _cast(x: torch.Tensor, dtype: str) -> torch.Tensor:
    return x.to(torch.bfloat16) if dtype == "bf16" else x.to(torch.float32)


def dense_entmax_inputs(B, H, N, d, seed, dtype="bf16", scale=1.0, varlen_range=None, device="cpu"):
    """Q, K, V ~ scale * N(0, 1) in [B, H, N, d]; optional lengths uniform in
    [lo, hi] (inclusive) as an int32 tensor on ``device``; N is then hi."""
    g = _gen(seed, device)
    lens = None
    if varlen_range is not None:
        lo, hi = varlen_range
        lens = torch.randint(lo, hi + 1, (B,), generator=g, device=device, dtype=torch.int64)
        lens = lens.to(torch.int32)
        N = hi
    q = torch.randn(B, H, N, d, generator=g, device=device) * scale
    k = torch.randn(B, H, N, d, generator=g, device=device) * scale
    v = torch.randn(B, H, N, d, generator=g, device=device) * scale
    return _cast(q, dtype), _cast(k, dtype), _cast(v, dtype), lens


def cotangent(shape, seed, dtype="bf16", device="cpu"):
    """A cotangent (upstream gradient) ~ N(0, 1) of the given shape."""
    g = _gen(seed, device)
    return _cast(torch.randn(*shape, generator=g, device=device), dtype)


def entmax_rows_inputs(rows, n, seed, dtype="f32", scale=1.0, device="cpu"):
    """Scores ~ scale * N(0, 1) in [rows, n]."""
    g = _gen(seed, device)
    return _cast(torch.randn(rows, n, generator=g, device=device) * scale, dtype)


def routed_prefill_inputs(B, Hq, Hkv, N, d, seed, planted=None, chunk_size=64, n_planted_chunks=20,
                          chunk_noise=0.1, needle_frac=0.01, needle_scale=4.0, dtype="bf16", device="cpu"):
    """Q [B,Hq,N,d], K/V [B,Hkv,N,d], head_cls [Hkv,d], all N(0, 1), plus planting.

    planted = "chunks": per (b, kv head), ``n_planted_chunks`` distinct complete
    chunks; every key of such a chunk is v_c + chunk_noise * eps (a
    high-similarity chunk). planted = "needles": per (b, kv head), a fraction
    ``needle_frac`` of token positions (round(N * frac)) whose keys are scaled by
    ``needle_scale``. Values are untouched.
    """
    g = _gen(seed, device)
    q = torch.randn(B, Hq, N, d, generator=g, device=device)
    k = torch.randn(B, Hkv, N, d, generator=g, device=device)
    v = torch.randn(B, Hkv, N, d, generator=g, device=device)
    cls = torch.randn(Hkv, d, generator=g, device=device)
    if planted == "chunks":
        n_complete = N // chunk_size
        m = min(n_planted_chunks, n_complete)
        for b in range(B):
            for h in range(Hkv):
                ids = torch.randperm(n_complete, generator=g, device=device)[:m]
                for c in ids.tolist():
                    vc = torch.randn(d, generator=g, device=device)
                    eps = torch.randn(chunk_size, d, generator=g, device=device)
                    k[b, h, c * chunk_size:(c + 1) * chunk_size] = vc[None, :] + chunk_noise * eps
    elif planted == "needles":
        m = int(round(N * needle_frac))
        for b in range(B):
            for h in range(Hkv):
                pos = torch.randperm(N, generator=g, device=device)[:m]
                k[b, h, pos] *= needle_scale
    elif planted is not None:
        raise ValueError(planted)
    return _cast(q, dtype), _cast(k, dtype), _cast(v, dtype), _cast(cls, dtype)


def decode_inputs(B, Hq, Hkv, L, d, seed, dtype="bf16", device="cpu", Lmax=None):
    """One decode step: caches K/V [B,Hkv,Lmax,d] holding L cached tokens plus the
    new token at position L (so seqlens = L + 1), the new queries q [B,Hq,1,d] and
    head_cls [Hkv,d]; all N(0, 1). Slots beyond the sequence are zero."""
    Lmax = Lmax if Lmax is not None else L + 1
    g = _gen(seed, device)
    kc = torch.zeros(B, Hkv, Lmax, d, device=device, dtype=torch.bfloat16 if dtype == "bf16" else torch.float32)
    vc = torch.zeros_like(kc)
    for b in range(B):  # per batch entry, to bound float32 temporaries
        kc[b, :, :L + 1] = _cast(torch.randn(Hkv, L + 1, d, generator=g, device=device), dtype)
        vc[b, :, :L + 1] = _cast(torch.randn(Hkv, L + 1, d, generator=g, device=device), dtype)
    q = _cast(torch.randn(B, Hq, 1, d, generator=g, device=device), dtype)
    cls = _cast(torch.randn(Hkv, d, generator=g, device=device), dtype)
    seqlens = torch.full((B,), L + 1, dtype=torch.int32, device=device)
    return q, kc, vc, cls, seqlens
