"""Benchmark of the hierarchical adaptive sparse attention hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]

One step is the whole prefill of the 32K-token workload: chunk summaries,
routing (scores, alpha-entmax tau, routed lists and priors) and sparse
attention, 32 query heads over 8 KV heads, head_dim 128, bf16, chunk 64, causal,
alpha 1.5, own chunk always attended, 1% needle keys scaled by 4 (synthetic,
seeded). ``value`` is tokens/s of that step. The same run also times one decode
step at 131072 cached tokens for a batch of 16 (routing against the summary
cache plus split-KV attention over the routed chunks) and the varlen dense
alpha-entmax attention workload; their figures are reported under "decode" and
"entmax". Inputs are resident in HBM before timing starts. Kernel durations
for the roofline come from HIP events recorded on the launch stream.

Prints one JSON line on stdout.
"""

from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

from adaptive_sparse_long_amd import _lib, api  # noqa: E402
from adaptive_sparse_long_amd.workloads import (  # noqa: E402
    WORKLOADS,
    decode_inputs,
    cotangent,
    dense_entmax_inputs,
    entmax_rows_inputs,
    routed_prefill_inputs,
)

PEAK_BF16_TFLOPS = 2500.0  # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0      # MI355X HBM3E
C = 64
FLUSH_BYTES = 512 * 1024 * 1024  # twice the Infinity Cache


class CacheEvictor:
    """Evicts the 256 MB Infinity Cache between timed steps by reading a 512 MB
    buffer (a sum): the cache is left holding clean lines of that buffer, as
    after another kernel's reads. (Writing the buffer instead would leave dirty
    lines whose write-back the next kernel would pay.)"""

    def __init__(self, dev):
        self.buf = torch.ones(FLUSH_BYTES // 4, dtype=torch.float32, device=dev)

    def __call__(self):
        self.buf.sum()
CSRC = os.path.join(ROOT, "adaptive_sparse_long_amd", "csrc")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")
# Sources each kernel's code depends on (a changed source voids its measured traffic).
KERNEL_SOURCES = {
    "k_route_fast": ["route.hip", "kernels.hpp", "cdna4.hpp", "tau_solve.hpp"],
    "k_prefill_cm": ["sparse_prefill.hip", "kernels.hpp", "cdna4.hpp", "tau_solve.hpp"],
    "k_sparse_decode": ["sparse_decode.hip", "kernels.hpp", "cdna4.hpp"],
    "k_entmax_buf": ["entmax_attn.hip", "kernels.hpp", "cdna4.hpp", "tau_solve.hpp"],
    "k_entmax_rows": ["entmax_rows.hip", "kernels.hpp", "cdna4.hpp", "tau_solve.hpp"],
    "k_entmax_rows_bwd": ["entmax_rows.hip", "kernels.hpp", "cdna4.hpp", "tau_solve.hpp"],
    "k_prefill_merge": ["sparse_prefill.hip", "kernels.hpp", "cdna4.hpp", "tau_solve.hpp"],
    "k_cm_scatter": ["sparse_prefill.hip", "kernels.hpp", "cdna4.hpp", "tau_solve.hpp"],
    "k_cm_plan": ["sparse_prefill.hip", "kernels.hpp", "cdna4.hpp", "tau_solve.hpp"],
    "k_sparse_prefill": ["sparse_prefill.hip", "kernels.hpp", "cdna4.hpp", "tau_solve.hpp"],
    "k_summarize_bwd": ["summarize.hip", "kernels.hpp", "cdna4.hpp"],
    "k_entmax_bwd_dq": ["entmax_attn_bwd.hip", "bwd_common.hpp", "kernels.hpp", "cdna4.hpp", "tau_solve.hpp"],
    "k_entmax_bwd_dkdv": ["entmax_attn_bwd.hip", "bwd_common.hpp", "kernels.hpp", "cdna4.hpp", "tau_solve.hpp"],
}
# the kernels of one dash_sparse_attn_prefill call
ATTN_KERNELS = ["k_cm_plan", "k_cm_scatter", "k_prefill_cm", "k_prefill_merge", "k_sparse_prefill"]


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def popcount32(x: torch.Tensor) -> torch.Tensor:
    x = x.to(torch.int64) & 0xFFFFFFFF
    x = x - ((x >> 1) & 0x55555555)
    x = (x & 0x33333333) + ((x >> 2) & 0x33333333)
    x = (x + (x >> 4)) & 0x0F0F0F0F
    return ((x * 0x01010101) & 0xFFFFFFFF) >> 24


def source_sha(kernel: str) -> str:
    import hashlib

    h = hashlib.sha256()
    for f in KERNEL_SOURCES[kernel]:
        with open(os.path.join(CSRC, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def measured_traffic(kernel: str, key: str = "hbm_bytes_per_launch"):
    """HBM bytes per launch from the committed PMC profile (FETCH_SIZE + WRITE_SIZE,
    each scaled by the plain-copy calibration; key "hbm_bytes_gather_scaled": the
    reads scaled by the random-row gather calibration instead), or None if the
    kernel source has changed since the counters were taken."""
    try:
        with open(TRAFFIC_FILE) as f:
            rec = json.load(f)["kernels"][kernel]
    except (OSError, KeyError, ValueError):
        return None
    if rec.get("source_sha") != source_sha(kernel) or key not in rec:
        return None
    return float(rec[key])


def _sum_or_none(parts):
    return None if any(p is None for p in parts) else float(sum(parts))


def attention_traffic(key: str = "hbm_bytes_per_launch"):
    """Measured HBM bytes of one dash_sparse_attn_prefill call (its kernels summed),
    or None if any of them changed since the counters were taken."""
    parts = [measured_traffic(k, key) for k in ATTN_KERNELS]
    return None if any(p is None for p in parts) else float(sum(parts))


def calibrate_copy(nbytes=1 << 30, reps=3):
    """A plain device-to-device copy of known size, for scaling the PMC byte counters."""
    src = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    src.fill_(1)
    torch.cuda.synchronize()
    for _ in range(reps):
        dst.copy_(src)
    torch.cuda.synchronize()
    log(f"calibration copy: {reps} x {nbytes} bytes")
    del src, dst
    calibrate_gather()


def calibrate_gather(rows=1 << 22, table_rows=1 << 23, reps=3):
    """A gather of known size with the query gathers' access pattern: `rows`
    distinct 256-byte rows (128 bf16) in random order out of a 2 GiB table (far
    larger than the 256 MB Infinity Cache, so nothing is re-read), for checking
    that the copy's scaling of the PMC byte counters holds for gathers."""
    g = torch.Generator(device="cuda")
    g.manual_seed(99)
    table = torch.ones(table_rows, 128, dtype=torch.bfloat16, device="cuda")
    idx = torch.randperm(table_rows, generator=g, device="cuda")[:rows].contiguous()
    torch.cuda.synchronize()
    for _ in range(reps):
        torch.index_select(table, 0, idx)
    torch.cuda.synchronize()
    log(f"calibration gather: {reps} x {rows} rows of 256 bytes (+ {rows * 8} bytes of indices)")


class Timer:
    """HIP events on the current (launch) stream."""

    def __init__(self):
        self.pairs = []

    def start(self):
        e = torch.cuda.Event(enable_timing=True)
        e.record()
        return e

    def stop(self, e0):
        e1 = torch.cuda.Event(enable_timing=True)
        e1.record()
        self.pairs.append((e0, e1))

    def mean_ms(self):
        torch.cuda.synchronize()
        return float(np.mean([a.elapsed_time(b) for a, b in self.pairs])) if self.pairs else float("nan")


# --------------------------------------------------------------------------- prefill
def prefill_work(bits: torch.Tensor, N: int, d: int):
    """Work counts of one prefill from the routed-chunk bits:
    alg: attention flops, 4 d per (row, visible key of a routed chunk);
    pair: MFMA flops of the chunk-major pass, 4 d x 64 keys per (row, routed
      chunk) pair (the own chunk is masked inside its 64 keys);
    dense: causal dense attention flops;
    scores: routing scores, one per (row, complete past chunk) (causal);
    per_row: routed chunks per row."""
    B, Hq, _, W = bits.shape
    n_slots = -(-N // C)
    c = torch.arange(n_slots, device=bits.device)
    on = ((bits[..., c // 32] >> (c % 32)) & 1).bool()  # [B, Hq, N, n_slots]
    i = torch.arange(N, device=bits.device)
    vis = torch.clamp(i[:, None] + 1 - c[None, :] * C, 0, C)  # causal visible tokens per (row, chunk)
    alg = 4.0 * d * float((on * vis).sum())
    pairs = float(on.sum())
    pair = 4.0 * d * C * pairs
    dense = 2.0 * 2.0 * d * (N * (N + 1) / 2.0) * B * Hq
    scores = float(B * Hq * sum(r // C for r in range(N)))
    return alg, pair, dense, scores, pairs / (B * Hq * N)


def route_alg_bytes(w, pairs):
    """Algorithmic HBM bytes of one prefill routing call: Q (bf16), the keys the
    own-chunk estimate reads (bf16, once per KV head), the float32 summaries in,
    tau per row out, and per attended (row, chunk) pair its chunk and weight
    (8 bytes)."""
    n_c = w.N // C
    return float(w.B * w.Hq * w.N * w.d * 2 + w.B * w.Hkv * w.N * w.d * 2 + w.B * w.Hkv * n_c * w.d * 4
                 + w.B * w.Hq * w.N * 4 + pairs * 8)


def bench_prefill(w, steps, warmup, summary_backward=True):
    dev = torch.device("cuda")
    Q, K, V, cls = routed_prefill_inputs(w.B, w.Hq, w.Hkv, w.N, w.d, w.seed, planted=w.planted, device=dev)
    p = api.Params(alpha=w.alpha, causal=w.causal, estimate_diagonal=w.estimate_diagonal)
    n_c = -(-w.N // C)
    S = torch.empty(w.B, w.Hkv, n_c, w.d, dtype=torch.float32, device=dev)
    ws = torch.empty(api.workspace_size(w.B, w.Hq, w.Hkv, w.N, w.N, w.d, False, p), dtype=torch.uint8, device=dev)
    O = torch.empty_like(Q)
    n_sum = w.N // C if w.causal else n_c
    t_sum, t_route, t_attn = Timer(), Timer(), Timer()
    # the Infinity Cache (256 MB) is evicted before every step, outside the timed events
    flush = CacheEvictor(dev)

    t_step = Timer()

    # timed=True: events around each part; timed="step": events around the whole
    # step only (no instrumentation between its calls)
    def step(timed):
        flush()
        parts = timed is True
        e0 = t_step.start() if timed == "step" else None
        e = t_sum.start() if parts else None
        api.summarize(K, cls, S, n_tokens=w.N, chunk_begin=0, chunk_end=n_sum, params=p)
        if parts:
            t_sum.stop(e)
            e = t_route.start()
        tau, bits, _ = api.route(Q, K, cls, S, p, with_bits=False, workspace=ws)
        if parts:
            t_route.stop(e)
            e = t_attn.start()
        api.sparse_attn_prefill(Q, K, V, ws, p, out=O)
        if parts:
            t_attn.stop(e)
        if e0 is not None:
            t_step.stop(e0)

    for _ in range(warmup):
        step(False)
    for _ in range(steps):
        step(True)
    for _ in range(steps):
        step("step")
    torch.cuda.synchronize()
    del flush
    # work counts (outside the timed region)
    _, bits, _ = api.route(Q, K, cls, S, p, with_bits=True, workspace=ws)
    counters = api.prefill_counters(ws, w.B, w.Hq, w.Hkv, w.N, w.d, p)
    alg, pair, dense, scores, per_row = prefill_work(bits, w.N, w.d)
    res = {
        "workspace_GB": ws.numel() / 1e9,
        "counters": counters,
        "ms_step": t_step.mean_ms(),
        "ms_summarize": t_sum.mean_ms(),
        "ms_route": t_route.mean_ms(),
        "ms_attention": t_attn.mean_ms(),
        "alg_flops": alg,
        "pair_flops": pair,
        "dense_causal_flops": dense,
        "route_scores": scores,
        "routed_chunks_per_row": per_row,
        "pairs": per_row * w.B * w.Hq * w.N,
    }
    if not summary_backward:
        del Q, K, V, S, ws, O, bits
        torch.cuda.empty_cache()
        return res
    # summary backward on the same keys (gradients of the summaries for a random
    # cotangent into dK and head_cls), outside the step
    dS = cotangent((w.B, w.Hkv, n_c, w.d), w.seed + 700, dtype="f32", device=dev)
    bufs = (torch.zeros(w.B, w.Hkv, w.N, w.d, dtype=torch.float32, device=dev),
            torch.empty(w.Hkv, w.d, dtype=torch.float32, device=dev),
            torch.empty(w.B, w.Hkv, n_sum, w.d, dtype=torch.float32, device=dev))
    t_sb = Timer()
    for it in range(warmup + steps):
        e = t_sb.start() if it >= warmup else None
        api.summarize_backward(K, cls, dS, n_tokens=w.N, chunk_begin=0, chunk_end=n_sum, params=p, out=bufs)
        if it >= warmup:
            t_sb.stop(e)
    ms_sb = t_sb.mean_ms()
    # algorithmic bytes: K read (bf16), dK written (fp32), dS read, dcls partials written and read
    sb_bytes = float(w.B * w.Hkv * n_sum * C * w.d * (2 + 4) + w.B * w.Hkv * n_sum * w.d * 4 * 3)
    del dS, bufs
    res["summary_backward"] = {"us": ms_sb * 1e3, "bytes_per_launch": sb_bytes,
                               "GBps": sb_bytes / (ms_sb / 1e3) / 1e9,
                               "frac": sb_bytes / (ms_sb / 1e3) / 1e9 / PEAK_HBM_GBS}
    del Q, K, V, S, ws, O, bits
    torch.cuda.empty_cache()
    return res


def bench_dash_backward(w, steps, warmup):
    """dash_sparse_attn_prefill_backward on a prefill workload: gradients into Q,
    K, V and head_cls for a random cotangent, timed with HIP events per call."""
    dev = torch.device("cuda")
    Q, K, V, cls = routed_prefill_inputs(w.B, w.Hq, w.Hkv, w.N, w.d, w.seed, planted=w.planted, device=dev)
    p = api.Params(alpha=w.alpha, causal=w.causal, estimate_diagonal=w.estimate_diagonal)
    _, tau, bits, S, ws = api.prefill(Q, K, V, cls, p)
    alg_fwd = prefill_work(bits, w.N, w.d)[0]
    del ws
    torch.cuda.empty_cache()
    dO = cotangent(tuple(Q.shape), w.seed + 800, dtype="bf16", device=dev)
    need = int(_lib.load().dash_backward_workspace_size(w.B, w.Hq, w.Hkv, w.N, w.N, w.d, p.c()))
    wsb = torch.empty(need, dtype=torch.uint8, device=dev)
    flush = CacheEvictor(dev)
    t = Timer()
    for it in range(warmup + steps):
        flush()
        e = t.start() if it >= warmup else None
        api.prefill_backward(Q, K, V, cls, S, dO, tau, bits, p, workspace=wsb)
        if it >= warmup:
            t.stop(e)
    torch.cuda.synchronize()
    ms = t.mean_ms()
    # five products per visible routed (row, key) entry: S and dP recomputed, dV, dQ, dK
    alg = alg_fwd * 2.5
    del Q, K, V, cls, tau, bits, S, dO, wsb, flush
    torch.cuda.empty_cache()
    return {"workload": w.name, "ms": ms, "alg_flops": alg, "alg_tflops": alg / (ms / 1e3) / 1e12,
            "alg_frac": alg / (ms / 1e3) / 1e12 / PEAK_BF16_TFLOPS, "workspace_GB": need / 1e9}


# --------------------------------------------------------------------------- decode
def bench_decode(w, steps, warmup):
    dev = torch.device("cuda")
    q, Kc, Vc, cls, seqlens = decode_inputs(w.B, w.Hq, w.Hkv, w.N, w.d, w.seed, device=dev)
    p = api.Params(alpha=w.alpha, estimate_diagonal=w.estimate_diagonal)
    Lmax = Kc.shape[2]
    S = torch.zeros(w.B, w.Hkv, -(-Lmax // C), w.d, dtype=torch.float32, device=dev)
    api.summarize(Kc, cls, S, seqlens=seqlens, chunk_begin=0, chunk_end=Lmax // C, params=p)
    ws = torch.empty(api.workspace_size(w.B, w.Hq, w.Hkv, 1, Lmax, w.d, True, p), dtype=torch.uint8, device=dev)
    O = torch.empty_like(q)
    lengths = [int(x) for x in seqlens.cpu()]
    # Infinity Cache (256 MB) holds the whole summary cache; evict it between steps
    flush = CacheEvictor(dev)
    t_route, t_attn, t_step = Timer(), Timer(), Timer()

    # timed=True: events around the routing and the attention (the parts);
    # timed="step": events around the whole step only, so that the step time
    # carries no instrumentation between its kernels
    def step(timed):
        parts = timed is True
        e = t_step.start() if timed == "step" else None
        e1 = t_route.start() if parts else None
        api.route(q, Kc, cls, S, p, seqlens=seqlens, with_bits=False, workspace=ws)
        if parts:
            t_route.stop(e1)
            e1 = t_attn.start()
        api.sparse_attn_decode(q, Kc, Vc, seqlens, ws, p, out=O)
        if parts:
            t_attn.stop(e1)
        done = sorted({n // C - 1 for n in lengths if n % C == 0})
        for c in done:
            api.summarize(Kc, cls, S, seqlens=seqlens, chunk_begin=c, chunk_end=c + 1, params=p)
        if e is not None:
            t_step.stop(e)

    for _ in range(warmup):
        flush()
        step(False)
    for _ in range(steps):
        flush()
        step(True)
    for _ in range(steps):
        flush()
        step("step")
    torch.cuda.synchronize()
    # chunks each (b, kv head) group read: union of its g heads' routed chunks
    _, bits, _ = api.route(q, Kc, cls, S, p, seqlens=seqlens, with_bits=True, workspace=ws)
    g = w.Hq // w.Hkv
    union = bits.view(w.B, w.Hkv, g, -1)
    acc = union[:, :, 0]
    for j in range(1, g):
        acc = acc | union[:, :, j]
    counts = popcount32(acc).sum(dim=-1).flatten().cpu().numpy()
    n_keys = w.N + 1
    kv_bytes = 0.0
    last_chunk = (n_keys - 1) // C
    for cnt in counts:
        # every listed chunk is full except the own (last) chunk, which has n_keys - last_chunk*C tokens
        kv_bytes += ((cnt - 1) * C + (n_keys - last_chunk * C)) * w.d * 2 * 2
    s_bytes = w.B * w.Hkv * (n_keys - 1) // C * w.d * 4
    res = {
        "us_per_step": t_step.mean_ms() * 1e3,
        "us_route": t_route.mean_ms() * 1e3,
        "us_attention": t_attn.mean_ms() * 1e3,
        "kv_bytes": kv_bytes,
        "summary_bytes": float(s_bytes),
        "dense_kv_bytes": float(w.B * w.Hkv * n_keys * w.d * 2 * 2),
        "union_chunk_frac": float(np.mean(counts)) / (last_chunk + 1),
    }
    del q, Kc, Vc, S, ws, O, flush
    torch.cuda.empty_cache()
    return res


# --------------------------------------------------------------------------- entmax
def bench_entmax(w, steps, warmup):
    dev = torch.device("cuda")
    q, k, v, lens = dense_entmax_inputs(w.B, w.Hq, w.N, w.d, w.seed, dtype=w.dtype, scale=w.scale,
                                        varlen_range=w.varlen_range, device=dev)
    t = Timer()
    for _ in range(warmup):
        api.entmax_attn(q, k, v, alpha=w.alpha, causal=w.causal, varlen=lens)
    for _ in range(steps):
        e = t.start()
        O, tau, mask = api.entmax_attn(q, k, v, alpha=w.alpha, causal=w.causal, varlen=lens)
        t.stop(e)
    ms = t.mean_ms()
    L = lens.cpu().numpy().astype(np.float64)
    qk_flops = float(np.sum(2.0 * L * L * w.d) * w.Hq)
    nT = -(-w.N // 64)
    c = torch.arange(nT, device=dev)
    on = ((mask[..., c // 32] >> (c % 32)) & 1).bool()
    tiles_on = float(on.sum())
    tiles_all = float(np.sum(np.ceil(L / 64) ** 2) * w.Hq)
    # backward (dQ, dK, dV for a random cotangent), skipping the mask's empty tiles
    dO = cotangent(q.shape, w.seed + 500, dtype=w.dtype, device=dev)
    tb = Timer()
    for _ in range(warmup):
        api.entmax_attn_backward(q, k, v, dO, tau, mask, alpha=w.alpha, causal=w.causal, varlen=lens)
    for _ in range(steps):
        e = tb.start()
        api.entmax_attn_backward(q, k, v, dO, tau, mask, alpha=w.alpha, causal=w.causal, varlen=lens)
        tb.stop(e)
    ms_b = tb.mean_ms()
    # algorithmic backward work: five products (S, dP, dV, dK, dQ) of 2 d flops per
    # allowed (row, key) entry of the tiles the mask keeps
    rows_in = torch.clamp(lens.to(dev).long()[:, None] - 64 * c[None, :], 0, 64).double()  # [B, nT]
    ent = (on.double() * rows_in[:, None, :, None] * rows_in[:, None, None, :]).sum()
    bwd_flops = float(ent) * 5 * 2 * w.d
    return {
        "ms": ms,
        "tokens_per_s": float(L.sum()) / (ms / 1e3),
        "qk_flops": qk_flops,
        "tflops_qk_pass": qk_flops / (ms / 1e3) / 1e12,
        "nonnull_tile_frac": tiles_on / tiles_all,
        "backward": {"ms": ms_b, "alg_flops": bwd_flops, "tflops": bwd_flops / (ms_b / 1e3) / 1e12,
                     "frac": bwd_flops / (ms_b / 1e3) / 1e12 / PEAK_BF16_TFLOPS,
                     "traffic": _sum_or_none([measured_traffic("k_entmax_bwd_dq"),
                                              measured_traffic("k_entmax_bwd_dkdv")])},
    }


def bench_entmax_small(w, steps, warmup):
    """The 128-token float32 dense entmax attention: HIP-event time per call
    (the whole entmax_attn call, launch included) over many back-to-back calls."""
    q, k, v, _ = dense_entmax_inputs(w.B, w.Hq, w.N, w.d, w.seed, dtype=w.dtype, device="cuda")
    for _ in range(warmup):
        api.entmax_attn(q, k, v, alpha=w.alpha, causal=w.causal)
    reps = max(steps, 50)
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        api.entmax_attn(q, k, v, alpha=w.alpha, causal=w.causal)
    e1.record()
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) / reps * 1e3
    flops = 2.0 * w.d * w.N * (w.N + 1) / 2.0 * 2 * w.B * w.Hq  # QK^T and PV over the causal triangle
    return {"workload": w.name, "us_per_call": us, "calls": reps, "causal_flops": flops}


def bench_entmax_rows(w, steps, warmup):
    """Row-wise entmax over w.B rows of w.N entries: HIP-event time per call and
    the algorithmic HBM bytes (every entry read once and written once, tau out)."""
    x = entmax_rows_inputs(w.B, w.N, w.seed, dtype=w.dtype, scale=w.scale, device="cuda")
    y = torch.empty_like(x)
    t = Timer()
    for _ in range(warmup):
        api.entmax(x, alpha=w.alpha, out=y)
    for _ in range(steps):
        e = t.start()
        api.entmax(x, alpha=w.alpha, out=y)
        t.stop(e)
    ms = t.mean_ms()
    nbytes = float(2 * x.numel() * x.element_size())
    # backward: Y and dY read, dX written
    dy = entmax_rows_inputs(w.B, w.N, w.seed + 100, dtype=w.dtype, device="cuda")
    dx = torch.empty_like(x)
    tb = Timer()
    for _ in range(warmup):
        api.entmax_backward(y, dy, alpha=w.alpha, out=dx)
    for _ in range(steps):
        e = tb.start()
        api.entmax_backward(y, dy, alpha=w.alpha, out=dx)
        tb.stop(e)
    ms_b = tb.mean_ms()
    return {"rows": w.B, "n": w.N, "us": ms * 1e3, "bytes_per_launch": nbytes,
            "GBps": nbytes / (ms / 1e3) / 1e9, "us_backward": ms_b * 1e3,
            "GBps_backward": 1.5 * nbytes / (ms_b / 1e3) / 1e9}


def sparsity_report(w, alphas=(1.333, 1.5, 2.0), scalings=(0.5, 1.0, 2.0, 4.0), depth_bins=8):
    """Measured routing sparsity on the needle workload: for each (alpha,
    scaling_factor), the attended chunks per row and their fraction of the row's
    candidates (its complete past chunks plus its own), overall, per query head
    (min / median / max) and per depth bin (query position in N / depth_bins)."""
    Q, K, V, cls = routed_prefill_inputs(w.B, w.Hq, w.Hkv, w.N, w.d, w.seed, planted=w.planted, device="cuda")
    del V
    n_c = -(-w.N // C)
    S = torch.empty(w.B, w.Hkv, n_c, w.d, dtype=torch.float32, device="cuda")
    ws = None
    pos = torch.arange(w.N, device="cuda")
    cand = (pos // C + 1).to(torch.float64)  # causal: complete past chunks + own
    rows = []
    for alpha in alphas:
        for sf in scalings:
            p = api.Params(alpha=alpha, scaling_factor=sf, causal=True, estimate_diagonal=w.estimate_diagonal)
            api.summarize(K, cls, S, n_tokens=w.N, chunk_begin=0, chunk_end=w.N // C, params=p)
            _, bits, ws = api.route(Q, K, cls, S, p, with_bits=True, workspace=ws)
            act = popcount32(bits).sum(dim=-1).to(torch.float64)[0]  # [Hq, N]
            frac = act / cand[None, :]
            head = frac.mean(dim=1).cpu().numpy()
            depth = frac.view(w.Hq, depth_bins, -1).mean(dim=(0, 2)).cpu().numpy()
            rows.append({
                "alpha": alpha, "scaling_factor": sf,
                "active_chunks_per_row": float(act.mean()),
                "active_frac": float(frac.mean()),
                "active_frac_by_head": [float(head.min()), float(np.median(head)), float(head.max())],
                "active_frac_by_depth": [float(x) for x in depth],
            })
            log(f"sparsity alpha={alpha} sf={sf}: {rows[-1]['active_chunks_per_row']:.2f} chunks/row")
    return {"workload": w.name, "depth_bins": depth_bins, "rows": rows}


def union_density_report(names=("routed_prefill_4k", "routed_prefill_32k"), block_rows=(16, 32, 64, 128),
                         thresholds=(0.25, 0.5, 0.75), depth_bins=8):
    """How dense the routed past chunks of a block of consecutive rows of one
    query head are: for blocks of R rows, the chunk union of the block (what a
    row-major tile loop executes, R x 64 keys per chunk of the union) against the
    rows' own routed past chunks (the chunk-major pairs). Per R: executed over
    routed pairs overall and per depth bin, and the share of routed pairs (and of
    blocks) in blocks at least `threshold` dense."""
    out = []
    for name in names:
        w = WORKLOADS[name]
        Q, K, V, cls = routed_prefill_inputs(w.B, w.Hq, w.Hkv, w.N, w.d, w.seed, planted=w.planted, device="cuda")
        del V
        p = api.Params(alpha=w.alpha, causal=w.causal, estimate_diagonal=w.estimate_diagonal)
        S = torch.empty(w.B, w.Hkv, -(-w.N // C), w.d, dtype=torch.float32, device="cuda")
        api.summarize(K, cls, S, n_tokens=w.N, chunk_begin=0, chunk_end=w.N // C, params=p)
        _, bits, ws = api.route(Q, K, cls, S, p, with_bits=True)
        del ws, Q, K
        B, H, N, W = bits.shape
        # past chunks only: clear each row's own chunk
        rows = torch.arange(N, device="cuda")
        own = torch.zeros(N, W, dtype=torch.int64, device="cuda")
        own[rows, (rows // C) // 32] = 1 << ((rows // C) % 32)
        past = (bits.to(torch.int64) & 0xFFFFFFFF) & ~own  # [B, H, N, W], 32-bit words in int64
        cnt = popcount32(past).sum(-1)  # [B, H, N]
        total = float(cnt.sum())
        rec = {"workload": name, "past_pairs": total, "rows": B * H * N, "past_chunks_per_row": total / (B * H * N),
               "blocks": []}
        for R in block_rows:
            u = past.view(B, H, N // R, R, W)
            while u.shape[3] > 1:
                h = u.shape[3] // 2
                u = u[:, :, :, :h] | u[:, :, :, h:2 * h]
            union = popcount32(u[:, :, :, 0]).sum(-1)  # [B, H, N/R]
            s = cnt.view(B, H, N // R, R).sum(-1)
            eff = s.double() / (R * union.clamp(min=1)).double()
            nb = N // R
            entry = {"rows_per_block": R, "executed_over_pairs": float((union * R).sum()) / total,
                     "executed_over_pairs_by_depth": [
                         float((union[:, :, k * nb // depth_bins:(k + 1) * nb // depth_bins] * R).sum())
                         / max(1.0, float(s[:, :, k * nb // depth_bins:(k + 1) * nb // depth_bins].sum()))
                         for k in range(depth_bins)],
                     "dense_blocks": []}
            for th in thresholds:
                sel = eff >= th
                ps = float(s[sel].sum())
                entry["dense_blocks"].append({"density_at_least": th, "pair_share": ps / total,
                                              "block_share": float(sel.double().mean()),
                                              "executed_over_pairs": float((union[sel] * R).sum()) / max(1.0, ps)})
            rec["blocks"].append(entry)
            log(f"union density {name} R={R}: executed/pairs {entry['executed_over_pairs']:.2f}")
        out.append(rec)
        del bits, past, cnt
    return {"depth_bins": depth_bins, "workloads": out}


# --------------------------------------------------------------------------- CPU oracle
def cpu_baseline(w, budget_s=20.0):
    """The float64 oracle on host cores, on a random sample of query rows of the
    prefill workload (all of their routing, and their attention), scaled to
    tokens/s: one token is one row in each of the Hq query heads."""
    import oracle

    try:
        from threadpoolctl import threadpool_info

        threads = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    except Exception:  # pragma: no cover
        threads = os.cpu_count() or 1
    Q, K, V, cls = routed_prefill_inputs(w.B, w.Hq, w.Hkv, w.N, w.d, w.seed, planted=w.planted, device="cpu")
    op = oracle.DashParams(chunk_size=C, alpha=w.alpha, causal=w.causal, estimate_diagonal=w.estimate_diagonal)
    rng = np.random.default_rng(w.seed)
    g = w.Hq // w.Hkv
    rows_done = 0
    t0 = time.perf_counter()
    summ_cache = {}
    while time.perf_counter() - t0 < budget_s:
        h = int(rng.integers(0, w.Hq))
        hk = h // g
        if hk not in summ_cache:
            keys = K[0, hk].double().numpy()
            summ_cache[hk] = (keys, V[0, hk].double().numpy(), cls[hk].double().numpy(),
                              oracle.chunk_summaries(keys, cls[hk].double().numpy(), C, w.N))
        keys, vals, clsv, summ = summ_cache[hk]
        rows = np.sort(rng.integers(0, w.N, 16))
        oracle.dash_rows(Q[0, h, rows].double().numpy(), rows, keys, vals, clsv, w.N, op, summ)
        rows_done += rows.size
    el = time.perf_counter() - t0
    return {
        "value": (rows_done / w.Hq) / el,
        "unit": "tokens/s",
        "cores": int(threads),
        "kind": "oracle",
        "sample": f"{rows_done} random query rows (uniform positions, random heads) of the 32K prefill "
                  f"workload incl. summaries of the KV heads touched, {el:.1f} s; tokens/s = rows / {w.Hq} / s",
    }


def _blas_info():
    try:
        from threadpoolctl import threadpool_info

        info = threadpool_info()
        return [{k: i.get(k) for k in ("internal_api", "version", "num_threads", "threading_layer")} for i in info]
    except Exception:  # pragma: no cover
        return []


def oracle_timings():
    """The float64 oracle on the other workloads (host cores; reported beside the
    GPU figures, not targets): the 128-token entmax attention and the 4K routed
    prefill in full, the varlen entmax workload and the batch-16 decode step on
    bounded samples scaled to the whole workload (the sample is stated)."""
    import oracle

    out = {"numpy": np.__version__, "blas": _blas_info(), "host_cpus": os.cpu_count()}
    # 1: dense entmax, 128 tokens, float32 inputs
    w1 = WORKLOADS["dense_entmax_128"]
    q, k, v, _ = dense_entmax_inputs(w1.B, w1.Hq, w1.N, w1.d, w1.seed, dtype=w1.dtype, device="cpu")
    t0 = time.perf_counter()
    reps = 20
    for _ in range(reps):
        oracle.entmax_attention(q.double().numpy(), k.double().numpy(), v.double().numpy(), w1.alpha, w1.causal)
    out["dense_entmax_128"] = {"us_per_call": (time.perf_counter() - t0) / reps * 1e6, "sample": "full, 20 calls"}
    # 2: routed prefill 4K, every head
    w2 = WORKLOADS["routed_prefill_4k"]
    Q, K, V, cls = routed_prefill_inputs(w2.B, w2.Hq, w2.Hkv, w2.N, w2.d, w2.seed, planted=w2.planted, device="cpu")
    op = oracle.DashParams(chunk_size=C, alpha=w2.alpha, causal=w2.causal, estimate_diagonal=w2.estimate_diagonal)
    t0 = time.perf_counter()
    oracle.dash_prefill(Q.double().numpy(), K.double().numpy(), V.double().numpy(), cls.double().numpy(), op)
    el = time.perf_counter() - t0
    out["routed_prefill_4k"] = {"s": el, "tokens_per_s": w2.N / el, "sample": "full (32 heads, 4096 rows)"}
    del Q, K, V, cls
    # 5: varlen entmax, one sampled block of 64 rows in each of 8 (b, h) pairs, scaled by rows
    w5 = WORKLOADS["varlen_entmax"]
    q, k, v, lens = dense_entmax_inputs(w5.B, w5.Hq, w5.N, w5.d, w5.seed, dtype=w5.dtype, scale=w5.scale,
                                        varlen_range=w5.varlen_range, device="cpu")
    rng = np.random.default_rng(w5.seed)
    L = lens.numpy()
    rows_done, t0 = 0, time.perf_counter()
    for _ in range(8):
        b, h = int(rng.integers(0, w5.B)), int(rng.integers(0, w5.Hq))
        r0 = int(rng.integers(0, max(1, L[b] - 64)))
        pos = np.arange(r0, min(L[b], r0 + 64))
        oracle.entmax_attention_rows(q[b, h, pos].double().numpy(), pos, k[b, h].double().numpy(),
                                     v[b, h].double().numpy(), int(L[b]), w5.alpha, w5.causal)
        rows_done += pos.size
    el = time.perf_counter() - t0
    total_rows = float(L.sum()) * w5.Hq
    out["varlen_entmax"] = {"s_extrapolated": el / rows_done * total_rows,
                            "tokens_per_s": float(L.sum()) / (el / rows_done * total_rows),
                            "sample": f"{rows_done} rows (8 blocks of 64) of {int(total_rows)}, {el:.1f} s"}
    del q, k, v
    # 4: decode step, one (b, kv head) group of 4 query heads, scaled by the 128 groups
    w4 = WORKLOADS["decode_128k"]
    g = w4.Hq // w4.Hkv
    qd, Kc, Vc, clsd, seqlens = decode_inputs(1, g, 1, w4.N, w4.d, w4.seed, device="cpu")
    op4 = oracle.DashParams(chunk_size=C, alpha=w4.alpha, causal=True, estimate_diagonal=w4.estimate_diagonal)
    t0 = time.perf_counter()
    oracle.dash_decode(qd[:, :, 0].double().numpy(), Kc.float().numpy(), Vc.float().numpy(), clsd.double().numpy(),
                       seqlens.numpy(), op4)
    el = time.perf_counter() - t0
    groups = w4.B * w4.Hkv
    out["decode_128k"] = {"us_per_step_extrapolated": el * groups * 1e6,
                          "sample": f"one (b, kv head) group of {g} query heads over {w4.N + 1} tokens, "
                                    f"{el:.1f} s, x {groups} groups"}
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--no-entmax", action="store_true")
    ap.add_argument("--no-4k", action="store_true", help="skip the 4K routed prefill workload")
    ap.add_argument("--no-long", action="store_true", help="skip the 64K and 128K routed prefill workloads")
    ap.add_argument("--no-backward", action="store_true", help="skip the 32K prefill backward")
    ap.add_argument("--no-oracle-timings", action="store_true",
                    help="skip the oracle timings of the other workloads (the cpu_baseline leg stays)")
    ap.add_argument("--sparsity", action="store_true",
                    help="only the measured-sparsity sweep (alpha x scaling_factor) on the 32K needle workload")
    ap.add_argument("--union-density", action="store_true",
                    help="only the density of the routed chunks of row blocks (row-major vs chunk-major work) "
                         "on the 4K and 32K workloads")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="also run a plain 1 GiB device copy (for scaling PMC byte counters)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: this library has no multi-GPU path (prefill would shard by "
              "(batch, KV head) with no exchange, decode by batch); run with --gpus 1", file=sys.stderr)
        sys.exit(2)
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    if args.sparsity:
        print(json.dumps(sparsity_report(WORKLOADS["routed_prefill_32k"])), flush=True)
        return
    if args.union_density:
        print(json.dumps(union_density_report()), flush=True)
        return

    if args.calibrate_copy:
        calibrate_copy()
    wp = WORKLOADS["routed_prefill_32k"]
    log(f"prefill {wp.name}: steps={args.steps} warmup={args.warmup}")
    pre = bench_prefill(wp, args.steps, args.warmup)
    # the step's time: events around the whole step (summaries, routing, attention)
    ms_step = pre["ms_step"]
    log(f"prefill done: {ms_step:.3f} ms/step")
    value = wp.N / (ms_step / 1e3)
    # Dominant work: the sparse attention call (two thirds of the step; its
    # k_prefill_cm is the longest kernel), timed with HIP events around the whole
    # dash_sparse_attn_prefill call (k_cm_plan, k_cm_scatter, k_prefill_cm,
    # k_prefill_merge, k_sparse_prefill). Bound: MFMA, on the algorithmic flops
    # (4 d per row and visible key of a routed chunk); its measured HBM traffic
    # (the gathered query rows and the partial results written and read back) is
    # reported beside it.
    attn_ach = pre["alg_flops"] / (pre["ms_attention"] / 1e3) / 1e12
    attn_traffic = attention_traffic()
    roof = {
        "kernel": "dash_sparse_attn_prefill (k_prefill_cm + k_prefill_merge + k_cm_scatter + k_cm_plan + k_sparse_prefill)",
        "bound": "mfma",
        "achieved": attn_ach,
        "peak": PEAK_BF16_TFLOPS,
        "unit": "TFLOP/s",
        "frac": attn_ach / PEAK_BF16_TFLOPS,
        "traffic": attn_traffic,
        # the same counters with the reads scaled as a 256-byte-row gather reads
        # (the copy's scaling overstates gathered rows): the traffic lies between
        "traffic_gather_scaled": attention_traffic("hbm_bytes_gather_scaled"),
        "alg_flops_per_launch": pre["alg_flops"],
        "ms_per_launch": pre["ms_attention"],
        "executed_pair_frac": pre["pair_flops"] / (pre["ms_attention"] / 1e3) / 1e12 / PEAK_BF16_TFLOPS,
        "hbm_GBps_measured": attn_traffic / (pre["ms_attention"] / 1e3) / 1e9 if attn_traffic else None,
    }
    # The routing (dash_route: a 5 us summary split, k_route_fast, and the general
    # kernel for the tiles it leaves, 6 us when it leaves none). Its lower bounds:
    # HBM for the algorithmic bytes below (the largest), MFMA for the scores (2 d
    # flops per score), VALU for the candidate tests.
    route_bytes = route_alg_bytes(wp, pre["pairs"])
    ach = route_bytes / (pre["ms_route"] / 1e3) / 1e9
    route_roof = {
        "kernel": "k_route_fast",
        "bound": "hbm",
        "achieved": ach,
        "peak": PEAK_HBM_GBS,
        "unit": "GB/s",
        "frac": ach / PEAK_HBM_GBS,
        "traffic": measured_traffic("k_route_fast"),
        "alg_bytes_per_launch": route_bytes,
        "ms_per_launch": pre["ms_route"],
        "mfma_frac": 2.0 * wp.d * pre["route_scores"] / (pre["ms_route"] / 1e3) / 1e12 / PEAK_BF16_TFLOPS,
    }
    out = {
        "metric": "sparse prefill tokens/s at 32K + decode us/step at 128K; % of MFMA/HBM roofline",
        "value": value,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": wp.name,
            "batch": wp.B, "q_heads": wp.Hq, "kv_heads": wp.Hkv, "seq_len": wp.N, "head_dim": wp.d,
            "chunk_size": wp.chunk_size, "alpha": wp.alpha, "causal": wp.causal,
            "estimate_diagonal": wp.estimate_diagonal, "needles": "1% keys x4", "seed": wp.seed,
        },
        "prefill": {
            # the parts, each timed on its own (their sum leaves out the launch gaps between them)
            "ms_summarize": pre["ms_summarize"], "ms_route": pre["ms_route"], "ms_attention": pre["ms_attention"],
            "ms_parts_sum": pre["ms_summarize"] + pre["ms_route"] + pre["ms_attention"],
            "routed_chunks_per_row": pre["routed_chunks_per_row"],
            "workspace_GB": pre["workspace_GB"],
            # pool pairs used / capacity, tiles left to the general routing kernel, row-major tiles
            "counters": pre["counters"],
            # algorithmic attention flops over those of dense causal attention
            "alg_over_dense": pre["alg_flops"] / pre["dense_causal_flops"],
            # sparse attention (dash_sparse_attn_prefill, all of its kernels): MFMA
            # rate on the executed (row, chunk) pair blocks and on the algorithmic work
            "attention_pair_tflops": pre["pair_flops"] / (pre["ms_attention"] / 1e3) / 1e12,
            "attention_pair_frac": pre["pair_flops"] / (pre["ms_attention"] / 1e3) / 1e12 / PEAK_BF16_TFLOPS,
            "attention_alg_tflops": pre["alg_flops"] / (pre["ms_attention"] / 1e3) / 1e12,
            "attention_traffic": attn_traffic,
            "route_roofline": route_roof,
            # the summaries' backward (dash_summarize_backward) on the same keys, against HBM
            "summary_backward": pre["summary_backward"],
        },
        "roofline": roof,
    }
    if not args.no_4k:
        w2 = WORKLOADS["routed_prefill_4k"]
        log("prefill 4k")
        p2 = bench_prefill(w2, args.steps, args.warmup, summary_backward=False)
        ms2 = p2["ms_step"]
        out["prefill_4k"] = {
            "workload": w2.name, "tokens_per_s": w2.N / (ms2 / 1e3), "ms_per_step": ms2,
            "ms_summarize": p2["ms_summarize"], "ms_route": p2["ms_route"], "ms_attention": p2["ms_attention"],
            "routed_chunks_per_row": p2["routed_chunks_per_row"], "counters": p2["counters"],
            "alg_flops": p2["alg_flops"], "pair_flops": p2["pair_flops"], "dense_causal_flops": p2["dense_causal_flops"],
            "attention_alg_frac": p2["alg_flops"] / (p2["ms_attention"] / 1e3) / 1e12 / PEAK_BF16_TFLOPS,
            "attention_pair_frac": p2["pair_flops"] / (p2["ms_attention"] / 1e3) / 1e12 / PEAK_BF16_TFLOPS,
        }
    if not args.no_long:
        # the 32K recipe at 64K and 128K tokens: the length ceiling of the path
        out["prefill_long"] = {}
        for name in ("routed_prefill_64k", "routed_prefill_128k"):
            wl = WORKLOADS[name]
            log(f"prefill {name}")
            pl = bench_prefill(wl, min(args.steps, 10), min(args.warmup, 3), summary_backward=False)
            msl = pl["ms_step"]
            out["prefill_long"][name] = {
                "tokens_per_s": wl.N / (msl / 1e3), "ms_per_step": msl,
                "ms_summarize": pl["ms_summarize"], "ms_route": pl["ms_route"], "ms_attention": pl["ms_attention"],
                "routed_chunks_per_row": pl["routed_chunks_per_row"],
                "alg_over_dense": pl["alg_flops"] / pl["dense_causal_flops"],
                "attention_alg_frac": pl["alg_flops"] / (pl["ms_attention"] / 1e3) / 1e12 / PEAK_BF16_TFLOPS,
                "attention_pair_frac": pl["pair_flops"] / (pl["ms_attention"] / 1e3) / 1e12 / PEAK_BF16_TFLOPS,
                "workspace_GB": pl["workspace_GB"], "counters": pl["counters"],
            }
    if not args.no_backward:
        log("prefill backward 32k")
        out["prefill_backward"] = bench_dash_backward(wp, min(args.steps, 10), min(args.warmup, 3))
    if not args.no_entmax:
        out["dense_entmax_128"] = bench_entmax_small(WORKLOADS["dense_entmax_128"], args.steps, args.warmup)
    if not args.no_decode:
        wd = WORKLOADS["decode_128k"]
        log("decode 128k")
        dec = bench_decode(wd, max(args.steps, 20), args.warmup)
        gbs = (dec["kv_bytes"]) / (dec["us_attention"] / 1e6) / 1e9
        step_bytes = dec["kv_bytes"] + dec["summary_bytes"]
        out["decode"] = {
            "workload": wd.name,
            "us_per_step": dec["us_per_step"],
            "us_route": dec["us_route"],
            "us_attention": dec["us_attention"],
            "union_chunk_frac": dec["union_chunk_frac"],
            "step_GBps": step_bytes / (dec["us_per_step"] / 1e6) / 1e9,
            "roofline": {
                "kernel": "k_sparse_decode", "bound": "hbm", "achieved": gbs, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                "frac": gbs / PEAK_HBM_GBS, "traffic": measured_traffic("k_sparse_decode"),
                "bytes_per_launch": dec["kv_bytes"],
                # the whole step (routing against the summary cache, attention, append)
                "step_bytes": step_bytes,
                "step_frac": step_bytes / (dec["us_per_step"] / 1e6) / 1e9 / PEAK_HBM_GBS,
            },
        }
    if not args.no_entmax:
        we = WORKLOADS["varlen_entmax"]
        log("entmax varlen")
        ent = bench_entmax(we, args.steps, args.warmup)
        out["entmax"] = {"workload": we.name, **ent,
                         "roofline": {"kernel": "k_entmax_buf", "bound": "mfma", "achieved": ent["tflops_qk_pass"],
                                      "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                                      "frac": ent["tflops_qk_pass"] / PEAK_BF16_TFLOPS,
                                      "traffic": measured_traffic("k_entmax_buf")}}
    if not args.no_entmax:
        log("entmax rows")
        big = bench_entmax_rows(WORKLOADS["entmax_rows_64k_1024"], args.steps, args.warmup)
        small = bench_entmax_rows(WORKLOADS["entmax_rows_128x256"], args.steps, args.warmup)
        out["entmax_rows"] = {
            "workload": "entmax_rows_64k_1024", **big, "us_128x256": small["us"],
            "us_backward_128x256": small["us_backward"],
            "roofline": {"kernel": "k_entmax_rows", "bound": "hbm", "achieved": big["GBps"], "peak": PEAK_HBM_GBS,
                         "unit": "GB/s", "frac": big["GBps"] / PEAK_HBM_GBS,
                         "traffic": measured_traffic("k_entmax_rows")}}
    if not args.no_cpu_baseline:
        log("cpu baseline (oracle)")
        out["cpu_baseline"] = cpu_baseline(wp)
        out["cpu_baseline"]["numpy"] = np.__version__
        out["cpu_baseline"]["blas"] = _blas_info()
        if not args.no_oracle_timings:
            log("oracle timings of the other workloads")
            out["oracle_timings"] = oracle_timings()
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
