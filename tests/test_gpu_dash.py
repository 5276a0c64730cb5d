"""GPU parity of the DashAttention path (summaries, routing, sparse prefill and
decode attention) against the float64 CPU oracle, through the C ABI.

Small cases compare every row (several 128-row tiles, ragged tails, first
chunk, GQA, causal with and without the own-chunk estimate, non-causal, the
three tau solver specialisations). Full-size workloads (4K and 32K prefill,
batch-16 decode at 131072 cached tokens) run exactly as the benchmark launches
them and are checked on sampled rows the oracle computes one by one.
"""

import numpy as np
import pytest
import torch

import oracle
from adaptive_sparse_long_amd import api
from adaptive_sparse_long_amd.workloads import WORKLOADS, decode_inputs, routed_prefill_inputs

from _helpers import TOL_BF16, assert_close, assert_sets_match, f64, tau_close, unpack_bits

pytestmark = pytest.mark.gpu
C = 64


def _oracle_params(p: api.Params) -> oracle.DashParams:
    return oracle.DashParams(chunk_size=p.chunk_size, alpha=p.alpha, scaling_factor=p.scaling_factor,
                             causal=p.causal, estimate_diagonal=p.estimate_diagonal)


def _pool_workspace(Q, K, p: api.Params, pool_pairs: int):
    B, Hq, N, d = Q.shape
    n = api.prefill_workspace_size(B, Hq, K.shape[1], N, K.shape[2], d, p, pool_pairs)
    assert n > 0
    return torch.empty(n, dtype=torch.uint8, device=Q.device)


def check_prefill(Q, K, V, cls, p: api.Params, rows_of=None, where="", pool_pairs=None):
    """Run the GPU prefill and compare rows with the oracle.

    rows_of(b, h) -> array of rows to check (default: all). pool_pairs: the
    partial-result pool's size (default: the workspace query's)."""
    ws = None if pool_pairs is None else _pool_workspace(Q, K, p, pool_pairs)
    O, tau, bits, S, ws = api.prefill(Q, K, V, cls, p, workspace=ws)
    torch.cuda.synchronize()
    B, Hq, N, d = Q.shape
    Hkv = K.shape[1]
    g = Hq // Hkv
    op = _oracle_params(p)
    n_slots = -(-N // C)
    S_ = f64(S)
    checked = 0
    for b in range(B):
        for hk in range(Hkv):
            keys = f64(K[b, hk, :N])
            vals = f64(V[b, hk, :N])
            clsv = f64(cls[hk])
            summ = oracle.chunk_summaries(keys, clsv, C, N)
            n_sum = N // C if p.causal else n_slots
            assert_close(S_[b, hk, :n_sum], summ[:n_sum], 1e-5, f"{where} summaries b{b} h{hk}")
            for h in range(hk * g, (hk + 1) * g):
                rows = np.arange(N) if rows_of is None else np.asarray(rows_of(b, h))
                if rows.size == 0:
                    continue
                ri = torch.as_tensor(rows, device=O.device)
                qr = f64(Q[b, h, ri])
                o_got, t_got, b_got = f64(O[b, h, ri]), f64(tau[b, h, ri]), bits[b, h, ri].cpu().numpy()
                Z, t_ref, _, logw = oracle.route_row(qr, rows, keys, clsv, N, op, summ)
                o_ref, t2, b_ref = oracle.dash_rows(qr, rows, keys, vals, clsv, N, op, summ)
                tau_close(t_got, t_ref, f"{where} b{b} h{h}")
                with np.errstate(invalid="ignore"):
                    umt = (p.alpha - 1.0) * Z - t_ref[:, None]
                assert_sets_match(unpack_bits(b_got, n_slots), np.isfinite(logw), umt, f"{where} b{b} h{h}")
                assert_close(o_got, o_ref, TOL_BF16, f"{where} O b{b} h{h}")
                checked += rows.size
    assert checked > 0
    return api.prefill_counters(ws, B, Hq, Hkv, N, d, p)


def _inputs(B, Hq, Hkv, N, seed, planted="chunks"):
    q, k, v, cls = routed_prefill_inputs(B, Hq, Hkv, N, 128, seed, planted=planted, device="cuda")
    return q, k, v, cls


@pytest.mark.parametrize(
    "B,Hq,Hkv,N,p,planted",
    [
        (1, 4, 1, 1000, api.Params(causal=True, estimate_diagonal=True), "chunks"),
        (1, 4, 1, 1000, api.Params(causal=True, estimate_diagonal=False), "needles"),
        (2, 4, 2, 700, api.Params(causal=False), "chunks"),
        (1, 8, 2, 2048, api.Params(alpha=2.0), "chunks"),
        (1, 2, 2, 520, api.Params(alpha=1.333, estimate_diagonal=True), "chunks"),
        (1, 4, 4, 300, api.Params(scaling_factor=3.0), None),
        (1, 1, 1, 64, api.Params(), None),
        (1, 1, 1, 37, api.Params(estimate_diagonal=False), None),
        (1, 8, 1, 700, api.Params(), "needles"),
        (2, 4, 2, 900, api.Params(estimate_diagonal=True), "chunks"),
    ],
)
def test_prefill_small(B, Hq, Hkv, N, p, planted):
    Q, K, V, cls = _inputs(B, Hq, Hkv, N, 7 + N, planted)
    check_prefill(Q, K, V, cls, p, where=f"N={N} {p}")


@pytest.mark.parametrize(
    "B,Hq,Hkv,N,p,planted,pool",
    [
        (1, 4, 1, 1000, api.Params(causal=True, estimate_diagonal=True), "chunks", None),
        (2, 4, 2, 700, api.Params(causal=False), "chunks", None),
        (1, 8, 2, 2048, api.Params(alpha=2.0), "needles", None),
        (1, 4, 4, 300, api.Params(scaling_factor=3.0), None, None),
        (1, 1, 1, 37, api.Params(estimate_diagonal=False), None, None),
        (1, 4, 1, 1000, api.Params(estimate_diagonal=True), "chunks", 0),  # every tile row-major
    ],
)
def test_prefill_head_dim_64(B, Hq, Hkv, N, p, planted, pool):
    """head_dim 64: the kernels run their 128-wide layouts with the upper dims
    zero; summaries, tau, routed sets and O against the oracle at d = 64."""
    Q, K, V, cls = routed_prefill_inputs(B, Hq, Hkv, N, 64, 11 + N, planted=planted, device="cuda")
    cnt = check_prefill(Q, K, V, cls, p, where=f"d64 N={N} {p}", pool_pairs=pool)
    if pool == 0:
        assert cnt["row_major_tiles"] > 0, cnt


@pytest.mark.parametrize(
    "B,Hq,Hkv,N,p",
    [
        (1, 2, 1, 1, api.Params()),                                # one token
        (1, 2, 1, 2, api.Params(estimate_diagonal=False)),
        (1, 4, 2, 63, api.Params()),                               # no complete chunk
        (1, 4, 2, 65, api.Params(estimate_diagonal=False)),        # one complete chunk + 1 token
        (2, 4, 1, 65, api.Params(alpha=2.0)),
        (1, 2, 2, 129, api.Params()),                              # one row past a 128-row tile
        (1, 2, 1, 1, api.Params(causal=False)),
        (1, 4, 4, 65, api.Params(causal=False, alpha=1.333)),
    ],
)
def test_prefill_tiny_edges(B, Hq, Hkv, N, p):
    """Tiny and ragged lengths around the chunk (64) and tile (128) sizes."""
    Q, K, V, cls = _inputs(B, Hq, Hkv, N, 900 + N, None)
    check_prefill(Q, K, V, cls, p, where=f"tiny N={N} {p}")


@pytest.mark.parametrize(
    "B,Hq,Hkv,N,p,planted",
    [
        (1, 4, 1, 1000, api.Params(causal=True, estimate_diagonal=True), "chunks"),
        (1, 4, 1, 1000, api.Params(causal=True, estimate_diagonal=False), "needles"),
        (2, 4, 2, 700, api.Params(causal=False), "chunks"),
        (1, 8, 2, 2048, api.Params(alpha=2.0), "chunks"),
        (1, 2, 2, 520, api.Params(alpha=1.333, estimate_diagonal=True), "chunks"),
    ],
)
def test_prefill_row_major_recomputed_weights(B, Hq, Hkv, N, p, planted):
    """With no partial-result pool every tile is attended row-major, each row's
    prior weight for a listed chunk recomputed from its tau, its routed-chunk
    bits and the split summaries: the same rows as the chunk-major path."""
    Q, K, V, cls = _inputs(B, Hq, Hkv, N, 7 + N, planted)
    cnt = check_prefill(Q, K, V, cls, p, where=f"N={N} {p} pool 0", pool_pairs=0)
    assert cnt["pool_capacity"] == 0 and cnt["pool_pairs"] == 0 and cnt["row_major_tiles"] > 0, cnt


def test_prefill_partial_pool_mixes_paths():
    """A pool of 40% of the routed past pairs: the tiles that reserve first go
    chunk-major, the rest row-major, in one call; every row matches the oracle."""
    Q, K, V, cls = _inputs(1, 8, 2, 2048, 31, "chunks")
    p = api.Params()
    _, _, bits, _, _ = api.prefill(Q, K, V, cls, p)
    n_slots = -(-2048 // C)
    att = unpack_bits(bits.cpu().numpy(), n_slots).sum()  # attended chunks, own ones included
    past = int(att) - 8 * 2048
    assert past > 0
    cnt = check_prefill(Q, K, V, cls, p, where="partial pool", pool_pairs=int(0.4 * past))
    assert 0 < cnt["pool_pairs"] <= cnt["pool_capacity"] and cnt["row_major_tiles"] > 0, cnt


def test_prefill_workspace_size_mismatch_gives_nan():
    """The pool's size follows ws_bytes, so routing and attention must be given
    the same size: a smaller one in the attention call is caught on the device
    and every output row is NaN (instead of reading a misplaced pool)."""
    Q, K, V, cls = _inputs(1, 4, 1, 1000, 5, "chunks")
    p = api.Params()
    ws = _pool_workspace(Q, K, p, 100000)
    api.prefill(Q, K, V, cls, p, workspace=ws)  # routes with the full size
    small = api.prefill_workspace_size(1, 4, 1, 1000, 1000, 128, p, 50000)
    O = api.sparse_attn_prefill(Q, K, V, ws[:small], p)
    torch.cuda.synchronize()
    assert torch.isnan(O.float()).all()
    O = api.sparse_attn_prefill(Q, K, V, ws, p)  # the matching size works
    torch.cuda.synchronize()
    assert torch.isfinite(O.float()).all()


def test_prefill_zero_scaling_is_dense_causal():
    """scaling_factor 0: uniform prior over all candidates, i.e. dense causal softmax."""
    Q, K, V, cls = _inputs(1, 4, 2, 640, 99, None)
    O, tau, bits, _, _ = api.prefill(Q, K, V, cls, api.Params(scaling_factor=0.0))
    ref = torch.nn.functional.scaled_dot_product_attention(
        Q.float().cpu(), K.float().cpu().repeat_interleave(2, 1), V.float().cpu().repeat_interleave(2, 1),
        is_causal=True)
    assert_close(f64(O), ref.double().numpy(), TOL_BF16, "dense causal")


def test_prefill_pool_exhausted_falls_back_to_row_major():
    """Uniform routing over 4096 causal keys needs about twice the default
    partial-result pool (16 pairs per row at this length): tiles that find it
    exhausted attend all their chunks row-major, the others chunk-major; both
    must give dense causal attention."""
    Q, K, V, cls = _inputs(1, 2, 1, 4096, 17, None)
    O, tau, bits, _, _ = api.prefill(Q, K, V, cls, api.Params(scaling_factor=0.0))
    ref = torch.nn.functional.scaled_dot_product_attention(
        Q.float().cpu(), K.float().cpu().repeat_interleave(2, 1), V.float().cpu().repeat_interleave(2, 1),
        is_causal=True)
    assert_close(f64(O), ref.double().numpy(), TOL_BF16, "dense causal, pool exhausted")


def test_prefill_routing_heavy_and_left_tiles():
    """Rows with a zero query score every past chunk alike, so every chunk is a
    routing candidate: some tiles then hold more candidates per lane than the
    routing kernel keeps in registers (read back from LDS) and some more than
    its LDS list (left to the general routing kernel), next to ordinary tiles
    of the same call and of the other head."""
    Q, K, V, cls = _inputs(1, 2, 1, 4096, 23)
    Q[:, 0, 1536:3584] = 0
    rng = np.random.default_rng(23)
    fixed = np.array([0, 100, 1535, 1536, 1600, 2047, 2048, 2100, 2175, 2176, 3000, 3583, 3584, 4095])
    cnt = check_prefill(Q, K, V, cls, api.Params(),
                        rows_of=lambda b, h: np.unique(np.concatenate([fixed, rng.integers(1536, 3584, 10)])),
                        where="heavy tiles")
    assert cnt["general_route_tiles"] > 0, cnt


def test_prefill_deterministic():
    Q, K, V, cls = _inputs(1, 8, 2, 1536, 5)
    p = api.Params()
    O1, t1, b1, _, _ = api.prefill(Q, K, V, cls, p)
    O2, t2, b2, _, _ = api.prefill(Q, K, V, cls, p)
    assert torch.equal(O1, O2) and torch.equal(t1, t2) and torch.equal(b1, b2)


def _sample_rows(N, rng, k=12):
    fixed = [0, 1, C - 1, C, 127, 128, N // 2, N - C, N - 1]
    return np.unique(np.concatenate([fixed, rng.integers(0, N, k)]))


def test_prefill_4k_workload_sampled():
    w = WORKLOADS["routed_prefill_4k"]
    Q, K, V, cls = routed_prefill_inputs(w.B, w.Hq, w.Hkv, w.N, w.d, w.seed, planted=w.planted, device="cuda")
    p = api.Params(alpha=w.alpha, causal=w.causal, estimate_diagonal=w.estimate_diagonal)
    rng = np.random.default_rng(w.seed)
    full = {0, 13}
    check_prefill(Q, K, V, cls, p, rows_of=lambda b, h: np.arange(w.N) if h in full else _sample_rows(w.N, rng, 6),
                  where="4k")


def test_prefill_32k_workload_sampled():
    w = WORKLOADS["routed_prefill_32k"]
    Q, K, V, cls = routed_prefill_inputs(w.B, w.Hq, w.Hkv, w.N, w.d, w.seed, planted=w.planted, device="cuda")
    p = api.Params(alpha=w.alpha, causal=w.causal, estimate_diagonal=w.estimate_diagonal)
    rng = np.random.default_rng(w.seed)
    heads = {0, 9, 22, 31}
    cnt = check_prefill(Q, K, V, cls, p, rows_of=lambda b, h: _sample_rows(w.N, rng, 10) if h in heads else [],
                        where="32k")
    # the default workspace's pool (5 pairs per row) holds every routed pair here
    assert cnt["row_major_tiles"] == 0 and cnt["pool_pairs"] < 0.8 * cnt["pool_capacity"], cnt


def test_prefill_32k_head_dim_64_sampled():
    """The 32K needle recipe at head_dim 64 (sampled rows of two heads)."""
    w = WORKLOADS["routed_prefill_32k"]
    Q, K, V, cls = routed_prefill_inputs(w.B, w.Hq, w.Hkv, w.N, 64, w.seed + 64, planted=w.planted, device="cuda")
    p = api.Params(alpha=w.alpha, causal=w.causal, estimate_diagonal=w.estimate_diagonal)
    rng = np.random.default_rng(w.seed + 64)
    heads = {3, 28}
    check_prefill(Q, K, V, cls, p, rows_of=lambda b, h: _sample_rows(w.N, rng, 10) if h in heads else [],
                  where="32k d64")


def test_prefill_32k_workload_full_tiles():
    """Complete 128-row tiles of the 32K needle workload at depths 4K, 8K, 16K
    and 32K - 128, for all four query heads of KV head 0: every row of each
    tile (its union list, pool slots and merge) against the oracle."""
    w = WORKLOADS["routed_prefill_32k"]
    Q, K, V, cls = routed_prefill_inputs(w.B, w.Hq, w.Hkv, w.N, w.d, w.seed, planted=w.planted, device="cuda")
    p = api.Params(alpha=w.alpha, causal=w.causal, estimate_diagonal=w.estimate_diagonal)
    rows = np.concatenate([np.arange(t0, t0 + 128) for t0 in (4096, 8192, 16384, w.N - 128)])
    check_prefill(Q, K, V, cls, p, rows_of=lambda b, h: rows if h < 4 else [], where="32k tiles")


def test_prefill_32k_workload_scaling4_sampled():
    """The 32K needle workload at scaling_factor 4 (one of the measured-sparsity
    sweep's points: sharper routing), sampled rows of four heads."""
    w = WORKLOADS["routed_prefill_32k"]
    Q, K, V, cls = routed_prefill_inputs(w.B, w.Hq, w.Hkv, w.N, w.d, w.seed, planted=w.planted, device="cuda")
    p = api.Params(alpha=w.alpha, scaling_factor=4.0, causal=w.causal, estimate_diagonal=w.estimate_diagonal)
    rng = np.random.default_rng(w.seed + 4)
    heads = {3, 12, 17, 30}
    check_prefill(Q, K, V, cls, p, rows_of=lambda b, h: _sample_rows(w.N, rng, 10) if h in heads else [],
                  where="32k sf4")


def test_prefill_long_general_routing_in_global_scratch():
    """Past 512 chunk slots (here 40000 tokens: 625) the list-based routing uses
    its 2048-slot form, and tiles it cannot keep (zero queries make every chunk
    a candidate) go to the general kernel's global-scratch form; sampled rows of
    both kinds of tile against the oracle."""
    Q, K, V, cls = _inputs(1, 2, 1, 40000, 41)
    Q[:, 0, 20000:24000] = 0
    rng = np.random.default_rng(41)
    fixed = np.array([0, 63, 64, 4095, 19999, 20000, 20100, 22000, 23999, 24000, 32767, 32768, 39935, 39999])
    cnt = check_prefill(Q, K, V, cls, api.Params(),
                        rows_of=lambda b, h: np.unique(np.concatenate([fixed, rng.integers(0, 40000, 8)])),
                        where="40k general")
    assert cnt["general_route_tiles"] > 0, cnt


def test_prefill_long_noncausal_sampled():
    """Non-causal past 512 chunk slots (36000 tokens: 563 slots, a partial last
    chunk): every row routes over every chunk, sampled rows against the oracle."""
    Q, K, V, cls = _inputs(1, 4, 2, 36000, 43, "chunks")
    rng = np.random.default_rng(43)
    fixed = np.array([0, 1, 127, 128, 17999, 35935, 35936, 35999])
    check_prefill(Q, K, V, cls, api.Params(causal=False),
                  rows_of=lambda b, h: np.unique(np.concatenate([fixed, rng.integers(0, 36000, 6)])),
                  where="36k non-causal")


def test_prefill_long_tile_union_over_1024_goes_general():
    """A tile whose routed chunks number more than 1024 (the 2048-slot list
    kernel's entry cap) although its candidate list is short: the keys of chunk
    c are 6 e_(c mod 128) (e_j one-hot, so the summaries are exactly those
    codes) and row i of the last tile queries 6 e_(i mod 128), so it routes the
    ~10 chunks carrying its code with equal weight and the tile's 128 rows route
    ~1240 chunks in all. The tile is routed by the general kernel (global
    scratch form); sampled rows of it and of other tiles against the oracle."""
    N = 80000
    Q, K, V, cls = _inputs(1, 1, 1, N, 47, None)
    eye = torch.zeros(128, 128, device="cuda")
    eye[torch.arange(128), torch.arange(128)] = 6.0
    codes = eye[torch.arange(N, device="cuda") // C % 128].to(K.dtype)
    K[0, 0] = codes
    last = torch.arange(N - N % 128 - 128, N - N % 128, device="cuda")
    Q[0, 0, last] = eye[last % 128].to(Q.dtype)
    rng = np.random.default_rng(47)
    rows = np.unique(np.concatenate([last.cpu().numpy()[::9], [0, 64, 5000, 40000, N - 1], rng.integers(0, N, 6)]))
    cnt = check_prefill(Q, K, V, cls, api.Params(), rows_of=lambda b, h: rows, where="union over 1024")
    assert cnt["general_route_tiles"] > 0, cnt


@pytest.mark.parametrize("name", ["routed_prefill_64k", "routed_prefill_128k"])
def test_prefill_long_workload_sampled(name):
    """The 32K needle recipe at 64K and 128K tokens (1024 and 2048 chunk
    slots): sampled rows of two heads, plus a complete tile at the end."""
    w = WORKLOADS[name]
    Q, K, V, cls = routed_prefill_inputs(w.B, w.Hq, w.Hkv, w.N, w.d, w.seed, planted=w.planted, device="cuda")
    p = api.Params(alpha=w.alpha, causal=w.causal, estimate_diagonal=w.estimate_diagonal)
    rng = np.random.default_rng(w.seed)
    last = np.arange(w.N - 128, w.N)
    cnt = check_prefill(Q, K, V, cls, p,
                        rows_of=lambda b, h: (np.unique(np.concatenate([_sample_rows(w.N, rng, 8), last]))
                                              if h in (5, 26) else []),
                        where=name)
    assert cnt["row_major_tiles"] == 0, cnt


# ----------------------------------------------------------------------------- decode


def check_decode(q, Kc, Vc, cls, seqlens, p: api.Params, pairs=None, where=""):
    """Summaries of complete chunks, one decode step, compare with the oracle."""
    B, Hkv, Lmax, d = Kc.shape
    Hq = q.shape[1]
    g = Hq // Hkv
    S = torch.zeros(B, Hkv, -(-Lmax // C), d, dtype=torch.float32, device=q.device)
    api.summarize(Kc, cls, S, seqlens=seqlens, chunk_begin=0, chunk_end=Lmax // C, params=p)
    O, tau, bits, _ = api.decode_step(q, Kc, Vc, cls, S, seqlens, p)
    torch.cuda.synchronize()
    op = _oracle_params(p)
    lens = seqlens.cpu().numpy()
    n_slots = -(-Lmax // C)
    O_, tau_, bits_ = f64(O), f64(tau), bits.cpu().numpy()
    pairs = pairs or [(b, h) for b in range(B) for h in range(Hq)]
    by_kv = {}
    for b, h in pairs:
        by_kv.setdefault((b, h // g), []).append(h)
    for (b, hk), heads in sorted(by_kv.items()):
        n = int(lens[b])
        keys, vals, clsv = f64(Kc[b, hk, :n]), f64(Vc[b, hk, :n]), f64(cls[hk])
        summ = oracle.chunk_summaries(keys, clsv, C, n)
        for h in heads:
            qr = f64(q[b, h])  # [1, d]
            pos = np.array([n - 1])
            Z, t_ref, _, logw = oracle.route_row(qr, pos, keys, clsv, n, op, summ)
            o_ref, _, _ = oracle.dash_rows(qr, pos, keys, vals, clsv, n, op, summ)
            tau_close(tau_[b, h, :1], t_ref, f"{where} b{b} h{h}")
            gb = unpack_bits(bits_[b, h, 0], n_slots)[: Z.shape[1]]
            with np.errstate(invalid="ignore"):
                umt = (p.alpha - 1.0) * Z[0] - t_ref[0]
            assert_sets_match(gb, np.isfinite(logw[0]), umt, f"{where} b{b} h{h}")
            assert not unpack_bits(bits_[b, h, 0], n_slots)[Z.shape[1]:].any()
            assert_close(O_[b, h, 0], o_ref[0], TOL_BF16, f"{where} O b{b} h{h}")
    return O


@pytest.mark.parametrize("est", [True, False])
@pytest.mark.parametrize("g", [1, 2, 4, 8])
def test_decode_small(est, g):
    Hkv = 2
    q, Kc, Vc, cls, _ = decode_inputs(3, Hkv * g, Hkv, 1100, 128, seed=31 + g, device="cuda", Lmax=1160)
    seqlens = torch.tensor([1025, 1088, 700], dtype=torch.int32, device="cuda")
    check_decode(q, Kc, Vc, cls, seqlens, api.Params(estimate_diagonal=est), where=f"g{g} est{est}")


@pytest.mark.parametrize("g,est", [(1, True), (4, True), (4, False), (8, True)])
def test_decode_head_dim_64(g, est):
    """Decode at head_dim 64 (caches, queries, head_cls and the summary cache
    64 wide) against the oracle."""
    Hkv = 2
    q, Kc, Vc, cls, _ = decode_inputs(3, Hkv * g, Hkv, 1100, 64, seed=41 + g, device="cuda", Lmax=1160)
    seqlens = torch.tensor([1025, 1088, 700], dtype=torch.int32, device="cuda")
    check_decode(q, Kc, Vc, cls, seqlens, api.Params(estimate_diagonal=est), where=f"d64 g{g} est{est}")


def test_decode_first_chunk_and_alpha2():
    q, Kc, Vc, cls, _ = decode_inputs(4, 4, 1, 200, 128, seed=3, device="cuda", Lmax=256)
    seqlens = torch.tensor([1, 2, 64, 65], dtype=torch.int32, device="cuda")
    check_decode(q, Kc, Vc, cls, seqlens, api.Params(alpha=2.0), where="short")


def test_decode_matches_prefill_row():
    N = 1000
    Q, K, V, cls = _inputs(1, 4, 1, N, 17)
    p = api.Params()
    O, tau, _, S, _ = api.prefill(Q, K, V, cls, p)
    for t in (63, 64, 500, N - 1):
        seqlens = torch.tensor([t + 1], dtype=torch.int32, device="cuda")
        q = Q[:, :, t : t + 1].contiguous()
        Od, td, _, _ = api.decode_step(q, K, V, cls, S, seqlens, p)
        assert_close(f64(Od[:, :, 0]), f64(O[:, :, t]), 2e-2, f"row {t}")
        assert_close(f64(td[:, :, 0]), f64(tau[:, :, t]), 2e-5, f"tau {t}")


def test_decode_append_matches_prefill_summary():
    q, Kc, Vc, cls, _ = decode_inputs(2, 4, 2, 300, 128, seed=8, device="cuda", Lmax=320)
    p = api.Params()
    S = torch.zeros(2, 2, 5, 128, dtype=torch.float32, device="cuda")
    seqlens = torch.tensor([256, 256], dtype=torch.int32, device="cuda")  # token 255 completes chunk 3
    api.summarize(Kc, cls, S, seqlens=seqlens, chunk_begin=0, chunk_end=3, params=p)
    assert torch.all(S[:, :, 3] == 0)
    api.decode_step(q, Kc, Vc, cls, S, seqlens, p, lengths=[256, 256])
    torch.cuda.synchronize()
    for b in range(2):
        for hk in range(2):
            ref = oracle.chunk_summary(f64(Kc[b, hk, 192:256]), f64(cls[hk]))
            assert_close(f64(S[b, hk, 3]), ref, 1e-5, "appended summary")


def test_decode_multi_step_with_appends_matches_prefill():
    """Resume from a prefix: the summary cache is built for the complete chunks of
    T tokens, then 20 decode steps each attend the next token and append the
    chunk it completes (batch entries at different lengths, each crossing a chunk
    boundary mid-way). Every step must equal the prefill's row at that position
    (which the prefill tests hold to the oracle), and the cache must end equal
    to the prefill's summaries."""
    T, steps = [250, 186], 20
    N = max(T) + steps
    Q, K, V, cls = _inputs(2, 4, 2, N, 61, "chunks")
    p = api.Params()
    O_pre, tau_pre, _, S_pre, _ = api.prefill(Q, K, V, cls, p)
    Lmax = 320
    Kc = torch.zeros(2, 2, Lmax, 128, dtype=K.dtype, device="cuda")
    Vc = torch.zeros_like(Kc)
    Kc[:, :, :N], Vc[:, :, :N] = K, V
    S = torch.zeros(2, 2, Lmax // C, 128, dtype=torch.float32, device="cuda")
    lens0 = torch.tensor(T, dtype=torch.int32, device="cuda")
    api.summarize(Kc, cls, S, seqlens=lens0, chunk_begin=0, chunk_end=Lmax // C, params=p)
    ws = None
    for k in range(steps):
        t = [T[0] + k, T[1] + k]
        seqlens = torch.tensor([t[0] + 1, t[1] + 1], dtype=torch.int32, device="cuda")
        q = torch.stack([Q[0, :, t[0]], Q[1, :, t[1]]])[:, :, None].contiguous()
        Od, td, _, ws = api.decode_step(q, Kc, Vc, cls, S, seqlens, p, lengths=[t[0] + 1, t[1] + 1], workspace=ws)
        torch.cuda.synchronize()
        for b in range(2):
            assert_close(f64(Od[b, :, 0]), f64(O_pre[b, :, t[b]]), 2e-2, f"step {k} b{b} row {t[b]}")
            assert_close(f64(td[b, :, 0]), f64(tau_pre[b, :, t[b]]), 2e-5, f"tau step {k} b{b} row {t[b]}")
    # chunks completed by the end: 0 .. (T + steps) // 64 - 1 per entry
    for b in range(2):
        n_done = (T[b] + steps) // C
        assert_close(f64(S[b, :, :n_done]), f64(S_pre[b, :, :n_done]), 1e-5, f"summary cache b{b}")
    assert T[0] // C < (T[0] + steps) // C and T[1] // C < (T[1] + steps) // C  # both crossed a boundary


def test_decode_128k_workload_sampled():
    w = WORKLOADS["decode_128k"]
    q, Kc, Vc, cls, seqlens = decode_inputs(w.B, w.Hq, w.Hkv, w.N, w.d, w.seed, device="cuda")
    rng = np.random.default_rng(w.seed)
    pairs = [(int(b), int(h)) for b, h in zip(rng.integers(0, w.B, 6), rng.integers(0, w.Hq, 6))]
    pairs += [(0, 0), (w.B - 1, w.Hq - 1)]
    # one complete (b, kv head) group: all g query heads that share its routed list
    g = w.Hq // w.Hkv
    pairs += [(5, 5 * g + j) for j in range(g)]
    check_decode(q, Kc, Vc, cls, seqlens, api.Params(alpha=w.alpha, estimate_diagonal=w.estimate_diagonal),
                 pairs=pairs, where="128k")
