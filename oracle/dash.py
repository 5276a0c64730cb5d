"""DashAttention hierarchy in float64 (CPU oracle; test infrastructure only).

Follows the DashAttention README page ("DashAttention: Differentiable and
Adaptive Sparse Hierarchical Attention"), section "How it works":

1. local chunk summarisation: one learned key summary per KV chunk, built with
   the per-KV-head vector ``head_cls`` ("Usage", "Core API": head_cls has shape
   [kv_heads, head_dim]);
2. entmax block routing: query-to-summary scores go through alpha-entmax, whose
   support is the routed chunk set and whose probabilities are the routing prior;
3. prior-induced sparse softmax: token-level softmax attention only over the
   routed chunks, with the prior entering the logits.

Prefill and decode share one definition: decode of the token at position t is
row t of prefill on t + 1 tokens ("How it works", last paragraph: prefill stores
complete chunk summaries, decoding reuses that cache and appends chunks as they
complete).

The page gives no formulas. The readings used here (all plain, all stated):

* summary of a chunk: softmax attention pooling of the chunk's keys with
  head_cls as the query and scale 1/sqrt(d):  s_c = sum_j a_j k_j,
  a = softmax_j(<k_j, head_cls> / sqrt(d));
* routing score: z_ic = scaling_factor * <q_i, s_c> / sqrt(d), prior
  pi_ic = entmax_alpha(z_i)_c, routed set A_i = support of pi_i;
* candidates, causal: complete chunks c < c_i = floor(i / C); with
  estimate_diagonal the row's own chunk is one more candidate whose summary is
  taken over the tokens [c_i * C, i] seen so far; without it the own chunk is
  not routed but always attended with weight 1;
* candidates, non-causal: every chunk, a partial last chunk summarised over the
  tokens it has (estimate_diagonal is ignored);
* prior in attention: logit_ij = <q_i, k_j>/sqrt(d) + log w_{i, c(j)} over the
  tokens of A_i (j <= i when causal), normalised by one softmax over all of
  them; w = pi (1 for the forced diagonal);
* GQA ("Core API", enable_gqa): query head h reads KV head h // (Hq / Hkv);
  routing is per query head.

Everything is computed "dense then mask" for clarity; row blocks only bound
memory and do not change any row's arithmetic.
"""

from __future__ import annotations

from dataclasses import dataclass

import numpy as np

from .entmax import entmax_backward, entmax_threshold_rows

__all__ = [
    "DashParams",
    "chunk_summary",
    "chunk_summaries",
    "route_row",
    "dash_rows",
    "dash_prefill",
    "dash_decode",
    "dash_backward",
]


@dataclass(frozen=True)
class DashParams:
    """Configuration mirroring the wrapper's arguments in "Core API"."""

    chunk_size: int = 64
    alpha: float = 1.5
    scaling_factor: float = 1.0
    causal: bool = True
    estimate_diagonal: bool = True


def _f64(x) -> np.ndarray:
    return np.asarray(x, dtype=np.float64)


def chunk_summary(keys, cls) -> np.ndarray:
    """Summary key of a run of keys [n, d] pooled with head_cls [d] ("How it works" 1)."""
    keys = _f64(keys)
    cls = _f64(cls)
    d = keys.shape[-1]
    logits = keys @ cls / np.sqrt(d)
    a = np.exp(logits - np.max(logits))
    a /= np.sum(a)
    return a @ keys


def chunk_summary_backward(keys, cls, ds):
    """Gradients of <chunk_summary(keys, cls), ds> with respect to the keys [n, d]
    and head_cls [d]: the chain rule through s = sum_j a_j k_j and
    a = softmax(e), e_j = <k_j, cls> / sqrt(d) (the pages differentiate the whole
    hierarchy, "How it works"; the steps are the summary's own definition):
        de_j = a_j (<k_j, ds> - <s, ds>),
        dk_j = a_j ds + de_j cls / sqrt(d),   dcls = sum_j de_j k_j / sqrt(d).
    """
    keys = _f64(keys)
    cls = _f64(cls)
    ds = _f64(ds)
    d = keys.shape[-1]
    e = keys @ cls / np.sqrt(d)
    a = np.exp(e - np.max(e))
    a /= np.sum(a)
    s = a @ keys
    de = a * (keys @ ds - s @ ds)
    dk = a[:, None] * ds[None, :] + de[:, None] * cls[None, :] / np.sqrt(d)
    dcls = de @ keys / np.sqrt(d)
    return dk, dcls


def chunk_summaries(keys, cls, chunk_size: int, n_tokens: int) -> np.ndarray:
    """Summaries [ceil(n_tokens / C), d] of one KV head; the last may be partial."""
    keys = _f64(keys)
    n_c = -(-n_tokens // chunk_size)
    out = np.zeros((n_c, keys.shape[-1]))
    for c in range(n_c):
        out[c] = chunk_summary(keys[c * chunk_size : min((c + 1) * chunk_size, n_tokens)], cls)
    return out


def _candidate_scores(q_rows, pos, keys, cls, summ, n_tokens, p: DashParams):
    """Routing scores [m, n_slots] (-inf = not a candidate) for query rows at ``pos``.

    Column c < n_slots is chunk c. For causal rows with estimate_diagonal the own
    chunk's column holds the score against the prefix summary.
    """
    C = p.chunk_size
    d = q_rows.shape[-1]
    n_slots = -(-n_tokens // C)
    m = q_rows.shape[0]
    Z = np.full((m, n_slots), -np.inf)
    scale = p.scaling_factor / np.sqrt(d)
    full = scale * (q_rows @ summ.T) if summ.shape[0] else np.zeros((m, 0))
    for r in range(m):
        i = int(pos[r])
        if p.causal:
            ci = i // C
            Z[r, :ci] = full[r, :ci]
            if p.estimate_diagonal:
                s_hat = chunk_summary(keys[ci * C : i + 1], cls)
                Z[r, ci] = scale * float(q_rows[r] @ s_hat)
        else:
            Z[r, :] = full[r, :n_slots]
    return Z


def route_row(q_rows, pos, keys, cls, n_tokens: int, p: DashParams, summ=None):
    """Route query rows of one (b, query head) ("How it works" 2).

    Returns (Z, tau, prior, logw): scores [m, n_slots], tau [m] in
    u = (alpha - 1) z units (+inf for a row without candidates), prior pi
    [m, n_slots] and log weights [m, n_slots] (-inf = chunk not attended).
    """
    q_rows = _f64(q_rows)
    keys = _f64(keys)
    C = p.chunk_size
    if summ is None:
        summ = chunk_summaries(keys, cls, C, n_tokens)
    Z = _candidate_scores(q_rows, pos, keys, cls, summ, n_tokens, p)
    tau = entmax_threshold_rows(Z, p.alpha)
    beta = 1.0 / (p.alpha - 1.0)
    U = (p.alpha - 1.0) * Z
    with np.errstate(invalid="ignore"):
        diff = np.where(np.isfinite(U) & np.isfinite(tau)[:, None], U - tau[:, None], -1.0)
    prior = np.where(diff > 0, np.power(np.maximum(diff, 0.0), beta), 0.0)
    with np.errstate(divide="ignore"):
        logw = np.where(prior > 0, np.log(np.where(prior > 0, prior, 1.0)), -np.inf)
    if p.causal and not p.estimate_diagonal:
        ci = np.asarray(pos) // C
        logw[np.arange(len(pos)), ci] = 0.0  # own chunk always attended, weight 1
    return Z, tau, prior, logw


def _attend_rows(q_rows, pos, keys, values, logw, n_tokens, p: DashParams):
    """Prior-induced sparse softmax ("How it works" 3), dense then mask."""
    C = p.chunk_size
    d = q_rows.shape[-1]
    j = np.arange(n_tokens)
    bias = logw[:, j // C]  # [m, n_tokens]
    if p.causal:
        bias = np.where(j[None, :] <= np.asarray(pos)[:, None], bias, -np.inf)
    logits = (q_rows @ keys[:n_tokens].T) / np.sqrt(d) + bias
    mx = np.max(logits, axis=1, keepdims=True)
    w = np.exp(logits - mx)
    w /= np.sum(w, axis=1, keepdims=True)
    return w @ values[:n_tokens]


def _bits(mask_bool: np.ndarray) -> np.ndarray:
    """Pack a boolean [m, n] chunk mask into [m, ceil(n/32)] uint32 (bit c%32 of word c//32)."""
    m, n = mask_bool.shape
    words = -(-n // 32) if n else 0
    out = np.zeros((m, words), dtype=np.uint32)
    for c in range(n):
        out[:, c // 32] |= mask_bool[:, c].astype(np.uint32) << np.uint32(c % 32)
    return out


def dash_rows(q_rows, pos, keys, values, cls, n_tokens: int, p: DashParams, summ=None):
    """Output, tau and attended-chunk bitmask for rows of one (b, query head).

    keys/values are the rows of the KV head this query head reads.
    """
    q_rows = _f64(q_rows)
    keys = _f64(keys)
    values = _f64(values)
    _, tau, _, logw = route_row(q_rows, pos, keys, cls, n_tokens, p, summ)
    out = _attend_rows(q_rows, pos, keys, values, logw, n_tokens, p)
    return out, tau, _bits(np.isfinite(logw))


def dash_prefill(Q, K, V, head_cls, p: DashParams, row_block: int = 256):
    """Full prefill. Q [B,Hq,N,d], K/V [B,Hkv,N,d], head_cls [Hkv,d].

    Returns O [B,Hq,N,d], tau [B,Hq,N], active bitmask [B,Hq,N,ceil(n_c/32)].
    """
    Q, K, V, head_cls = _f64(Q), _f64(K), _f64(V), _f64(head_cls)
    B, Hq, N, d = Q.shape
    Hkv = K.shape[1]
    if Hq % Hkv:
        raise ValueError("Hq must be a multiple of Hkv")
    g = Hq // Hkv
    n_c = -(-N // p.chunk_size)
    O = np.zeros_like(Q)
    tau = np.zeros((B, Hq, N))
    bits = np.zeros((B, Hq, N, -(-n_c // 32)), dtype=np.uint32)
    for b in range(B):
        for hk in range(Hkv):
            summ = chunk_summaries(K[b, hk], head_cls[hk], p.chunk_size, N)
            for h in range(hk * g, (hk + 1) * g):
                for r0 in range(0, N, row_block):
                    pos = np.arange(r0, min(N, r0 + row_block))
                    o, t, bt = dash_rows(Q[b, h, pos], pos, K[b, hk], V[b, hk], head_cls[hk], N, p, summ)
                    O[b, h, pos] = o
                    tau[b, h, pos] = t
                    bits[b, h, pos] = bt
    return O, tau, bits


def dash_decode(q, Kc, Vc, head_cls, seqlens, p: DashParams):
    """One decode step. q [B,Hq,d]; caches Kc/Vc [B,Hkv,Lmax,d] holding the new
    token's key/value at position seqlens[b] - 1, which is the query position.

    Returns O [B,Hq,d], tau [B,Hq], bitmask [B,Hq,ceil(ceil(t+1 / C)/32)] per row
    as a list (rows of different batches may have different widths).
    """
    q, head_cls = _f64(q), _f64(head_cls)
    B, Hq, d = q.shape
    Hkv = Kc.shape[1]
    g = Hq // Hkv
    O = np.zeros((B, Hq, d))
    tau = np.zeros((B, Hq))
    bits = [[None] * Hq for _ in range(B)]
    for b in range(B):
        n = int(seqlens[b])
        t = n - 1
        for hk in range(Hkv):
            keys = _f64(Kc[b, hk, :n])  # converted one (b, kv head) at a time
            values = _f64(Vc[b, hk, :n])
            summ = chunk_summaries(keys, head_cls[hk], p.chunk_size, n)
            for h in range(hk * g, (hk + 1) * g):
                o, tt, bt = dash_rows(q[b, h][None, :], np.array([t]), keys, values, head_cls[hk], n, p, summ)
                O[b, h] = o[0]
                tau[b, h] = tt[0]
                bits[b][h] = bt[0]
    return O, tau, bits


def dash_backward(Q, K, V, head_cls, dO, p: DashParams):
    """Gradients of L = sum(O * dO) for the prefill O = dash_prefill(Q, K, V,
    head_cls, p) with respect to Q, K, V and head_cls.

    The DashAttention README calls the router "adaptive, differentiable" and has
    stage 3 use the stage-1 prior "to preserve differentiability through the
    hierarchy" ("Documentation", "How it works" item 3). The pages print no
    formula; this is the chain rule through the forward defined above, step by
    step, nothing more:

    * attention (per row i, over its allowed tokens j): P = softmax(logits),
      dP_ij = <dO_i, v_j>, dlogit_ij = P_ij (dP_ij - sum_j P_ij dP_ij),
      dV_j += sum_i P_ij dO_i, dQ_i += sum_j dlogit_ij k_j / sqrt(d),
      dK_j += sum_i dlogit_ij q_i / sqrt(d);
    * prior (logit_ij contains log w_{i, c(j)}): g_ic = sum_{j in c} dlogit_ij
      is the gradient of log w_ic; a routed chunk has w = pi, so
      d pi_ic = g_ic / pi_ic; the own chunk attended with weight 1 (causal,
      estimate_diagonal off) is not a routing candidate and passes nothing on;
    * routing: pi_i = entmax_alpha(z_i) over the row's candidates, so
      dz_i = the entmax vector-Jacobian product at (pi_i, d pi_i)
      (``entmax_backward``; chunks off the support get 0);
    * scores z_ic = scaling_factor <q_i, s_c> / sqrt(d):
      dQ_i += scaling_factor / sqrt(d) sum_c dz_ic s_c, ds_c += scaling_factor /
      sqrt(d) sum_i dz_ic q_i (over every row and query head of the KV head);
      with estimate_diagonal the own chunk's candidate is scored against the
      prefix summary s^_i of tokens [c_i C, i], whose gradient
      scaling_factor / sqrt(d) dz_i,c_i q_i goes through ``chunk_summary_backward``
      of those tokens;
    * summaries: ``chunk_summary_backward`` of every summarised chunk for its ds.

    Returns (dQ [B,Hq,N,d], dK [B,Hkv,N,d], dV [B,Hkv,N,d], dcls [Hkv,d]).
    """
    Q, K, V, head_cls, dO = _f64(Q), _f64(K), _f64(V), _f64(head_cls), _f64(dO)
    B, Hq, N, d = Q.shape
    Hkv = K.shape[1]
    if Hq % Hkv:
        raise ValueError("Hq must be a multiple of Hkv")
    g = Hq // Hkv
    C = p.chunk_size
    n_c = -(-N // C)
    rt = p.scaling_factor / np.sqrt(d)
    dQ = np.zeros_like(Q)
    dK = np.zeros_like(K)
    dV = np.zeros_like(V)
    dcls = np.zeros_like(head_cls)
    pos = np.arange(N)
    j = np.arange(N)
    for b in range(B):
        for hk in range(Hkv):
            keys, vals, cls = K[b, hk], V[b, hk], head_cls[hk]
            summ = chunk_summaries(keys, cls, C, N)
            ds = np.zeros_like(summ)
            for h in range(hk * g, (hk + 1) * g):
                q, do = Q[b, h], dO[b, h]
                Z, tau, prior, logw = route_row(q, pos, keys, cls, N, p, summ)
                # ---- attention, dense then mask
                bias = logw[:, j // C]
                if p.causal:
                    bias = np.where(j[None, :] <= pos[:, None], bias, -np.inf)
                logits = (q @ keys.T) / np.sqrt(d) + bias
                P = np.exp(logits - np.max(logits, axis=1, keepdims=True))
                P /= np.sum(P, axis=1, keepdims=True)
                dP = do @ vals.T
                dlog = P * (dP - np.sum(P * dP, axis=1, keepdims=True))
                dV[b, hk] += P.T @ do
                dQ[b, h] += dlog @ keys / np.sqrt(d)
                dK[b, hk] += dlog.T @ q / np.sqrt(d)
                # ---- prior: gradient of log w per (row, chunk)
                gw = np.zeros((N, n_c))
                for c in range(n_c):
                    gw[:, c] = np.sum(dlog[:, c * C : min((c + 1) * C, N)], axis=1)
                # ---- routing: entmax over each row's candidates (finite Z)
                dZ = np.zeros_like(Z)
                for i in range(N):
                    cand = np.isfinite(Z[i])
                    if not cand.any():
                        continue
                    pi = prior[i, cand]
                    dpi = np.where(pi > 0, gw[i, cand] / np.where(pi > 0, pi, 1.0), 0.0)
                    dZ[i, cand] = entmax_backward(pi, dpi, p.alpha)
                # ---- scores against the summaries (and the own-chunk estimate)
                for i in range(N):
                    ci = i // C
                    for c in range(n_c):
                        if dZ[i, c] == 0.0:
                            continue
                        if p.causal and c == ci:
                            # the estimate of the own chunk from tokens [ci*C, i]
                            s_hat = chunk_summary(keys[ci * C : i + 1], cls)
                            dQ[b, h, i] += rt * dZ[i, c] * s_hat
                            dk, dc = chunk_summary_backward(keys[ci * C : i + 1], cls, rt * dZ[i, c] * q[i])
                            dK[b, hk, ci * C : i + 1] += dk
                            dcls[hk] += dc
                        else:
                            dQ[b, h, i] += rt * dZ[i, c] * summ[c]
                            ds[c] += rt * dZ[i, c] * q[i]
            # ---- summaries of the chunks the routing read
            for c in range(n_c):
                if not np.any(ds[c]):
                    continue
                lo, hi = c * C, min((c + 1) * C, N)
                dk, dc = chunk_summary_backward(keys[lo:hi], cls, ds[c])
                dK[b, hk, lo:hi] += dk
                dcls[hk] += dc
    return dQ, dK, dV, dcls
