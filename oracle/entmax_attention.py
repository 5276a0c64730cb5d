"""Dense alpha-entmax attention with a per-tile block mask, float64 (CPU oracle;
test infrastructure only).

Follows the AdaSplash README page ("AdaSplash: Adaptive Sparse Flash Attention"):

* "Usage", "AdaSplash with Block Masking": attention whose row normaliser is
  alpha-entmax instead of softmax, q/k/v in [batch, heads, seq, head_dim], with
  arguments alpha, niter, is_causal and varlen, plus one stored bit per
  (query block, key block) saying whether the block holds any non-zero weight;
* "Key Features": ``varlen`` gives each batch entry's actual length; alpha
  controls sparsity; causal and non-causal masking.

Readings (the page prints no formula):

* score s_ij = <q_i, k_j> / sqrt(d) over allowed keys: j < len_b, and j <= i
  when causal;
* weights P_i = entmax_alpha(s_i) (exact threshold, see ``oracle.entmax``);
  output O_i = sum_j P_ij v_j; tau_i is reported in u = (alpha - 1) s units;
* rows i >= len_b output zeros and tau = 0;
* block mask bit (I, J), 64 x 64 tiles: 1 iff some allowed (i, j) in the tile has
  P_ij > 0. Layout [B, H, nT, ceil(nT / 32)] uint32 with bit J % 32 of word
  J // 32, nT = ceil(N / 64).

The backward (the page runs these kernels forward and backward, "Usage", and
lists block-sparse forward and backward passes among its "Key Features") is the
chain rule through those definitions, nothing more: dV = P^T dO, dP = dO V^T,
dS_i = the alpha-entmax vector-Jacobian product of row i at (P_i, dP_i)
(``oracle.entmax.entmax_backward``), dQ = dS K / sqrt(d), dK = dS^T Q / sqrt(d).
"""

from __future__ import annotations

import numpy as np

from .entmax import entmax_backward, entmax_threshold_rows

__all__ = ["entmax_attention", "entmax_attention_rows", "entmax_attention_backward", "TILE"]

TILE = 64


def _f64(x) -> np.ndarray:
    return np.asarray(x, dtype=np.float64)


def entmax_attention_rows(q_rows, pos, keys, values, length: int, alpha: float, causal: bool):
    """Rows of one (b, h): returns (O [m, d], tau [m], P [m, length])."""
    q_rows, keys, values = _f64(q_rows), _f64(keys), _f64(values)
    d = q_rows.shape[-1]
    pos = np.asarray(pos)
    S = (q_rows @ keys[:length].T) / np.sqrt(d)
    j = np.arange(length)
    allowed = np.ones_like(S, dtype=bool)
    if causal:
        allowed &= j[None, :] <= pos[:, None]
    S = np.where(allowed, S, -np.inf)
    tau = entmax_threshold_rows(S, alpha)
    beta = 1.0 / (alpha - 1.0)
    with np.errstate(invalid="ignore"):
        diff = np.where(allowed, (alpha - 1.0) * S - tau[:, None], -1.0)
    pos_part = np.maximum(diff, 0.0)
    if beta == 1.0:
        P = pos_part
    elif beta == 2.0:
        P = pos_part * pos_part
    else:
        with np.errstate(divide="ignore"):
            P = np.where(diff > 0, np.exp(beta * np.log(np.where(diff > 0, diff, 1.0))), 0.0)
    O = P @ values[:length]
    return O, tau, P


def entmax_attention(Q, K, V, alpha: float, causal: bool, varlen=None, row_block: int = 512):
    """Q/K/V [B, H, N, d] -> (O [B,H,N,d], tau [B,H,N], block mask [B,H,nT,ceil(nT/32)])."""
    Q, K, V = _f64(Q), _f64(K), _f64(V)
    B, H, N, d = Q.shape
    nT = -(-N // TILE)
    words = -(-nT // 32)
    O = np.zeros_like(Q)
    tau = np.zeros((B, H, N))
    mask = np.zeros((B, H, nT, words), dtype=np.uint32)
    for b in range(B):
        L = N if varlen is None else int(varlen[b])
        for h in range(H):
            for r0 in range(0, L, row_block):
                pos = np.arange(r0, min(L, r0 + row_block))
                o, t, P = entmax_attention_rows(Q[b, h, pos], pos, K[b, h], V[b, h], L, alpha, causal)
                O[b, h, pos] = o
                tau[b, h, pos] = t
                nz = P > 0
                for I in np.unique(pos // TILE):
                    rows = (pos // TILE) == I
                    cols = np.any(nz[rows], axis=0)
                    for J in np.unique(np.nonzero(cols)[0] // TILE):
                        mask[b, h, I, J // 32] |= np.uint32(1) << np.uint32(J % 32)
    return O, tau, mask


def entmax_attention_backward(Q, K, V, dO, alpha: float, causal: bool, varlen=None):
    """Gradients of sum(O * dO) with respect to Q, K and V, float64.

    Q/K/V/dO [B, H, N, d] -> (dQ, dK, dV), each [B, H, N, d]. Rows and keys at or
    past varlen[b] get zero gradients (they take no part in the forward).
    """
    Q, K, V, dO = _f64(Q), _f64(K), _f64(V), _f64(dO)
    B, H, N, d = Q.shape
    dQ, dK, dV = np.zeros_like(Q), np.zeros_like(K), np.zeros_like(V)
    for b in range(B):
        L = N if varlen is None else int(varlen[b])
        if L <= 0:
            continue
        pos = np.arange(L)
        for h in range(H):
            _, _, P = entmax_attention_rows(Q[b, h, :L], pos, K[b, h], V[b, h], L, alpha, causal)
            dP = dO[b, h, :L] @ V[b, h, :L].T
            dS = np.stack([entmax_backward(P[i], dP[i], alpha) for i in range(L)])
            dV[b, h, :L] = P.T @ dO[b, h, :L]
            dQ[b, h, :L] = dS @ K[b, h, :L] / np.sqrt(d)
            dK[b, h, :L] = dS.T @ Q[b, h, :L] / np.sqrt(d)
    return dQ, dK, dV
