"""Dense fp64 attention: the definition, forward and backward.

Test infrastructure only (see the package docstring).

Forward, per (batch b, head h), following bornlex.github.io "Flash Attention",
section "Standard Attention" (S = QK^T, P = softmax(S) row-wise, O = PV) with
two additions the pages leave open:
  * a scale: S = scale * Q K^T (scale = 1 gives the pages' formula);
  * masks: an entry S[i, j] is -inf when key j is not allowed for query i
    (``allowed``); such entries get probability exactly 0.
The softmax is the safe form with the row maximum subtracted (bornlex
"Flash Attention", section "Tiling", the rewritten softmax with m(x)).
The per-row statistic kept for the backward pass is lse = m + ln(l), the
natural log of the row normaliser of the scaled scores (the pages keep (l, m),
FlashAttention reading guide "Ide Utama", recomputation bullet; lse holds the
same information because P = exp(S - lse)).

A row with no allowed key gets O = 0, lse = -inf and contributes nothing to
any gradient.

Backward: the pages print no backward equations (they only say S and P are
recomputed, bornlex "Flash Attention" section "Recomputation").  With
L = sum(O * dO) the chain rule through O = PV and the row softmax gives
  dV = P^T dO,   dP = dO V^T,   D_i = sum_j P_ij dP_ij,
  dS = P * (dP - D),   dQ = scale * dS K,   dK = scale * dS^T Q.
"""
from __future__ import annotations

import numpy as np

CELL = 128


def allowed(rows, nk, causal=False, block_mask=None, kv_len=None, cell=CELL, keys=None, causal_offset=0):
    """Boolean [len(rows), nk]; True where key j may be attended by query i.

    causal: j <= i + causal_offset.  With as many queries as keys the offset
    is 0 (queries and keys share positions, top-left aligned); for Nq queries
    against Nk >= Nq keys it is Nk - Nq, the queries being the last Nq
    positions (bottom-right aligned).
    kv_len: j < kv_len (key padding).
    block_mask: block_mask[i // cell, j // cell] == 1 (block-sparse cells,
    FlashAttention reading guide "Ekstensi: Block-Sparse FlashAttention").
    The three conditions are combined with AND.  With ``keys`` given, the
    columns are those key positions instead of 0 .. nk-1."""
    i = np.asarray(rows, dtype=np.int64)[:, None]
    j = (np.arange(nk, dtype=np.int64) if keys is None else np.asarray(keys, dtype=np.int64))[None, :]
    nk = j.shape[1]
    ok = np.ones((i.shape[0], nk), dtype=bool)
    if causal:
        ok &= j <= i + int(causal_offset)
    if kv_len is not None:
        ok &= j < int(kv_len)
    if block_mask is not None:
        bm = np.asarray(block_mask).astype(bool)
        ok &= bm[i // cell, j // cell]
    return ok


def _probs(Sm):
    """Row softmax of masked scores (-inf = masked). Returns (P, lse)."""
    m = Sm.max(axis=1)
    empty = ~np.isfinite(m)
    shift = np.where(empty, 0.0, m)
    E = np.exp(Sm - shift[:, None])
    l = E.sum(axis=1)
    P = E / np.where(empty, 1.0, l)[:, None]
    lse = np.where(empty, -np.inf, shift + np.log(np.where(empty, 1.0, l)))
    return P, lse


def head_forward(Q, K, V, scale, rows=None, causal=False, block_mask=None, kv_len=None, causal_offset=0):
    """One (b, h): O[rows], lse[rows] with Q [Nq, d] and K, V [Nk, d]."""
    Q = np.asarray(Q, np.float64)
    K = np.asarray(K, np.float64)
    V = np.asarray(V, np.float64)
    rows = np.arange(Q.shape[0]) if rows is None else np.asarray(rows)
    S = scale * (Q[rows] @ K.T)
    S = np.where(allowed(rows, K.shape[0], causal, block_mask, kv_len, causal_offset=causal_offset), S, -np.inf)
    P, lse = _probs(S)
    return P @ V, lse


def forward(q, k, v, scale, causal=False, block_mask=None, kv_len=None, row_block=1024):
    """O [B,H,N,d] and lse [B,H,N] in float64."""
    B, H, N, d = q.shape
    O = np.zeros((B, H, N, v.shape[-1]), np.float64)
    lse = np.zeros((B, H, N), np.float64)
    for b in range(B):
        L = None if kv_len is None else int(kv_len[b])
        for h in range(H):
            for r0 in range(0, N, row_block):
                rows = np.arange(r0, min(N, r0 + row_block))
                O[b, h, rows], lse[b, h, rows] = head_forward(
                    q[b, h], k[b, h], v[b, h], scale, rows, causal, block_mask, L)
    return O, lse


def head_backward(Q, K, V, dO, scale, causal=False, block_mask=None, kv_len=None,
                  row_block=1024):
    """One (b, h): dQ, dK, dV ([N, d] each) by the chain rule above."""
    Q = np.asarray(Q, np.float64)
    K = np.asarray(K, np.float64)
    V = np.asarray(V, np.float64)
    dO = np.asarray(dO, np.float64)
    N = Q.shape[0]
    dQ = np.zeros_like(Q)
    dK = np.zeros_like(K)
    dV = np.zeros_like(V)
    for r0 in range(0, N, row_block):
        rows = np.arange(r0, min(N, r0 + row_block))
        S = scale * (Q[rows] @ K.T)
        S = np.where(allowed(rows, K.shape[0], causal, block_mask, kv_len), S, -np.inf)
        P, _ = _probs(S)
        dV += P.T @ dO[rows]
        dP = dO[rows] @ V.T
        D = (P * dP).sum(axis=1)
        dS = P * (dP - D[:, None])
        dQ[rows] = scale * (dS @ K)
        dK += scale * (dS.T @ Q[rows])
    return dQ, dK, dV


def backward(q, k, v, do, scale, causal=False, block_mask=None, kv_len=None, row_block=1024):
    """dQ, dK, dV [B,H,N,d] in float64 for the loss sum(O * dO)."""
    B, H, N, d = q.shape
    dq = np.zeros(q.shape, np.float64)
    dk = np.zeros(k.shape, np.float64)
    dv = np.zeros(v.shape, np.float64)
    for b in range(B):
        L = None if kv_len is None else int(kv_len[b])
        for h in range(H):
            dq[b, h], dk[b, h], dv[b, h] = head_backward(
                q[b, h], k[b, h], v[b, h], do[b, h], scale, causal, block_mask, L, row_block)
    return dq, dk, dv
