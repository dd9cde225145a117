"""Attention with dropout on the probabilities -- test infrastructure only.

The pages name dropout as one of the operations the fused kernel performs
together with the matrix products, masking and softmax (FlashAttention reading
guide, xyznot.com, "Ide Utama", kernel-fusion bullet; bornlex.github.io "Flash
Attention", section "Standard Attention", which lists masking and dropout as
the other elementwise operations beside the softmax), but give neither its
formula nor a random-number generator.
The plainest reading, used here and by the kernels:

  * dropout acts on P after the softmax; the row normaliser is the one of the
    un-dropped scores, so lse is unchanged.  An entry is kept with
    probability 1 - p and kept entries are scaled by 1 / (1 - p):
        O = (P * Z) V,   Z_ij = keep_ij / (1 - p);
  * p = t / 256 for an integer t in [0, 255]; entry (b, h, i, j) (query i,
    key j) is kept iff its random byte u >= t, an integer decision;
  * the random bytes come from Philox4x32-10 (J. K. Salmon, M. A. Moraes,
    R. O. Dror, D. E. Shaw, "Parallel Random Numbers: As Easy as 1, 2, 3",
    SC 2011), a counter-based generator, so the backward pass regenerates the
    same bytes: key (seed mod 2^32, seed >> 32), counter
    (j >> 2, i >> 2, b * H + h, 0); u is byte (j & 3) (bits 8 (j & 3) ..
    8 (j & 3) + 7) of output word (i & 3).  One generator call covers the
    4 x 4 block of queries 4 (i >> 2) .. +3 and keys 4 (j >> 2) .. +3.

Backward (chain rule through O = (P * Z) V and the row softmax, as in
``attention``):
  dV = (P * Z)^T dO,   dP = (dO V^T) * Z,   D_i = sum_j P_ij dP_ij,
  dS = P * (dP - D),   dQ = scale dS K,   dK = scale dS^T Q;
D_i also equals dO_i . O_i with the dropout O, as without dropout.
"""
from __future__ import annotations

import numpy as np

from .attention import _probs, allowed

# Philox4x32 constants: round multipliers and the Weyl key increments (Salmon et
# al., section on the Philox family).
PHILOX_M0, PHILOX_M1 = 0xD2511F53, 0xCD9E8D57
PHILOX_W0, PHILOX_W1 = 0x9E3779B9, 0xBB67AE85
MASK32 = 0xFFFFFFFF


def philox4x32_10(c0, c1, c2, c3, k0, k1):
    """Philox4x32 with 10 rounds on arrays of 32-bit counters (broadcast).

    One round maps (c0, c1, c2, c3) with key (k0, k1) to
        (hi(M1 c2) ^ c1 ^ k0,  lo(M1 c2),  hi(M0 c0) ^ c3 ^ k1,  lo(M0 c0))
    where hi / lo are the upper / lower 32 bits of the 64-bit product; the key
    is advanced by the Weyl increments (W0, W1) before every round but the
    first.  Returns four uint32 arrays."""
    c = [np.asarray(x, dtype=np.uint64) & np.uint64(MASK32) for x in (c0, c1, c2, c3)]
    c = list(np.broadcast_arrays(*c))
    key0, key1 = int(k0) & MASK32, int(k1) & MASK32
    m0, m1 = np.uint64(PHILOX_M0), np.uint64(PHILOX_M1)
    sh, lo = np.uint64(32), np.uint64(MASK32)
    for r in range(10):
        if r:
            key0 = (key0 + PHILOX_W0) & MASK32
            key1 = (key1 + PHILOX_W1) & MASK32
        p0 = m0 * c[0]          # < 2^64: no overflow in uint64
        p1 = m1 * c[2]
        c = [(p1 >> sh) ^ c[1] ^ np.uint64(key0), p1 & lo, (p0 >> sh) ^ c[3] ^ np.uint64(key1), p0 & lo]
    return [x.astype(np.uint32) for x in c]


def random_bytes(bh, rows, keys, seed):
    """u[r, k] (uint8 values as int64) for queries rows x keys of head bh."""
    i = np.asarray(rows, dtype=np.int64)[:, None]
    j = np.asarray(keys, dtype=np.int64)[None, :]
    w = philox4x32_10(j >> 2, i >> 2, bh, 0, seed & MASK32, (seed >> 32) & MASK32)
    word = np.choose(i & 3, [x.astype(np.int64) for x in w])
    return (word >> (8 * (j & 3))) & 0xFF


def keep_scale(bh, rows, keys, t, seed):
    """Z[r, k] = keep / (1 - t/256) for queries rows x keys of head bh."""
    keep = random_bytes(bh, rows, keys, seed) >= int(t)
    return keep / (1.0 - int(t) / 256.0)


def head_forward(Q, K, V, scale, bh, t, seed, rows=None, causal=False, block_mask=None, kv_len=None):
    """One head (index bh = b * H + h): O[rows] and lse[rows] with dropout."""
    Q = np.asarray(Q, np.float64)
    K = np.asarray(K, np.float64)
    V = np.asarray(V, np.float64)
    rows = np.arange(Q.shape[0]) if rows is None else np.asarray(rows)
    S = scale * (Q[rows] @ K.T)
    S = np.where(allowed(rows, K.shape[0], causal, block_mask, kv_len), S, -np.inf)
    P, lse = _probs(S)
    Z = keep_scale(bh, rows, np.arange(K.shape[0]), t, seed)
    return (P * Z) @ V, lse


def _row_grads(Q, K, V, dO, scale, bh, t, seed, rows, causal, block_mask, kv_len):
    """P * Z and dS of the given query rows (every term of a row is row-local:
    its softmax, its keep pattern, dP = (dO V^T) * Z and D = sum_j P dP)."""
    keys = np.arange(K.shape[0])
    S = scale * (Q[rows] @ K.T)
    S = np.where(allowed(rows, K.shape[0], causal, block_mask, kv_len), S, -np.inf)
    P, _ = _probs(S)
    Z = keep_scale(bh, rows, keys, t, seed)
    dP = (dO[rows] @ V.T) * Z
    D = (P * dP).sum(axis=1)
    return P * Z, P * (dP - D[:, None])


def head_backward(Q, K, V, dO, scale, bh, t, seed, causal=False, block_mask=None, kv_len=None,
                  row_block=1024):
    """One head: dQ, dK, dV with dropout, by the chain rule in the module docstring."""
    Q = np.asarray(Q, np.float64)
    K = np.asarray(K, np.float64)
    V = np.asarray(V, np.float64)
    dO = np.asarray(dO, np.float64)
    N = Q.shape[0]
    dQ, dK, dV = np.zeros_like(Q), np.zeros_like(K), np.zeros_like(V)
    for r0 in range(0, N, row_block):
        rows = np.arange(r0, min(N, r0 + row_block))
        PZ, dS = _row_grads(Q, K, V, dO, scale, bh, t, seed, rows, causal, block_mask, kv_len)
        dV += PZ.T @ dO[rows]
        dQ[rows] = scale * (dS @ K)
        dK += scale * (dS.T @ Q[rows])
    return dQ, dK, dV


def head_backward_rows(Q, K, V, dO, scale, bh, t, seed, rows, causal=False, block_mask=None, kv_len=None):
    """dQ[rows] of one head with dropout (for long sequences, where the full
    backward would hold N x N arrays)."""
    Q, K, V, dO = (np.asarray(x, np.float64) for x in (Q, K, V, dO))
    rows = np.asarray(rows, np.int64)
    _, dS = _row_grads(Q, K, V, dO, scale, bh, t, seed, rows, causal, block_mask, kv_len)
    return scale * (dS @ K)


def forward(q, k, v, scale, t, seed, causal=False, block_mask=None, kv_len=None):
    """O [B,H,N,d] and lse [B,H,N] in float64, with dropout."""
    B, H, N, _ = q.shape
    O = np.zeros(q.shape[:3] + (v.shape[-1],), np.float64)
    lse = np.zeros((B, H, N), np.float64)
    for b in range(B):
        L = None if kv_len is None else int(kv_len[b])
        for h in range(H):
            O[b, h], lse[b, h] = head_forward(q[b, h], k[b, h], v[b, h], scale, b * H + h, t, seed, None,
                                              causal, block_mask, L)
    return O, lse


def backward(q, k, v, do, scale, t, seed, causal=False, block_mask=None, kv_len=None):
    """dQ, dK, dV [B,H,N,d] in float64 for the loss sum(O * dO), with dropout."""
    B, H = q.shape[:2]
    dq, dk, dv = (np.zeros(x.shape, np.float64) for x in (q, k, v))
    for b in range(B):
        L = None if kv_len is None else int(kv_len[b])
        for h in range(H):
            dq[b, h], dk[b, h], dv[b, h] = head_backward(q[b, h], k[b, h], v[b, h], do[b, h], scale,
                                                         b * H + h, t, seed, causal, block_mask, L)
    return dq, dk, dv
