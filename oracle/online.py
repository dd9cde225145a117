"""The incremental softmax statistics and the tiled forward, as the pages state them.

Test infrastructure only (see the package docstring).  Nothing here is used to
produce expected values for the GPU; the pin tests use it to show that the
block-by-block method reaches the plain definition in ``attention`` exactly
(up to rounding), which is the pages' exactness claim.

f, l and the two-block merge: bornlex.github.io "Flash Attention", section
"Tiling" (f(x) = exp(x - m(x)), l(x) = sum f(x), softmax = f / l, and the
merge of m, f and l over x = [x1, x2]); FlashAttention reading guide
(xyznot.com), "Pelacakan Softmax Inkremental" (the merge of m and l).

Tiled forward: the key axis of each query block is cut into blocks, and the
statistics of the whole row are a left fold of the two-block merge above over
those blocks (reading guide, "Pelacakan Softmax Inkremental"; the per-block
procedure is the reading guide's "Metode").  The output is carried the same
way: each block contributes its unnormalised f(x) V, weighted by
exp(m_block - m), and the row is divided by l once, after the last block.
Scale and masks are added as in ``attention``.  A block whose entries are all
masked has m = -inf and weight 0, so it adds nothing.
"""
from __future__ import annotations

import numpy as np

from .attention import allowed


def m_of(x):
    return np.max(x, axis=-1)


def f_of(x):
    m = m_of(x)
    return np.exp(x - m[..., None])


def l_of(x):
    return f_of(x).sum(axis=-1)


def _w(a, b):
    """exp(a - b), with 0 where a is -inf (an empty block carries no weight)."""
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    out = np.zeros(np.broadcast(a, b).shape)
    fin = np.isfinite(a) & np.isfinite(b)
    np.exp(np.broadcast_to(a - np.where(np.isfinite(b), b, 0.0), out.shape), out=out, where=fin)
    return out


def merge(m1, l1, m2, l2):
    """Statistics (m, l) of [x1, x2] from those of x1 and x2."""
    m = np.maximum(m1, m2)
    return m, _w(m1, m) * l1 + _w(m2, m) * l2


def merge_f(m1, f1, m2, f2):
    """f of [x1, x2] from the blocks: [exp(m1 - m) f1, exp(m2 - m) f2]."""
    m = np.maximum(m1, m2)
    return np.concatenate([_w(m1, m)[..., None] * f1, _w(m2, m)[..., None] * f2], axis=-1)


def _block_stats(S):
    """(m, l, F) of one block of masked scores: row max, row sum of f and f itself."""
    m = S.max(axis=1)
    F = _w(S, m[:, None])
    return m, F.sum(axis=1), F


def tiled_head_forward(Q, K, V, scale, Br, Bc, causal=False, block_mask=None, kv_len=None):
    """One (b, h) folded block by block; returns O, m, l ([N,d], [N], [N])."""
    Q = np.asarray(Q, np.float64)
    K = np.asarray(K, np.float64)
    V = np.asarray(V, np.float64)
    N, Nk = Q.shape[0], K.shape[0]
    O = np.zeros((N, V.shape[1]))
    m_all = np.full(N, -np.inf)
    l_all = np.zeros(N)
    for i0 in range(0, N, Br):
        rows = np.arange(i0, min(N, i0 + Br))
        ok = allowed(rows, Nk, causal, block_mask, kv_len)
        m = np.full(rows.size, -np.inf)
        l = np.zeros(rows.size)
        acc = np.zeros((rows.size, V.shape[1]))      # unnormalised output, relative to m
        for j0 in range(0, Nk, Bc):
            cols = np.arange(j0, min(Nk, j0 + Bc))
            S = np.where(ok[:, cols], scale * (Q[rows] @ K[cols].T), -np.inf)
            mb, lb, F = _block_stats(S)
            m_new, l = merge(m, l, mb, lb)
            acc = _w(m, m_new)[:, None] * acc + _w(mb, m_new)[:, None] * (F @ V[cols])
            m = m_new
        inv = np.where(l > 0, 1.0 / np.where(l > 0, l, 1.0), 0.0)
        O[rows], m_all[rows], l_all[rows] = inv[:, None] * acc, m, l
    return O, m_all, l_all
