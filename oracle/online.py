"""The incremental softmax statistics and the tiled forward, as the pages state them.

Test infrastructure only (see the package docstring).  Nothing here is used to
produce expected values for the GPU; the pin tests use it to show that the
block-by-block method reaches the plain definition in ``attention`` exactly
(up to rounding), which is the pages' exactness claim.

f, l and the two-block merge: bornlex.github.io "Flash Attention", section
"Tiling" (f(x) = exp(x - m(x)), l(x) = sum f(x), softmax = f / l, and the
merge of m, f and l over x = [x1, x2]); FlashAttention reading guide
(xyznot.com), "Pelacakan Softmax Inkremental" (the merge of m and l).

Tiled forward: FlashAttention reading guide, "Metode", steps 1-4 -- per query
block i and key block j: the block scores, the block statistics (row max,
exp, row sum), the update of the running (m, l), and the update of the running
output, which is re-normalised at every step.  Scale and masks are added as in
``attention``.  A block whose rows are all masked so far keeps m = -inf; the
exponent of (-inf) - (-inf) is taken as 0 weight, i.e. the -inf block adds
nothing.
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


def tiled_head_forward(Q, K, V, scale, Br, Bc, causal=False, block_mask=None, kv_len=None):
    """One (b, h) with the block-by-block update; returns O, m, l ([N,d], [N], [N])."""
    Q = np.asarray(Q, np.float64)
    K = np.asarray(K, np.float64)
    V = np.asarray(V, np.float64)
    N, Nk = Q.shape[0], K.shape[0]
    O = np.zeros((N, V.shape[1]))
    m_all = np.full(N, -np.inf)
    l_all = np.zeros(N)
    for i0 in range(0, N, Br):
        rows = np.arange(i0, min(N, i0 + Br))
        Oi = np.zeros((rows.size, V.shape[1]))
        mi = np.full(rows.size, -np.inf)
        li = np.zeros(rows.size)
        for j0 in range(0, Nk, Bc):
            cols = np.arange(j0, min(Nk, j0 + Bc))
            # step 1: block scores
            S = scale * (Q[rows] @ K[cols].T)
            ok = allowed(rows, Nk, causal, block_mask, kv_len)[:, cols]
            S = np.where(ok, S, -np.inf)
            # step 2: block statistics
            mt = S.max(axis=1)
            Pt = _w(S, mt[:, None])
            lt = Pt.sum(axis=1)
            # step 3: running statistics
            mn, ln = merge(mi, li, mt, lt)
            # step 4: running output, normalised by the new l
            a = _w(mi, mn) * li
            b = _w(mt, mn)
            inv = np.where(ln > 0, 1.0 / np.where(ln > 0, ln, 1.0), 0.0)
            Oi = inv[:, None] * (a[:, None] * Oi + b[:, None] * (Pt @ V[cols]))
            mi, li = mn, ln
        O[rows], m_all[rows], l_all[rows] = Oi, mi, li
    return O, m_all, l_all
