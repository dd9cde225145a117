"""The dense definition restricted to allowed 128x128 cells.

Test infrastructure only (see the package docstring).

For query cell i, every key outside the cells (i, j) that survive the mask
(block_mask[i][j] = 1, j <= i when causal, 128*j < kv_len) has score -inf and
probability exactly 0, so the softmax over the gathered keys of the surviving
cells equals the softmax over all N keys.  This is the same definition as
``attention``, evaluated at a fraction of the cost; the elementwise masks
inside the surviving cells are applied by ``attention.allowed`` on the
gathered key positions.  Used for the 16K and 64K workloads and for sampled
rows / columns; pinned against ``attention`` by the tests.

``head_stats`` also returns D_i = sum_j P_ij dP_ij (the chain-rule form, see
``attention``), needed by sampled backward columns.
"""
from __future__ import annotations

import numpy as np

from .attention import CELL, _probs, allowed


def cell_keys(i_cell, N, causal, block_mask, kv_len, cell=CELL):
    """Key positions of the surviving cells of query cell i_cell, ascending."""
    T = -(-N // cell)
    L = N if kv_len is None else int(kv_len)
    j = np.arange(T)
    keep = (j * cell < L)
    if block_mask is not None:
        keep &= np.asarray(block_mask[i_cell]).astype(bool)
    if causal:
        keep &= j <= i_cell
    keys = [np.arange(cell * c, min(N, cell * (c + 1))) for c in np.flatnonzero(keep)]
    return np.concatenate(keys) if keys else np.zeros(0, np.int64)


def _row_probs(Q, K, rows, keys, scale, causal, block_mask, kv_len):
    S = scale * (Q[rows] @ K[keys].T)
    ok = allowed(rows, K.shape[0], causal, block_mask, kv_len, keys=keys)
    return _probs(np.where(ok, S, -np.inf))


def head_forward_rows(Q, K, V, scale, rows, causal=False, block_mask=None, kv_len=None):
    """O[rows], lse[rows] for one (b, h); rows may be any query positions."""
    Q = np.asarray(Q, np.float64)
    K = np.asarray(K, np.float64)
    V = np.asarray(V, np.float64)
    rows = np.asarray(rows, np.int64)
    N = K.shape[0]
    O = np.zeros((rows.size, V.shape[1]))
    lse = np.full(rows.size, -np.inf)
    for c in np.unique(rows // CELL):
        sel = np.flatnonzero(rows // CELL == c)
        keys = cell_keys(c, N, causal, block_mask, kv_len)
        if keys.size == 0:
            continue
        P, lse[sel] = _row_probs(Q, K, rows[sel], keys, scale, causal, block_mask, kv_len)
        O[sel] = P @ V[keys]
    return O, lse


def head_backward_rows(Q, K, V, dO, scale, rows, causal=False, block_mask=None, kv_len=None):
    """dQ[rows] for one (b, h)."""
    Q = np.asarray(Q, np.float64)
    K = np.asarray(K, np.float64)
    V = np.asarray(V, np.float64)
    dO = np.asarray(dO, np.float64)
    rows = np.asarray(rows, np.int64)
    N = K.shape[0]
    dQ = np.zeros((rows.size, Q.shape[1]))
    for c in np.unique(rows // CELL):
        sel = np.flatnonzero(rows // CELL == c)
        keys = cell_keys(c, N, causal, block_mask, kv_len)
        if keys.size == 0:
            continue
        P, _ = _row_probs(Q, K, rows[sel], keys, scale, causal, block_mask, kv_len)
        dP = dO[rows[sel]] @ V[keys].T
        D = (P * dP).sum(axis=1)
        dQ[sel] = scale * ((P * (dP - D[:, None])) @ K[keys])
    return dQ


def head_forward(Q, K, V, scale, causal=False, block_mask=None, kv_len=None):
    """O and lse for all rows of one (b, h)."""
    return head_forward_rows(Q, K, V, scale, np.arange(Q.shape[0]), causal, block_mask, kv_len)


def head_backward(Q, K, V, dO, scale, causal=False, block_mask=None, kv_len=None, key_cols=None):
    """dQ, dK, dV for one (b, h); with key_cols given, dK and dV are returned
    only for those key positions (dQ is then None)."""
    Q = np.asarray(Q, np.float64)
    K = np.asarray(K, np.float64)
    V = np.asarray(V, np.float64)
    dO = np.asarray(dO, np.float64)
    N = Q.shape[0]
    T = -(-N // CELL)
    want_all = key_cols is None
    dK = np.zeros_like(K)
    dV = np.zeros_like(V)
    dQ = np.zeros_like(Q) if want_all else None
    keep = None if want_all else np.zeros(N, bool)
    if keep is not None:
        keep[np.asarray(key_cols)] = True
    for c in range(T):
        rows = np.arange(c * CELL, min(N, (c + 1) * CELL))
        keys = cell_keys(c, N, causal, block_mask, kv_len)
        if keys.size == 0:
            continue
        if keep is not None:
            if not keep[keys].any():
                continue
        P, _ = _row_probs(Q, K, rows, keys, scale, causal, block_mask, kv_len)
        dP = dO[rows] @ V[keys].T
        D = (P * dP).sum(axis=1)
        dS = P * (dP - D[:, None])
        if keep is not None:
            sub = keep[keys]
            ks = keys[sub]
            dV[ks] += P[:, sub].T @ dO[rows]
            dK[ks] += scale * (dS[:, sub].T @ Q[rows])
        else:
            dV[keys] += P.T @ dO[rows]
            dK[keys] += scale * (dS.T @ Q[rows])
            dQ[rows] = scale * (dS @ K[keys])
    if keep is not None:
        cols = np.asarray(key_cols)
        return None, dK[cols], dV[cols]
    return dQ, dK, dV
