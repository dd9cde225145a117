"""Pins of the CPU oracle against what the pages and the mathematics fix.

None of these compares the oracle with itself: each check is a closed form, an
identity, a brute-force loop written independently, a library routine, or a
finite-difference derivative of the forward definition.
"""
import itertools
import json
import math
import os

import numpy as np
import pytest

from oracle import attention, online, sparse, visits
from workloads import band_random_mask

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def rand(rng, *shape, s=1.0):
    return rng.standard_normal(shape) * s


# ---------------------------------------------------------------- softmax / P

def test_softmax_rows_sum_to_one(rng):
    S = rand(rng, 37, 53, s=5.0)
    S[3, :] = -np.inf                    # a fully masked row
    S[5, ::2] = -np.inf
    P, lse = attention._probs(S)
    sums = P.sum(axis=1)
    assert np.all(np.abs(np.delete(sums, 3) - 1.0) <= 1e-14)
    assert np.all(P[3] == 0) and lse[3] == -np.inf
    assert np.all(P[5, ::2] == 0)


def test_safe_softmax_large_scores_one_hot():
    # safe softmax with the row max subtracted (bornlex "Tiling"): huge scores stay finite
    S = np.array([[1e4, -1e4, 0.0], [-1e4, -1e4 + 1.0, -2e4]])
    P, lse = attention._probs(S)
    assert np.all(np.isfinite(P))
    assert np.allclose(P[0], [1.0, 0.0, 0.0], atol=0)
    e = math.exp(1.0)
    assert abs(P[1, 1] - e / (1 + e)) < 1e-15 and abs(P[1, 0] - 1 / (1 + e)) < 1e-15
    assert lse[0] == 1e4


# ---------------------------------------------------------------- forward closed forms

def test_hand_example_golden():
    g = json.load(open(os.path.join(GOLD, "hand_example_n2.json")))
    q, k, v = (np.array(g[x]) for x in ("q", "k", "v"))
    O, lse = attention.head_forward(q, k, v, g["scale"])
    assert np.allclose(O, g["O"], rtol=0, atol=1e-15)
    assert np.allclose(lse, g["lse"], rtol=0, atol=1e-15)
    O, lse = attention.head_forward(q, k, v, g["scale"], causal=True)
    assert np.allclose(O, g["causal_O"], rtol=0, atol=1e-15)
    assert np.allclose(lse, g["causal_lse"], rtol=0, atol=1e-15)


@pytest.mark.parametrize("causal,use_len,use_mask", list(itertools.product([0, 1], [0, 1], [0, 1])))
def test_zero_query_gives_mean_of_allowed_values(rng, causal, use_len, use_mask):
    N, d = 300, 8
    K, V = rand(rng, N, d), rand(rng, N, d)
    Q = np.zeros((N, d))
    L = 213 if use_len else None
    bm = None
    if use_mask:
        bm = np.ones((3, 3), np.uint8)
        bm[2, 1] = 0
        bm[1, 0] = 0
    O, lse = attention.head_forward(Q, K, V, 0.7, causal=bool(causal), block_mask=bm, kv_len=L)
    for i in range(N):
        js = [j for j in range(N)
              if (not causal or j <= i) and (L is None or j < L)
              and (bm is None or bm[i // 128][j // 128])]
        if not js:
            assert np.all(O[i] == 0) and lse[i] == -np.inf
            continue
        assert np.allclose(O[i], V[js].mean(axis=0), rtol=0, atol=1e-13)
        assert abs(lse[i] - math.log(len(js))) < 1e-13


def test_single_key_gives_value(rng):
    q, k, v = rand(rng, 1, 5), rand(rng, 1, 5), rand(rng, 1, 5)
    O, lse = attention.head_forward(q, k, v, 0.3)
    assert np.array_equal(O, v)
    assert abs(lse[0] - 0.3 * float(q[0] @ k[0])) < 1e-15


def test_shift_invariances(rng):
    N, d = 70, 6
    Q, K, V = rand(rng, N, d), rand(rng, N, d), rand(rng, N, d)
    u, c = rand(rng, d), rand(rng, d)
    O, _ = attention.head_forward(Q, K, V, 0.5, causal=True)
    O2, _ = attention.head_forward(Q, K + u, V, 0.5, causal=True)   # every score of a row shifts equally
    O3, _ = attention.head_forward(Q, K, V + c, 0.5, causal=True)   # rows of P sum to 1
    assert np.allclose(O2, O, atol=1e-13)
    assert np.allclose(O3, O + c, atol=1e-13)


def test_brute_force_loops(rng):
    """Pure-Python loops with math.exp, no numpy reductions: the definition term by term."""
    N, d, scale = 9, 3, 0.8
    Q, K, V = rand(rng, N, d), rand(rng, N, d), rand(rng, N, d)
    bm = np.array([[1]], np.uint8)
    for causal, L in [(False, None), (True, None), (False, 6), (True, 4)]:
        O, lse = attention.head_forward(Q, K, V, scale, causal=causal, block_mask=bm, kv_len=L)
        for i in range(N):
            js = [j for j in range(N) if (not causal or j <= i) and (L is None or j < L)]
            s = {j: scale * sum(Q[i, t] * K[j, t] for t in range(d)) for j in js}
            if not js:
                assert lse[i] == -np.inf
                continue
            z = sum(math.exp(s[j]) for j in js)
            for t in range(d):
                ref = sum(math.exp(s[j]) / z * V[j, t] for j in js)
                assert abs(O[i, t] - ref) < 1e-13
            assert abs(lse[i] - math.log(z)) < 1e-13


@pytest.mark.parametrize("causal", [False, True])
def test_against_torch_sdpa_cpu_fp64(rng, causal):
    """Cross-check with torch.nn.functional.scaled_dot_product_attention (the PyTorch
    routine named in datacamp "Penjelasan Flash Attention", "Integrasi PyTorch"),
    on the CPU in float64, with a boolean mask (no fully-masked rows)."""
    torch = pytest.importorskip("torch")
    B, H, N, d = 2, 3, 200, 16
    q, k, v = rand(rng, B, H, N, d), rand(rng, B, H, N, d), rand(rng, B, H, N, d)
    kv_len = np.array([150, 200])
    bm = np.array([[1, 0], [1, 1]], np.uint8)
    O, _ = attention.forward(q, k, v, 0.3, causal=causal, block_mask=bm, kv_len=kv_len)
    t = [torch.from_numpy(x) for x in (q, k, v)]
    for b in range(B):
        ok = attention.allowed(np.arange(N), N, causal, bm, int(kv_len[b]))
        ref = torch.nn.functional.scaled_dot_product_attention(
            t[0][b:b + 1], t[1][b:b + 1], t[2][b:b + 1],
            attn_mask=torch.from_numpy(ok), scale=0.3).numpy()
        assert np.abs(O[b] - ref[0]).max() < 1e-12


# ---------------------------------------------------------------- merge and tiled method

def test_two_block_merge_equals_full_softmax(rng):
    B = 16
    for trial in range(20):
        x1, x2 = rand(rng, B, s=3.0), rand(rng, B, s=3.0)
        if trial == 1:
            x1[:] = -np.inf                       # an empty block
        x = np.concatenate([x1, x2])
        m1, m2 = (np.max(x1), np.max(x2))
        l1 = np.exp(x1 - m1).sum() if np.isfinite(m1) else 0.0
        l2 = np.exp(x2 - m2).sum()
        m, l = online.merge(m1, l1, m2, l2)
        assert m == np.max(x)
        assert abs(l - np.exp(x - np.max(x)).sum()) <= 1e-14 * l
        f1 = np.exp(x1 - m1) if np.isfinite(m1) else np.zeros(B)
        f = online.merge_f(m1, f1, m2, np.exp(x2 - m2))
        assert np.allclose(f / l, np.exp(x - x.max()) / np.exp(x - x.max()).sum(), rtol=0, atol=1e-15)
        # e^(x1 - m(x1)) e^(m(x1) - m(x)) = e^(x1 - m(x))
        if np.isfinite(m1):
            assert np.allclose(np.exp(x1 - m1) * np.exp(m1 - m), np.exp(x1 - m), rtol=1e-14, atol=0)


@pytest.mark.parametrize("Br,Bc", [(16, 16), (32, 8), (64, 128), (7, 13)])
@pytest.mark.parametrize("causal", [False, True])
def test_tiled_method_equals_definition(rng, Br, Bc, causal):
    N, d = 150, 8
    Q, K, V = rand(rng, N, d), rand(rng, N, d), rand(rng, N, d)
    bm = np.array([[1, 1], [0, 1]], np.uint8)
    for mask, L in [(None, None), (bm, 97)]:
        O, lse = attention.head_forward(Q, K, V, 0.4, causal=causal, block_mask=mask, kv_len=L)
        Ot, m, l = online.tiled_head_forward(Q, K, V, 0.4, Br, Bc, causal, mask, L)
        assert np.abs(O - Ot).max() < 1e-13
        fin = np.isfinite(lse)
        assert np.abs(lse[fin] - (m[fin] + np.log(l[fin]))).max() < 1e-13


# ---------------------------------------------------------------- backward

def _loss(Q, K, V, dO, scale, **kw):
    O, _ = attention.head_forward(Q, K, V, scale, **kw)
    return float((O * dO).sum())


@pytest.mark.parametrize("kw", [dict(), dict(causal=True), dict(kv_len=9),
                                dict(causal=True, kv_len=11)])
def test_backward_finite_differences(rng, kw):
    N, d, scale, h = 13, 5, 0.7, 1e-6
    Q, K, V, dO = (rand(rng, N, d) for _ in range(4))
    dQ, dK, dV = attention.head_backward(Q, K, V, dO, scale, **kw)
    for X, G in ((Q, dQ), (K, dK), (V, dV)):
        num = np.zeros_like(X)
        for idx in np.ndindex(*X.shape):
            old = X[idx]
            X[idx] = old + h
            lp = _loss(Q, K, V, dO, scale, **kw)
            X[idx] = old - h
            lm = _loss(Q, K, V, dO, scale, **kw)
            X[idx] = old
            num[idx] = (lp - lm) / (2 * h)
        assert np.abs(num - G).max() <= 1e-6 * max(1.0, np.abs(G).max())


def test_backward_invariants(rng):
    N, d = 90, 7
    Q, K, V, dO = (rand(rng, N, d) for _ in range(4))
    L = 80
    dQ, dK, dV = attention.head_backward(Q, K, V, dO, 0.6, causal=True, kv_len=L)
    assert np.abs(dK.sum(axis=0)).max() < 1e-12          # rows of dS sum to 0
    assert np.allclose(dV.sum(axis=0), dO.sum(axis=0), atol=1e-12)   # every row sees key 0
    assert np.all(dK[L:] == 0) and np.all(dV[L:] == 0)
    u = rand(rng, d)
    dQ2, _, _ = attention.head_backward(Q, K + u, V, dO, 0.6, causal=True, kv_len=L)
    assert np.allclose(dQ2, dQ, atol=1e-12)


def test_backward_against_torch_autograd_fp64(rng):
    torch = pytest.importorskip("torch")
    N, d, scale = 64, 8, 0.35
    Q, K, V, dO = (rand(rng, N, d) for _ in range(4))
    dQ, dK, dV = attention.head_backward(Q, K, V, dO, scale, causal=True)
    t = [torch.tensor(x, requires_grad=True) for x in (Q, K, V)]
    out = torch.nn.functional.scaled_dot_product_attention(
        t[0][None], t[1][None], t[2][None], is_causal=True, scale=scale)[0]
    (out * torch.from_numpy(dO)).sum().backward()
    for a, b in zip((dQ, dK, dV), t):
        assert np.abs(a - b.grad.numpy()).max() < 1e-12


# ---------------------------------------------------------------- gathered (sparse) form

@pytest.mark.parametrize("N", [300, 4096])
def test_sparse_form_equals_dense(rng, N):
    d = 16
    T = -(-N // 128)
    Q, K, V, dO = (rand(rng, N, d) for _ in range(4))
    bm = band_random_mask(T, 7)
    for causal, L in [(False, None), (True, None), (False, N - 77)]:
        O, lse = attention.head_forward(Q, K, V, 0.25, causal=causal, block_mask=bm, kv_len=L)
        Os, lses = sparse.head_forward(Q, K, V, 0.25, causal, bm, L)
        assert np.abs(O - Os).max() <= 1e-12 * max(1, np.abs(O).max())
        fin = np.isfinite(lse)
        assert np.array_equal(fin, np.isfinite(lses))
        assert np.abs(lse[fin] - lses[fin]).max() < 1e-12
        if N > 1000:
            continue
        g = attention.head_backward(Q, K, V, dO, 0.25, causal, bm, L)
        gs = sparse.head_backward(Q, K, V, dO, 0.25, causal, bm, L)
        for a, b in zip(g, gs):
            assert np.abs(a - b).max() <= 1e-12 * max(1, np.abs(a).max())
        cols = np.array([0, 5, 130, N - 1])
        _, dKc, dVc = sparse.head_backward(Q, K, V, dO, 0.25, causal, bm, L, key_cols=cols)
        assert np.abs(dKc - g[1][cols]).max() < 1e-12
        assert np.abs(dVc - g[2][cols]).max() < 1e-12
        rows = np.array([1, 128, 129, N - 1])
        dQr = sparse.head_backward_rows(Q, K, V, dO, 0.25, rows, causal, bm, L)
        assert np.abs(dQr - g[0][rows]).max() < 1e-12


# ---------------------------------------------------------------- visit set

def test_expected_visits_hand_enumerated():
    bm = np.array([[1, 0, 1], [0, 1, 1], [1, 1, 0]], np.uint8)
    N = 300                                  # 3 cells, last one partial
    ev = visits.expected_visits(2, N, causal=True, block_mask=bm, kv_len=[300, 129])
    want0 = [[1, 0, 0], [0, 1, 0], [1, 1, 0]]
    want1 = [[1, 0, 0], [0, 1, 0], [1, 1, 0]]   # kv_len 129 keeps cells 0 and 1 (128 < 129)
    assert ev[0].tolist() == want0 and ev[1].tolist() == want1
    ev = visits.expected_visits(1, N, causal=False, block_mask=None, kv_len=[128])
    assert ev[0].tolist() == [[1, 0, 0]] * 3
    ev = visits.expected_visits(1, 1, causal=True)
    assert ev.tolist() == [[[1]]]


# ---------------------------------------------------------------- fewer queries than keys

def test_bottom_right_causal_by_brute_force():
    """Nq queries against Nk >= Nq keys, causal with the queries as the last Nq
    positions: query i may see key j iff j <= i + (Nk - Nq).  Pure-Python loops."""
    import math
    rng = np.random.Generator(np.random.PCG64(60))
    Nq, Nk, d, scale = 5, 9, 3, 0.7
    Q, K, V = rng.standard_normal((Nq, d)), rng.standard_normal((Nk, d)), rng.standard_normal((Nk, d))
    O, lse = attention.head_forward(Q, K, V, scale, causal=True, causal_offset=Nk - Nq)
    for i in range(Nq):
        keys = [j for j in range(Nk) if j <= i + Nk - Nq]
        s = [scale * sum(Q[i, t] * K[j, t] for t in range(d)) for j in keys]
        m = max(s)
        w = [math.exp(x - m) for x in s]
        den = sum(w)
        for t in range(d):
            assert abs(O[i, t] - sum(wj * V[j, t] for wj, j in zip(w, keys)) / den) < 1e-12
        assert abs(lse[i] - (m + math.log(den))) < 1e-12
    # with as many queries as keys the offset is zero and this is the top-left causal mask
    O1, _ = attention.head_forward(Q, K[:Nq], V[:Nq], scale, causal=True, causal_offset=0)
    O2, _ = attention.head_forward(Q, K[:Nq], V[:Nq], scale, causal=True)
    assert np.array_equal(O1, O2)


def test_key_splits_merge_to_the_full_softmax():
    """Splitting the keys into contiguous ranges and combining the per-range
    (m, l, O) with the pages' two-block merge gives the full result (what a
    split-key forward relies on)."""
    rng = np.random.Generator(np.random.PCG64(61))
    Nq, Nk, d, scale = 7, 50, 4, 0.5
    Q, K, V = rng.standard_normal((Nq, d)), rng.standard_normal((Nk, d)), rng.standard_normal((Nk, d))
    O, lse = attention.head_forward(Q, K, V, scale, causal=True, causal_offset=Nk - Nq)
    ok = attention.allowed(np.arange(Nq), Nk, causal=True, causal_offset=Nk - Nq)
    m_run = np.full(Nq, -np.inf)
    l_run = np.zeros(Nq)
    acc = np.zeros((Nq, d))
    for lo, hi in ((0, 13), (13, 31), (31, 50)):
        S = np.where(ok[:, lo:hi], scale * Q @ K[lo:hi].T, -np.inf)
        m_b = S.max(axis=1)
        live = np.isfinite(m_b)
        E = np.where(live[:, None], np.exp(S - np.where(live, m_b, 0.0)[:, None]), 0.0)
        l_b = E.sum(axis=1)
        o_b = E @ V[lo:hi]                                   # unnormalised block output
        m_new, l_new = online.merge(m_run, l_run, m_b, l_b)
        wa = np.where(np.isfinite(m_run), np.exp(m_run - m_new), 0.0)
        wb = np.where(live, np.exp(m_b - m_new), 0.0)
        acc = wa[:, None] * acc + wb[:, None] * o_b
        m_run, l_run = m_new, l_new
    assert np.allclose(acc / l_run[:, None], O, rtol=1e-12, atol=1e-12)
    assert np.allclose(m_run + np.log(l_run), lse, rtol=1e-12, atol=1e-12)


def test_offset_causal_is_the_tail_of_the_square_problem():
    """The last Nq rows of the square causal problem over Nk positions are the
    offset problem with those Nq queries; with more queries than keys the first
    Nq - Nk rows have no key (O = 0, lse = -inf) and the rest see j <= i - (Nq - Nk)."""
    rng = np.random.Generator(np.random.PCG64(62))
    Nk, d, scale = 40, 5, 0.6
    Q, K, V = rng.standard_normal((Nk, d)), rng.standard_normal((Nk, d)), rng.standard_normal((Nk, d))
    O_sq, lse_sq = attention.head_forward(Q, K, V, scale, causal=True)
    for Nq in (1, 7, 40):
        O, lse = attention.head_forward(Q[Nk - Nq:], K, V, scale, causal=True, causal_offset=Nk - Nq)
        assert np.allclose(O, O_sq[Nk - Nq:], rtol=1e-13, atol=1e-13)
        assert np.allclose(lse, lse_sq[Nk - Nq:], rtol=1e-13, atol=1e-13)
    Nq = 46
    Qx = rng.standard_normal((Nq, d))
    O, lse = attention.head_forward(Qx, K, V, scale, causal=True, causal_offset=Nk - Nq)
    assert np.all(O[:Nq - Nk] == 0) and np.all(np.isneginf(lse[:Nq - Nk]))
    # row Nq - Nk + t sees keys 0..t, exactly like square row t
    Osq2, lsesq2 = attention.head_forward(Qx[Nq - Nk:], K, V, scale, causal=True)
    assert np.allclose(O[Nq - Nk:], Osq2, rtol=1e-13, atol=1e-13)
    assert np.allclose(lse[Nq - Nk:], lsesq2, rtol=1e-13, atol=1e-13)


# ---------------------------------------------------------------- batched backward and row blocks

def _autograd_grads(torch, Q, K, V, dO, scale, ok):
    """dQ, dK, dV of sum(O * dO) by torch autograd through the CPU fp64
    scaled_dot_product_attention with a boolean mask (True = allowed)."""
    t = [torch.tensor(x, requires_grad=True) for x in (Q, K, V)]
    out = torch.nn.functional.scaled_dot_product_attention(
        t[0][None], t[1][None], t[2][None], attn_mask=torch.from_numpy(ok), scale=scale)[0]
    (out * torch.from_numpy(dO)).sum().backward()
    return [x.grad.numpy() for x in t]


def test_batched_backward_per_batch_kv_len_against_autograd(rng):
    """attention.backward picks kv_len[b] for batch entry b and the block mask
    for every head: each (b, h) is checked against autograd with that entry's
    own mask, so a wrong batch index or a dropped mask condition fails."""
    torch = pytest.importorskip("torch")
    B, H, N, d, scale = 2, 2, 300, 8, 0.3
    q, k, v, do = (rand(rng, B, H, N, d) for _ in range(4))
    kv_len = np.array([150, 300])
    bm = np.array([[1, 0, 0], [1, 1, 0], [1, 0, 1]], np.uint8)   # first column kept: no empty row
    dq, dk, dv = attention.backward(q, k, v, do, scale, causal=True, block_mask=bm, kv_len=kv_len)
    for b in range(B):
        ok = attention.allowed(np.arange(N), N, True, bm, int(kv_len[b]))
        assert ok.any(axis=1).all()
        for h in range(H):
            ref = _autograd_grads(torch, q[b, h], k[b, h], v[b, h], do[b, h], scale, ok)
            for got, want in zip((dq[b, h], dk[b, h], dv[b, h]), ref):
                assert np.abs(got - want).max() < 1e-12
    # the padded keys of entry 0 get no gradient, those of entry 1 do
    assert np.all(dk[0, :, 150:] == 0) and np.all(dv[0, :, 150:] == 0)
    assert np.abs(dv[1, :, 150:]).max() > 0


@pytest.mark.parametrize("row_block", [64, 100, 299])
def test_head_backward_accumulates_across_row_blocks(rng, row_block):
    """head_backward walks the queries in row blocks and adds every block's
    contribution to dK and dV: with several blocks (N = 300) it must equal
    autograd, which a '=' in place of '+=' would break."""
    torch = pytest.importorskip("torch")
    N, d, scale = 300, 8, 0.35
    Q, K, V, dO = (rand(rng, N, d) for _ in range(4))
    ok = attention.allowed(np.arange(N), N, causal=True, kv_len=270)
    got = attention.head_backward(Q, K, V, dO, scale, causal=True, kv_len=270, row_block=row_block)
    ref = _autograd_grads(torch, Q, K, V, dO, scale, ok)
    for a, b in zip(got, ref):
        assert np.abs(a - b).max() < 1e-12
