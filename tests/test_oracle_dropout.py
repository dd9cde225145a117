"""Pins of the dropout oracle (oracle/dropout.py) against facts fixed outside it:
the generator's published known-answer vectors, the no-dropout definition,
the keep rate, finite differences, and the delta identity."""
import numpy as np
import pytest

from oracle import attention, dropout

# Known-answer vectors of Philox4x32-10 published with the generator (Salmon,
# Moraes, Dror and Shaw, "Parallel Random Numbers: As Easy as 1, 2, 3", SC 2011,
# and its reference implementation's test vectors): counter, key -> output.
PHILOX_KAT = [
    ((0x00000000, 0x00000000, 0x00000000, 0x00000000), (0x00000000, 0x00000000),
     (0x6627E8D5, 0xE169C58D, 0xBC57AC4C, 0x9B00DBD8)),
    ((0xFFFFFFFF, 0xFFFFFFFF, 0xFFFFFFFF, 0xFFFFFFFF), (0xFFFFFFFF, 0xFFFFFFFF),
     (0x408F276D, 0x41C83B0E, 0xA20BC7C6, 0x6D5451FD)),
    ((0x243F6A88, 0x85A308D3, 0x13198A2E, 0x03707344), (0xA4093822, 0x299F31D0),
     (0xD16CFE09, 0x94FDCCEB, 0x5001E420, 0x24126EA1)),
]


@pytest.mark.parametrize("case", PHILOX_KAT, ids=["zero", "ones", "pi"])
def test_philox_known_answers(case):
    ctr, key, want = case
    got = dropout.philox4x32_10(*ctr, *key)
    assert [int(x) for x in got] == list(want)


def test_philox_vectorised_over_counters():
    """Each element of a batched call equals the scalar call on its counter."""
    rng = np.random.Generator(np.random.PCG64(40))
    c = rng.integers(0, 2 ** 32, size=(4, 37), dtype=np.uint64)
    batch = dropout.philox4x32_10(*c, 0x1234, 0xABCD)
    for n in (0, 5, 36):
        one = dropout.philox4x32_10(*(int(x[n]) for x in c), 0x1234, 0xABCD)
        assert [int(w[n]) for w in batch] == [int(w) for w in one]


def small(N=40, d=8, seed=41, causal=False):
    rng = np.random.Generator(np.random.PCG64(seed))
    q, k, v, do = (rng.standard_normal((N, d)) for _ in range(4))
    return q, k, v, do


def test_zero_threshold_is_plain_attention():
    """t = 0 keeps every entry with scale 1: exactly the definition."""
    q, k, v, do = small()
    for kw in (dict(), dict(causal=True), dict(kv_len=23)):
        O, lse = dropout.head_forward(q, k, v, 0.3, 5, 0, 99, **kw)
        O0, lse0 = attention.head_forward(q, k, v, 0.3, **kw)
        assert np.array_equal(O, O0) and np.array_equal(lse, lse0)
        g = dropout.head_backward(q, k, v, do, 0.3, 5, 0, 99, **kw)
        g0 = attention.head_backward(q, k, v, do, 0.3, **kw)
        for a, b in zip(g, g0):
            assert np.array_equal(a, b)


@pytest.mark.parametrize("t", [1, 64, 128, 255])
def test_keep_rate_matches_threshold(t):
    """Over 512 x 512 entries the kept fraction is 1 - t/256 within 5 sigma."""
    Z = dropout.keep_scale(3, np.arange(512), np.arange(512), t, 2024)
    frac = float((Z > 0).mean())
    p_keep = 1 - t / 256
    sigma = np.sqrt(p_keep * (1 - p_keep) / Z.size)
    assert abs(frac - p_keep) <= 5 * sigma + 1e-12
    assert np.allclose(Z[Z > 0], 256.0 / (256 - t))


def test_random_bytes_are_uniform_and_depend_on_every_coordinate():
    u = dropout.random_bytes(0, np.arange(256), np.arange(1024), 7)
    counts = np.bincount(u.ravel(), minlength=256)
    expect = u.size / 256
    chi2 = float(((counts - expect) ** 2 / expect).sum())
    assert 255 - 6 * np.sqrt(2 * 255) < chi2 < 255 + 6 * np.sqrt(2 * 255)
    base = dropout.random_bytes(0, np.arange(8), np.arange(8), 7)
    for other in (dropout.random_bytes(1, np.arange(8), np.arange(8), 7),          # head
                  dropout.random_bytes(0, np.arange(8), np.arange(8), 8),          # seed low word
                  dropout.random_bytes(0, np.arange(8), np.arange(8), 7 + (1 << 32)),   # seed high word
                  dropout.random_bytes(0, np.arange(8, 16), np.arange(8), 7),      # queries
                  dropout.random_bytes(0, np.arange(8), np.arange(8, 16), 7)):     # keys
        assert (other != base).mean() > 0.9


def test_byte_layout_within_a_block():
    """Entry (i, j) is byte (j & 3) of word (i & 3) of the call on counter (j>>2, i>>2, bh, 0)."""
    bh, seed = 9, 0x0123456789ABCDEF
    u = dropout.random_bytes(bh, np.arange(8), np.arange(8), seed)
    for i in (0, 3, 5):
        for j in (0, 2, 7):
            w = dropout.philox4x32_10(j >> 2, i >> 2, bh, 0, seed & 0xFFFFFFFF, seed >> 32)[i & 3]
            assert u[i, j] == (int(w) >> (8 * (j & 3))) & 0xFF


@pytest.mark.parametrize("kw", [dict(), dict(causal=True), dict(kv_len=29)])
def test_dropout_gradients_finite_differences(kw):
    """dQ, dK, dV of L = sum(O * dO) with a fixed dropout pattern, against
    central differences (1e-6 relative)."""
    q, k, v, do = small(N=24, d=6, seed=42)
    t, seed, bh, scale = 77, 1234, 2, 0.4

    def loss(q_, k_, v_):
        O, _ = dropout.head_forward(q_, k_, v_, scale, bh, t, seed, **kw)
        return float((O * do).sum())

    g = dropout.head_backward(q, k, v, do, scale, bh, t, seed, **kw)
    eps = 1e-6
    rng = np.random.Generator(np.random.PCG64(43))
    for which, grad in zip(range(3), g):
        for _ in range(6):
            i, j = int(rng.integers(24)), int(rng.integers(6))
            args = [q.copy(), k.copy(), v.copy()]
            args[which][i, j] += eps
            up = loss(*args)
            args[which][i, j] -= 2 * eps
            dn = loss(*args)
            fd = (up - dn) / (2 * eps)
            assert abs(fd - grad[i, j]) <= 1e-6 * max(1.0, abs(fd)), (which, i, j, fd, grad[i, j])


def test_delta_equals_rowsum_of_dO_times_O_with_dropout():
    """D_i = sum_j P_ij dP_ij equals dO_i . O_i, so the preprocess kernel is unchanged."""
    q, k, v, do = small(N=32, d=8, seed=44)
    t, seed, bh, scale = 100, 5, 1, 0.5
    O, _ = dropout.head_forward(q, k, v, scale, bh, t, seed)
    S = scale * (q @ k.T)
    P, _ = attention._probs(S)
    Z = dropout.keep_scale(bh, np.arange(32), np.arange(32), t, seed)
    D = (P * ((do @ v.T) * Z)).sum(axis=1)
    assert np.allclose(D, (do * O).sum(axis=1), rtol=1e-12, atol=1e-12)


def test_dropout_is_unbiased_in_expectation():
    """Averaged over seeds, the dropout output approaches the plain output."""
    q, k, v, _ = small(N=16, d=4, seed=45)
    O0, _ = attention.head_forward(q, k, v, 0.5)
    acc = np.zeros_like(O0)
    n = 400
    for s in range(n):
        acc += dropout.head_forward(q, k, v, 0.5, 0, 128, 1000 + s)[0]
    # per entry the estimate has standard error < max|V| / sqrt(n) (keep rate 1/2, scale 2)
    assert np.abs(acc / n - O0).max() < 5 * np.abs(v).max() / np.sqrt(n)


def test_dq_rows_equal_the_full_backward():
    """head_backward_rows (sampled rows, for long sequences) gives the same dQ
    rows as the full backward, under each mask setting."""
    q, k, v, do = small(N=40, d=6, seed=46)
    rows = np.array([0, 3, 17, 39])
    for kw in (dict(), dict(causal=True), dict(kv_len=21)):
        full = dropout.head_backward(q, k, v, do, 0.4, 3, 90, 77, **kw)[0]
        part = dropout.head_backward_rows(q, k, v, do, 0.4, 3, 90, 77, rows, **kw)
        assert np.allclose(part, full[rows], rtol=1e-13, atol=1e-13)
