"""GPU parity of the dropout entry points (fa_fwd_dropout / fa_bwd_dropout)
against the dropout oracle.

The keep pattern itself is checked bit for bit where an identity operand
makes it visible: with V = I (N <= d) the forward output is O = P * Z, with
dO = I the backward gives dV = (P * Z)^T, and with K = I the backward gives
dQ = scale dS, so a single wrong keep bit shows up as a wrong element."""
import numpy as np
import pytest

from oracle import dropout as odrop
from workloads import band_random_mask, draw_kv_len, draw_qkvdo

from gpu_cases import TOL, compare_forward, compare_grad, host, say, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import exact_io_aware_flashattention_amd as fa
    fa.load_library()


def run(q, k, v, do, scale, t, seed, causal=False, block_mask=None, kv_len=None, backward=True):
    import torch

    import exact_io_aware_flashattention_amd as fa
    tq, tk, tv, tdo = (to_dev(x, "bf16") for x in (q, k, v, do))
    bm = None if block_mask is None else torch.from_numpy(block_mask).cuda()
    kl = None if kv_len is None else torch.from_numpy(np.asarray(kv_len, np.int32)).cuda()
    kw = dict(scale=scale, causal=causal, block_mask=bm, kv_len=kl, dropout_p=t / 256.0, seed=seed)
    o, lse = fa.fa_fwd(tq, tk, tv, **kw)
    out = {}
    if backward:
        dq, dk, dv = fa.fa_bwd(tq, tk, tv, o, tdo, lse, **kw)
    torch.cuda.synchronize()
    out["o"], out["lse"] = host(o), lse.cpu().numpy().astype(np.float64)
    if backward:
        out["dq"], out["dk"], out["dv"] = host(dq), host(dk), host(dv)
    return out


def allowed_mask(N, causal, kv=None):
    i, j = np.arange(N)[:, None], np.arange(N)[None, :]
    ok = np.ones((N, N), bool)
    if causal:
        ok &= j <= i
    if kv is not None:
        ok &= j < kv
    return ok


@pytest.mark.parametrize("N,causal,t", [(128, False, 64), (128, True, 200), (97, True, 1), (128, False, 255)])
def test_forward_keep_pattern_is_exact(N, causal, t):
    """V = I: O[i, j] = P_ij Z_ij, nonzero exactly where the oracle keeps (i, j)."""
    B, H, d, seed = 1, 3, 128, 0x9E3779B97F4A7C15 + N + t
    q, k, _, do = draw_qkvdo(B, H, N, d, "bf16", 1.0, 300 + N)
    v = np.zeros((B, H, N, d), np.float32)
    v[:, :, np.arange(N), np.arange(N)] = 1.0
    say(f"dropout keep pattern fwd: N={N} causal={causal} t={t}")
    out = run(q, k, v, do, 0.125, t, seed, causal=causal, backward=False)
    ok = allowed_mask(N, causal)
    for h in range(H):
        keep = odrop.random_bytes(h, np.arange(N), np.arange(N), seed) >= t
        got = out["o"][0, h][:, :N] != 0
        assert np.array_equal(got[ok], keep[ok]), f"head {h}: {np.argwhere(got != (keep & ok))[:5]}"
        assert not got[~ok].any()


@pytest.mark.parametrize("N,causal,t", [(128, False, 100), (90, True, 30)])
def test_backward_keep_pattern_is_exact(N, causal, t):
    """dO = I: dV[j, i] = P_ij Z_ij (nonzero exactly where kept); K = I:
    dQ = scale dS element-wise against the oracle."""
    B, H, d, seed = 1, 2, 128, 1234567 + N
    q, _, v, _ = draw_qkvdo(B, H, N, d, "bf16", 1.0, 310 + N)
    eye = np.zeros((B, H, N, d), np.float32)
    eye[:, :, np.arange(N), np.arange(N)] = 1.0
    _, k, _, do = draw_qkvdo(B, H, N, d, "bf16", 1.0, 320 + N)
    say(f"dropout keep pattern bwd (dO = I): N={N} causal={causal} t={t}")
    out = run(q, k, v, eye, 0.125, t, seed, causal=causal)
    ok = allowed_mask(N, causal)
    for h in range(H):
        keep = odrop.random_bytes(h, np.arange(N), np.arange(N), seed) >= t
        got = (out["dv"][0, h][:, :N] != 0).T          # [i, j]
        assert np.array_equal(got[ok], keep[ok]), f"head {h}"
    say(f"dropout dQ with K = I: N={N} causal={causal} t={t}")
    out = run(q, eye, v, do, 0.125, t, seed, causal=causal)
    for h in range(H):
        g = odrop.head_backward(q[0, h], eye[0, h], v[0, h], do[0, h], 0.125, h, t, seed, causal=causal)
        ref = g[0][:, :N]
        err = np.abs(out["dq"][0, h][:, :N] - ref)
        assert err.max() <= TOL["bf16"]["grad"] * np.abs(ref).max(), f"head {h}: {err.max()} vs {np.abs(ref).max()}"
        # Every entry: dQ_ij = scale P_ij (Z_ij dP_ij - D_i) with dP = dO V^T.
        # bf16 rounding moves it by a small fraction of the terms that cancel,
        # scale P (Z |dP| + |D|), while a wrong keep bit moves it by about
        # scale P Z |dP| -- the whole first term.
        S = 0.125 * (q[0, h].astype(np.float64) @ eye[0, h].T)
        S = np.where(allowed_mask(N, causal), S, -np.inf)
        P, _ = odrop._probs(S)
        Z = odrop.keep_scale(h, np.arange(N), np.arange(N), t, seed)
        dP = do[0, h].astype(np.float64) @ v[0, h].astype(np.float64).T
        D = (P * dP * Z).sum(axis=1, keepdims=True)
        terms = 0.125 * P * (Z * np.abs(dP) + np.abs(D))
        bad = err > 0.05 * terms + 1e-3 * terms.max()
        assert not bad.any(), f"head {h}: {np.argwhere(bad)[:5]}"


CASES = [
    # B, H, N, d, causal, kv, mask, t
    (2, 2, 200, 64, True, None, None, 51),
    (1, 3, 333, 128, False, "rand", None, 128),
    (2, 2, 256, 64, True, None, "band", 10),
    (1, 2, 513, 128, True, None, None, 230),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: "B{}H{}N{}d{}{}{}{}t{}".format(
    c[0], c[1], c[2], c[3], "c" if c[4] else "", "k" if c[5] else "", "m" if c[6] else "", c[7]))
def test_dropout_parity(case):
    B, H, N, d, causal, kv, mask, t = case
    seed = 0xABCDEF0123 + N
    q, k, v, do = draw_qkvdo(B, H, N, d, "bf16", 1.0, 330 + N)
    kv_len = draw_kv_len(B, 1, N, 340 + N) if kv else None
    bm = band_random_mask(-(-N // 128), 350 + N, n_random=1) if mask else None
    say(f"dropout parity {case}")
    out = run(q, k, v, do, 1 / np.sqrt(d), t, seed, causal=causal, block_mask=bm, kv_len=kv_len)
    O, lse = odrop.forward(q, k, v, 1 / np.sqrt(d), t, seed, causal=causal, block_mask=bm, kv_len=kv_len)
    # The bf16 tolerances are stated for attention outputs of magnitude <~ 1;
    # dropout scales kept entries by 1 / (1 - p) (up to ~10 here), and bf16's
    # half-ulp grows with the value, so O is compared after undoing that known
    # factor: (1 - p) O = sum_j P_ij keep_ij V_j has the plain magnitude.
    keep_frac = 1 - t / 256
    compare_forward(out["o"] * keep_frac, out["lse"], O * keep_frac, lse, "bf16", f"dropout {case}")
    g = odrop.backward(q, k, v, do, 1 / np.sqrt(d), t, seed, causal=causal, block_mask=bm, kv_len=kv_len)
    for name, a, r in zip(("dq", "dk", "dv"), (out["dq"], out["dk"], out["dv"]), g):
        compare_grad(a, r, "bf16", f"dropout {case} {name}")


def test_dropout_determinism_and_seed_dependence():
    q, k, v, do = draw_qkvdo(1, 2, 256, 64, "bf16", 1.0, 360)
    a = run(q, k, v, do, 0.125, 77, 42)
    b = run(q, k, v, do, 0.125, 77, 42)
    c = run(q, k, v, do, 0.125, 77, 43)
    for n in ("o", "dq", "dk", "dv"):
        assert np.array_equal(a[n], b[n]), n
        assert not np.array_equal(a[n], c[n]), n
    assert np.array_equal(a["lse"], c["lse"])      # lse does not depend on dropout


def test_zero_rate_equals_plain():
    import torch

    import exact_io_aware_flashattention_amd as fa
    q, k, v, do = draw_qkvdo(1, 2, 200, 128, "bf16", 1.0, 370)
    tq, tk, tv, tdo = (to_dev(x, "bf16") for x in (q, k, v, do))
    o0, l0 = fa.fa_fwd(tq, tk, tv, causal=True)
    o1, l1 = fa.fa_fwd(tq, tk, tv, causal=True, dropout_p=0.0, seed=9)
    o2, l2 = fa.fa_fwd(tq, tk, tv, causal=True, dropout_p=0.001, seed=9)   # rounds to t = 0
    torch.cuda.synchronize()
    assert torch.equal(o0, o1) and torch.equal(o0, o2) and torch.equal(l0, l2)


def test_dropout_full_size_sampled():
    """The long-context workload (B1 H16 N16384 d128 causal) with the rate and
    seed bench.py --dropout times (t = 26, seed 2024): sampled rows of O, lse
    and dQ on the first and last head against the dropout oracle."""
    from workloads import WORKLOADS, make_inputs
    w = WORKLOADS[4]
    inp = make_inputs(w)
    t, seed, N = 26, 2024, w.N
    say(f"dropout full size: t={t} seed={seed}")
    out = run(inp["q"], inp["k"], inp["v"], inp["do"], w.scale, t, seed, causal=True)
    rng = np.random.Generator(np.random.PCG64(380))
    rows = np.unique(np.concatenate([[0, 1, 127, 128, N // 2, N - 1], rng.integers(0, N, 34)]))
    keep_frac = 1 - t / 256
    for h in (0, w.H - 1):
        Q, K, V, dO = (inp[n][0, h] for n in ("q", "k", "v", "do"))
        O, lse = odrop.head_forward(Q, K, V, w.scale, h, t, seed, rows=rows, causal=True)
        compare_forward(out["o"][0, h][rows] * keep_frac, out["lse"][0, h][rows], O * keep_frac, lse, "bf16",
                        f"dropout full h{h}")
        dQ = odrop.head_backward_rows(Q, K, V, dO, w.scale, h, t, seed, rows, causal=True)
        compare_grad(out["dq"][0, h][rows], dQ, "bf16", f"dropout full h{h} dq rows")


@pytest.mark.parametrize("d", [64, 256])
def test_dropout_split_key_column(d):
    """Dropout with a block mask whose key columns are split over work-groups
    in dK/dV (chunk 16 cells, set columns visited by 40 query cells): the
    split partial sums, at d = 64 and at d = 256."""
    from test_parity import split_mask
    N = 40 * 128 - 37
    T = -(-N // 128)
    bm = split_mask(T, 390 + d, 20)
    B, H, t, seed = 1, 1, 51, 0x5151 + d
    q, k, v, do = draw_qkvdo(B, H, N, d, "bf16", 1.0, 391 + d)
    say(f"dropout split column d={d} N={N}")
    out = run(q, k, v, do, 1 / np.sqrt(d), t, seed, block_mask=bm)
    O, lse = odrop.forward(q, k, v, 1 / np.sqrt(d), t, seed, block_mask=bm)
    keep_frac = 1 - t / 256
    compare_forward(out["o"] * keep_frac, out["lse"], O * keep_frac, lse, "bf16", f"dropout split d{d}")
    g = odrop.backward(q, k, v, do, 1 / np.sqrt(d), t, seed, block_mask=bm)
    for name, a, r in zip(("dq", "dk", "dv"), (out["dq"], out["dk"], out["dv"]), g):
        compare_grad(a, r, "bf16", f"dropout split d{d} {name}")
