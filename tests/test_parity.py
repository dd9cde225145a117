"""GPU parity: the HIP path (through the C ABI) against the CPU fp64 oracle on the
same seeded inputs.  Small shapes are compared element by element against the
full dense oracle; the five workloads at full size are compared on sampled
heads, rows and key columns with the gathered (sparse) form of the oracle."""
import numpy as np
import pytest

from oracle import attention, sparse
from workloads import WORKLOADS, band_random_mask, draw_kv_len, draw_qkvdo, make_inputs

from gpu_cases import compare_forward, compare_grad, run_gpu, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import exact_io_aware_flashattention_amd as fa
    fa.load_library()


def small_inputs(B, H, N, d, dtype, causal, kv=None, mask=None, seed=0, sigma=1.0, scale=None):
    q, k, v, do = draw_qkvdo(B, H, N, d, dtype, sigma, seed)
    T = -(-N // 128)
    kv_len = None
    if isinstance(kv, str):
        kv_len = draw_kv_len(B, 1, N, 1000 + seed)
    elif kv is not None:
        kv_len = np.asarray(kv, np.int32)
    bm = None
    if isinstance(mask, str) and mask == "band":
        bm = band_random_mask(T, 2000 + seed, n_random=1)
    elif isinstance(mask, str) and mask == "bern":
        rng = np.random.Generator(np.random.PCG64(3000 + seed))
        bm = (rng.random((T, T)) < 0.5).astype(np.uint8)
        bm[:, 0] = 1
    elif mask is not None:
        bm = np.asarray(mask, np.uint8)
    return dict(q=q, k=k, v=v, do=do, kv_len=kv_len, block_mask=bm, B=B, H=H, N=N, d=d, dtype=dtype,
                causal=causal, scale=(1.0 / np.sqrt(d)) if scale is None else scale)


def check_full(inp, what, backward=True):
    say(f"case {what}: B={inp['B']} H={inp['H']} N={inp['N']} d={inp['d']} {inp['dtype']} "
        f"causal={inp['causal']} kv={inp['kv_len'] is not None} mask={inp['block_mask'] is not None}")
    out = run_gpu(inp, backward)
    kw = dict(causal=inp["causal"], block_mask=inp["block_mask"], kv_len=inp["kv_len"])
    O, lse = attention.forward(inp["q"], inp["k"], inp["v"], inp["scale"], **kw)
    compare_forward(out["o"], out["lse"], O, lse, inp["dtype"], what)
    if backward:
        g = attention.backward(inp["q"], inp["k"], inp["v"], inp["do"], inp["scale"], **kw)
        zs = float(np.abs(inp["do"]).max() * np.abs(inp["v"]).max() * inp["scale"]
                   * max(np.abs(inp["k"]).max(), np.abs(inp["q"]).max(), 1.0))
        for name, a, r in zip(("dq", "dk", "dv"), (out["dq"], out["dk"], out["dv"]), g):
            compare_grad(a, r, inp["dtype"], f"{what} {name}", zero_scale=zs)
    return out


SMALL = [
    # B, H, N, d, dtype, causal, kv, mask
    (1, 1, 1, 64, "bf16", False, None, None),
    (1, 1, 1, 128, "f32", True, None, None),
    (1, 2, 63, 64, "bf16", True, None, None),
    (2, 1, 64, 128, "bf16", False, None, None),
    (1, 2, 65, 64, "f32", False, None, None),
    (1, 2, 127, 128, "bf16", True, None, None),
    (2, 2, 129, 64, "bf16", True, "rand", None),
    (1, 3, 200, 128, "bf16", False, "rand", None),
    (2, 2, 256, 64, "bf16", True, None, "bern"),
    (1, 2, 300, 128, "f32", True, "rand", "band"),
    (3, 2, 333, 64, "bf16", False, "rand", "bern"),
    (1, 2, 513, 128, "bf16", True, None, "band"),
    (1, 1, 1000, 64, "f32", True, None, None),
    (2, 1, 1000, 128, "bf16", False, "rand", None),
    (1, 1, 640, 64, "bf16", False, None, "band"),
]


@pytest.mark.parametrize("case", SMALL, ids=lambda c: "B{}H{}N{}d{}{}{}{}{}".format(
    c[0], c[1], c[2], c[3], c[4], "c" if c[5] else "", "k" if c[6] else "", "m" if c[7] else ""))
def test_small_shapes(case):
    B, H, N, d, dt, causal, kv, mask = case
    check_full(small_inputs(B, H, N, d, dt, causal, kv, mask, seed=N + d + B), str(case))


def test_tiny_exact_config_fp32():
    """Workload 1 at its own size: fp32, B=1 H=2 N=128 d=64, no mask."""
    check_full(make_inputs(WORKLOADS[1]), "workload-1")


def test_fully_masked_rows():
    """kv_len = 0 (no key at all), kv_len > N (clamped), and a mask row of zeros."""
    inp = small_inputs(3, 2, 256, 64, "bf16", False, kv=[0, 5000, 129], seed=5)
    out = check_full(inp, "kv0")
    assert np.all(out["o"][0] == 0) and np.all(out["lse"][0] == -np.inf)
    assert np.all(out["dq"][0] == 0) and np.all(out["dk"][0] == 0) and np.all(out["dv"][0] == 0)
    bm = np.ones((2, 2), np.uint8)
    bm[1, :] = 0
    inp = small_inputs(1, 2, 256, 128, "bf16", True, mask=bm, seed=6)
    out = check_full(inp, "mask-empty-row")
    assert np.all(out["lse"][:, :, 128:] == -np.inf)


def test_large_scores_stay_finite():
    """Scores of magnitude ~1e3 (sigma 6, d 64, scale 1), where exp without the
    running max would overflow.  The fp32 scores themselves carry rounding of
    about d * 2^-24 * sum_t |q_t k_t| (up to ~1e-2 here), which moves each
    probability by that relative amount, so O is held to that derived bound
    (2 * max score error * max|V|) instead of the 1e-5 of unit-scale inputs."""
    inp = small_inputs(1, 2, 384, 64, "f32", True, seed=8, sigma=6.0, scale=1.0)
    out = run_gpu(inp, backward=False)
    O, lse = attention.forward(inp["q"], inp["k"], inp["v"], 1.0, causal=True)
    q, k = np.abs(inp["q"]).astype(np.float64), np.abs(inp["k"]).astype(np.float64)
    s_err = 64 * 2.0 ** -24 * np.einsum("bhid,bhjd->bhij", q, k).max()
    bound = 2 * s_err * np.abs(inp["v"]).max()
    assert np.all(np.isfinite(out["o"])) and np.all(np.isfinite(out["lse"]))
    err = np.abs(out["o"] - O).max()
    say(f"  large-scores: max|dO| {err:.3e}, derived bound {bound:.3e}, max|lse| {np.abs(lse).max():.1f}")
    assert err <= bound
    assert np.abs(out["lse"] - lse).max() <= s_err


def test_deterministic_repeat():
    inp = small_inputs(1, 4, 700, 128, "bf16", True, "rand", "bern", seed=9)
    a = run_gpu(inp)
    b = run_gpu(inp)
    for n in ("o", "lse", "dq", "dk", "dv"):
        assert np.array_equal(a[n], b[n]), n


def split_mask(T, seed, heavy_col):
    """Band + one random cell per row + a global column 0 (band_random_mask)
    plus one more fully set column: two key columns that every query cell
    visits."""
    bm = band_random_mask(T, seed, n_random=1)
    bm[:, heavy_col] = 1
    return bm


SPLIT_CASES = [
    # B, H, N, d, causal, kv_len
    (2, 2, 5083, 64, False, None),
    (1, 2, 5083, 128, True, None),
    (2, 1, 5083, 64, True, [5083, 1000]),   # b = 1: the set column 20 lies past kv_len
]


@pytest.mark.parametrize("case", SPLIT_CASES, ids=lambda c: "B{}H{}N{}d{}{}{}".format(
    c[0], c[1], c[2], c[3], "c" if c[4] else "", "k" if c[5] else ""))
def test_split_key_columns(case):
    """Block-sparse dK/dV with key columns long enough to be split over several
    work-groups (a column is split when it holds more visited cells than the
    chunk, max(16, ceil(visited cells of all heads / 512)) = 16 here, and the
    set columns hold 20-40).  Element-wise against the dense oracle, and the
    order-fixed reduction of the partial sums makes a repeat bit-identical."""
    B, H, N, d, causal, kv = case
    T = -(-N // 128)
    bm = split_mask(T, 2100 + d, 20)
    per_head = bm[np.arange(T)[:, None] >= np.arange(T)[None, :]].sum() if causal else bm.sum()
    chunk = max(16, -(-int(B * H * per_head) // 512))
    assert chunk == 16 and (bm[:, 0].sum() > chunk)
    inp = small_inputs(B, H, N, d, "bf16", causal, kv=kv, mask=bm, seed=N + d)
    out = check_full(inp, f"split {case}")
    again = run_gpu(inp)
    for n in ("dk", "dv"):
        assert np.array_equal(out[n], again[n]), n
    if kv is not None:
        assert np.all(out["dk"][1, :, kv[1]:] == 0) and np.all(out["dv"][1, :, kv[1]:] == 0)


def test_maximum_mask_size():
    """The largest block mask the library accepts: T = 2048 cells per side
    (N = 262144), causal band mask with a global first column (split in
    dK/dV).  Sampled rows of O, lse, dQ and sampled key columns of dK, dV
    (including the global column) against the gathered oracle."""
    N, d = 2048 * 128, 64
    bm = band_random_mask(2048, 2200, n_random=1)
    q, k, v, do = draw_qkvdo(1, 1, N, d, "bf16", 1.0, 2201)
    inp = dict(q=q, k=k, v=v, do=do, kv_len=None, block_mask=bm, B=1, H=1, N=N, d=d, dtype="bf16",
               causal=True, scale=0.125)
    say(f"maximum mask size: N={N} T=2048 cells={int(bm.sum())}")
    out = run_gpu(inp)
    for n in ("o", "dq", "dk", "dv"):
        assert np.all(np.isfinite(out[n])), n
    rng = np.random.Generator(np.random.PCG64(2202))
    rows = np.unique(np.concatenate([[0, 1, 127, 128, N // 2, N - 129, N - 1], rng.integers(0, N, 25)]))
    cols = np.unique(np.concatenate([[0, 1, 127, 128, N - 1], rng.integers(0, N, 11)]))
    Q, K, V, dO = q[0, 0], k[0, 0], v[0, 0], do[0, 0]
    kw = dict(causal=True, block_mask=bm, kv_len=None)
    O, lse = sparse.head_forward_rows(Q, K, V, 0.125, rows, **kw)
    compare_forward(out["o"][0, 0][rows], out["lse"][0, 0][rows], O, lse, "bf16", "max-size rows")
    compare_grad(out["dq"][0, 0][rows], sparse.head_backward_rows(Q, K, V, dO, 0.125, rows, **kw), "bf16",
                 "max-size dq rows")
    _, dK, dV = sparse.head_backward(Q, K, V, dO, 0.125, key_cols=cols, **kw)
    compare_grad(out["dk"][0, 0][cols], dK, "bf16", "max-size dk cols")
    compare_grad(out["dv"][0, 0][cols], dV, "bf16", "max-size dv cols")


def test_empty_problem_is_a_no_op():
    import torch

    import exact_io_aware_flashattention_amd as fa
    q = torch.zeros((0, 2, 16, 64), dtype=torch.bfloat16, device="cuda")
    o, lse = fa.fa_fwd(q, q, q)
    assert o.shape == q.shape and lse.shape == (0, 2, 16)


# ---------------------------------------------------------------- full-size workloads

def _sample_heads(B, H, n, seed):
    rng = np.random.Generator(np.random.PCG64(seed))
    pairs = {(0, 0), (B - 1, H - 1)}
    while len(pairs) < min(n, B * H):
        pairs.add((int(rng.integers(B)), int(rng.integers(H))))
    return sorted(pairs)


def _check_heads_dense(inp, out, pairs, what):
    for (b, h) in pairs:
        L = None if inp["kv_len"] is None else int(inp["kv_len"][b])
        args = (inp["q"][b, h], inp["k"][b, h], inp["v"][b, h])
        O, lse = attention.head_forward(*args, inp["scale"], causal=inp["causal"], kv_len=L,
                                        block_mask=inp["block_mask"])
        compare_forward(out["o"][b, h], out["lse"][b, h], O, lse, inp["dtype"], f"{what} b{b}h{h}")
        g = attention.head_backward(*args, inp["do"][b, h], inp["scale"], inp["causal"], inp["block_mask"], L)
        for name, a, r in zip(("dq", "dk", "dv"), (out["dq"], out["dk"], out["dv"]), g):
            compare_grad(a[b, h], r, inp["dtype"], f"{what} b{b}h{h} {name}")


@pytest.mark.parametrize("key", [2, 3])
def test_workload_full_size_sampled_heads(key):
    inp = make_inputs(WORKLOADS[key])
    say(f"workload {key} ({WORKLOADS[key].name}) full size")
    out = run_gpu(inp)
    for n in ("o", "dq", "dk", "dv"):
        assert np.all(np.isfinite(out[n])), n
    _check_heads_dense(inp, out, _sample_heads(inp["B"], inp["H"], 6, key), f"w{key}")


@pytest.mark.parametrize("shape", [(2048, 128, False), (4096, 64, True)], ids=["N2048d128", "N4096d64c"])
def test_sweep_shapes_sampled_heads(shape):
    """Shapes of the N = 1K..16K sweep timed by bench.py --sweep (B = 16K / N,
    H = 16, the same seeded draw reshaped), on sampled heads against the dense
    oracle."""
    N, d, causal = shape
    B = 16384 // N
    flat = draw_qkvdo(1, 16, 16384, d, "bf16", 1.0, 6)
    q, k, v, do = (a.reshape(B, 16, N, d) for a in flat)
    inp = dict(q=q, k=k, v=v, do=do, kv_len=None, block_mask=None, B=B, H=16, N=N, d=d, dtype="bf16",
               causal=causal, scale=1.0 / np.sqrt(d))
    say(f"sweep shape B={B} H=16 N={N} d={d} causal={causal}")
    out = run_gpu(inp)
    _check_heads_dense(inp, out, _sample_heads(B, 16, 3, N + d), f"sweep N{N}d{d}")


@pytest.mark.parametrize("key", [4, 5, 6, 7, 8])
def test_workload_long_sequence_sampled(key):
    """N = 16K causal (d = 96, 128, 160 and 256) and N = 64K block-sparse: sampled rows of
    O, lse and dQ and sampled key columns of dK, dV on two heads, against the
    gathered oracle."""
    inp = make_inputs(WORKLOADS[key])
    say(f"workload {key} ({WORKLOADS[key].name}) full size")
    out = run_gpu(inp)
    for n in ("o", "dq", "dk", "dv"):
        assert np.all(np.isfinite(out[n])), n
    N = inp["N"]
    rng = np.random.Generator(np.random.PCG64(77 + key))
    rows = np.unique(np.concatenate([[0, 1, 127, 128, N // 2, N - 129, N - 1], rng.integers(0, N, 57)]))
    cols = np.unique(np.concatenate([[0, 1, 127, 128, N - 1], rng.integers(0, N, 27)]))
    kw = dict(causal=inp["causal"], block_mask=inp["block_mask"], kv_len=None)
    for h in (0, inp["H"] - 1):
        Q, K, V, dO = (inp[n][0, h] for n in ("q", "k", "v", "do"))
        O, lse = sparse.head_forward_rows(Q, K, V, inp["scale"], rows, **kw)
        compare_forward(out["o"][0, h][rows], out["lse"][0, h][rows], O, lse, "bf16", f"w{key} h{h} rows")
        dQ = sparse.head_backward_rows(Q, K, V, dO, inp["scale"], rows, **kw)
        # normalised by the largest oracle value among the sampled entries
        compare_grad(out["dq"][0, h][rows], dQ, "bf16", f"w{key} h{h} dq rows")
        _, dK, dV = sparse.head_backward(Q, K, V, dO, inp["scale"], key_cols=cols, **kw)
        compare_grad(out["dk"][0, h][cols], dK, "bf16", f"w{key} h{h} dk cols")
        compare_grad(out["dv"][0, h][cols], dV, "bf16", f"w{key} h{h} dv cols")
