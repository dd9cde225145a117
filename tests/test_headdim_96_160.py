"""GPU parity at head dimensions 96 and 160 (bf16 only).

These are not powers of two: the kernels stage K, V, Q and dO tiles in LDS
with rows of the next power of two (128, 256), filling the pad chunks with
zeros from past the end of the buffer, and the decoding kernel serves a key
row with a power-of-two group of lanes whose extra lanes read zeros.  d = 96
runs like d = 128 (two waves per SIMD, dK and dV together); d = 160 like
d = 256 (one wave per SIMD).  Cases, against the fp64
oracle: plain, causal, key padding, both mask kinds, ragged N, a split key
column, dropout, the split-key forward (decoding and matrix-core paths) and
decoding against an E4M3 key/value cache."""
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
    (1, 2, 63, True, None, None),
    (1, 2, 300, True, None, None),
    (2, 1, 257, False, "rand", None),
    (1, 2, 513, True, None, "band"),
    (2, 1, 700, False, "rand", "bern"),
    (1, 2, 2048, True, None, None),
]


@pytest.mark.parametrize("d", [96, 160])
@pytest.mark.parametrize("case", CASES, ids=lambda c: "B{}H{}N{}{}{}{}".format(
    c[0], c[1], c[2], "c" if c[3] else "", "k" if c[4] else "", "m" if c[5] else ""))
def test_parity(case, d):
    B, H, N, causal, kv, mask = case
    check_full(small_inputs(B, H, N, d, "bf16", causal, kv, mask, seed=N + d + B), f"d{d} {case}")


@pytest.mark.parametrize("d", [96, 160])
def test_split_key_column(d):
    """A key column visited by 18 query cells (more than the chunk of 16) is
    split over work-groups (for d = 160 in both dK/dV passes).  Element-wise
    against the dense oracle, and bit-identical on a repeat."""
    N = 18 * 128 - 95
    bm = split_mask(18, 2300 + d, 9)
    inp = small_inputs(1, 2, N, d, "bf16", False, mask=bm, seed=2301 + d)
    out = check_full(inp, f"d{d} split column")
    again = run_gpu(inp)
    for n in ("dk", "dv"):
        assert np.array_equal(out[n], again[n]), n


@pytest.mark.parametrize("d", [96, 160])
def test_dropout(d):
    import torch

    import exact_io_aware_flashattention_amd as fa
    B, H, N, t, seed = 1, 2, 333, 51, 0x5EED000 + d
    inp = small_inputs(B, H, N, d, "bf16", True, seed=2400 + d)
    q, k, v, do = inp["q"], inp["k"], inp["v"], inp["do"]
    tq, tk, tv, tdo = (to_dev(x, "bf16") for x in (q, k, v, do))
    scale = 1 / np.sqrt(d)
    kw = dict(scale=scale, causal=True, dropout_p=t / 256, seed=seed)
    say(f"d{d} dropout N={N} t={t}")
    o, lse = fa.fa_fwd(tq, tk, tv, **kw)
    dq, dk, dv = fa.fa_bwd(tq, tk, tv, o, tdo, lse, **kw)
    torch.cuda.synchronize()
    O, L = odrop.forward(q, k, v, scale, t, seed, causal=True)
    keep = 1 - t / 256
    compare_forward(host(o) * keep, lse.cpu().numpy().astype(np.float64), O * keep, L, "bf16", f"d{d} dropout")
    g = odrop.backward(q, k, v, do, scale, t, seed, causal=True)
    for name, a, r in zip(("dq", "dk", "dv"), (dq, dk, dv), g):
        compare_grad(host(a), r, "bf16", f"d{d} dropout {name}")


@pytest.mark.parametrize("d", [96, 160])
@pytest.mark.parametrize("Nq,causal,ns", [(1, False, 0), (3, True, 5), (4, False, 3), (130, True, 5)])
def test_splitkv(Nq, causal, ns, d):
    import torch

    import exact_io_aware_flashattention_amd as fa
    B, H, Nk = 2, 2, 1500
    q, k, v = draw_split_qkv(B, H, Nq, Nk, d, 1.0, 2500 + Nq + d)
    tq, tk, tv = (to_dev(x, "bf16") for x in (q, k, v))
    scale = 1 / np.sqrt(d)
    say(f"d{d} splitkv Nq={Nq} Nk={Nk} causal={causal} num_splits={ns}")
    o, lse = fa.fa_fwd_splitkv(tq, tk, tv, scale=scale, causal=causal, num_splits=ns)
    torch.cuda.synchronize()
    O = np.zeros((B * H, Nq, d))
    L = np.zeros((B * H, Nq))
    for n, (b, h) in enumerate([(b, h) for b in range(B) for h in range(H)]):
        O[n], L[n] = attention.head_forward(q[b, h], k[b, h], v[b, h], scale, causal=causal,
                                            causal_offset=Nk - Nq)
    compare_forward(host(o).reshape(B * H, Nq, d), lse.cpu().numpy().astype(np.float64).reshape(B * H, Nq), O, L,
                    "bf16", f"d{d} splitkv Nq={Nq}")


@pytest.mark.parametrize("d", [96, 160])
@pytest.mark.parametrize("Nq,causal,kv", [(1, False, False), (4, True, True)])
def test_fp8kv_decode(Nq, causal, kv, d):
    """Decoding against an E4M3 cache: exact attention of the bf16 queries
    against the real values of the codes is the oracle."""
    from oracle import fp8 as ofp8
    from test_splitkv import draw, oracle, run_fp8kv
    from workloads import draw_kv_len, quantize_e4m3
    B, H, Nk = 3, 2, 2001
    q, k, v = draw(B, H, Nq, Nk, d, 760 + Nq + d)
    (k8, dk), (v8, dv) = quantize_e4m3(k), quantize_e4m3(v)
    kv_len = None
    if kv:
        kv_len = draw_kv_len(B, 0, Nk, 770 + d)
        kv_len[0] = 0
    say(f"d{d} fp8kv decode Nq={Nq} causal={causal} kv={kv}")
    scale = 1 / np.sqrt(d)
    o, lse = run_fp8kv(q, k8, v8, dk, dv, scale, causal, kv_len)
    K, V = ofp8.dequantize(k8, dk), ofp8.dequantize(v8, dv)
    O, L = oracle(q, K, V, scale, causal, kv_len)
    compare_forward(o.reshape(B * H, Nq, d), lse.reshape(B * H, Nq), O, L, "bf16", f"d{d} fp8kv Nq={Nq}")
