"""GPU parity of the split-key forward (fa_fwd_splitkv) against the oracle.

The oracle is the definition for Nq queries against Nk keys with the causal
mask aligned to the last Nq key positions (key j allowed for query i iff
j <= i + Nk - Nq); the library computes it as per-range partial results
merged with the two-block softmax rule, so the comparison also checks the
merge.  Cases cover decoding (one query), chunked prefill, ragged key
counts, kv_len padding (including batches with no keys), more queries than
keys under the causal mask, Nk = 0, explicit and clamped range counts, and
the two benchmark shapes at full size on sampled rows."""
import numpy as np
import pytest

from oracle import attention
from workloads import SPLITKV_WORKLOADS, draw_kv_len, draw_split_qkv

from gpu_cases import compare_forward, host, say, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import exact_io_aware_flashattention_amd as fa
    fa.load_library()


def draw(B, H, Nq, Nk, d, seed):
    return draw_split_qkv(B, H, Nq, Nk, d, 1.0, seed)


def run(q, k, v, scale, causal=False, kv_len=None, num_splits=0):
    import torch

    import exact_io_aware_flashattention_amd as fa
    tq, tk, tv = (to_dev(x, "bf16") for x in (q, k, v))
    kl = None if kv_len is None else torch.from_numpy(np.asarray(kv_len, np.int32)).cuda()
    o, lse = fa.fa_fwd_splitkv(tq, tk, tv, scale=scale, causal=causal, kv_len=kl, num_splits=num_splits)
    torch.cuda.synchronize()
    return host(o), lse.cpu().numpy().astype(np.float64)


def oracle(q, k, v, scale, causal=False, kv_len=None, rows=None, heads=None):
    B, H, Nq, d = q.shape
    Nk = k.shape[2]
    rows = np.arange(Nq) if rows is None else np.asarray(rows)
    heads = [(b, h) for b in range(B) for h in range(H)] if heads is None else heads
    O = np.zeros((len(heads), len(rows), d))
    lse = np.zeros((len(heads), len(rows)))
    for n, (b, h) in enumerate(heads):
        L = None if kv_len is None else int(kv_len[b])
        O[n], lse[n] = attention.head_forward(q[b, h], k[b, h], v[b, h], scale, rows, causal, None, L,
                                              causal_offset=Nk - Nq)
    return O, lse


CASES = [
    # B, H, Nq, Nk, d, causal, kv, num_splits
    (4, 8, 1, 5000, 128, False, False, 0),      # decode, ragged keys, auto ranges
    (3, 4, 1, 4096, 64, True, True, 0),         # decode with padding (one batch may have no key)
    (1, 4, 300, 2000, 64, True, False, 5),      # chunked prefill, ragged query cell
    (2, 2, 128, 1111, 128, True, True, 3),      # prefill + padding
    (1, 2, 200, 150, 128, True, False, 0),      # more queries than keys: first 50 rows empty
    (1, 3, 257, 257, 64, True, False, 2),       # Nq = Nk: fa_fwd's causal mask
    (2, 2, 5, 700, 128, False, False, 64),      # more ranges asked than 128-key cells: clamped
    (1, 2, 64, 3000, 128, False, False, 1),     # one range: no merge needed, still exact
    # at most four queries: the decoding kernel (one wave per key range)
    (2, 3, 2, 3001, 128, True, False, 0),       # two queries, causal: the last sees one key more
    (3, 2, 3, 2500, 64, True, True, 0),         # three queries (padded to four), padding, d = 64
    (1, 4, 4, 777, 128, False, True, 7),        # four queries, ragged last block
    (2, 2, 4, 5, 64, True, False, 0),           # fewer keys than one block
    (1, 2, 1, 20000, 64, False, False, 300),    # many short ranges (one tile each)
    (2, 1, 3, 2, 128, True, False, 0),          # causal with more queries than keys: row 0 empty
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: "B{}H{}q{}k{}d{}{}{}s{}".format(
    c[0], c[1], c[2], c[3], c[4], "c" if c[5] else "", "p" if c[6] else "", c[7]))
def test_splitkv_parity(case):
    B, H, Nq, Nk, d, causal, kv, ns = case
    q, k, v = draw(B, H, Nq, Nk, d, 500 + Nq + Nk)
    kv_len = None
    if kv:
        kv_len = draw_kv_len(B, 0, Nk, 510 + Nk)
        kv_len[0] = 0                       # a batch with no key: O = 0, lse = -inf
    say(f"splitkv parity {case} kv_len={None if kv_len is None else kv_len.tolist()}")
    scale = 1 / np.sqrt(d)
    o, lse = run(q, k, v, scale, causal, kv_len, ns)
    O, L = oracle(q, k, v, scale, causal, kv_len)
    compare_forward(o.reshape(B * H, Nq, d), lse.reshape(B * H, Nq), O, L, "bf16", f"splitkv {case}")


def test_splitkv_matches_plain_forward_when_square():
    """Nq = Nk with one range is the plain forward's computation; with many
    ranges it differs from it only by the order of fp32 additions."""
    import torch

    import exact_io_aware_flashattention_amd as fa
    q, k, v = draw(2, 3, 640, 640, 128, 520)
    tq, tk, tv = (to_dev(x, "bf16") for x in (q, k, v))
    o0, l0 = fa.fa_fwd(tq, tk, tv, causal=True)
    o1, l1 = fa.fa_fwd_splitkv(tq, tk, tv, causal=True, num_splits=5)
    torch.cuda.synchronize()
    assert fa.fa_fwd_splitkv_num_splits(2, 3, 640, 640, 5) == 5
    assert (o0.float() - o1.float()).abs().max().item() <= 2 ** -7
    assert (l0 - l1).abs().max().item() <= 1e-5


def test_splitkv_no_keys():
    import torch

    import exact_io_aware_flashattention_amd as fa
    q, _, _ = draw(2, 2, 3, 1, 64, 530)
    tq = to_dev(q, "bf16")
    empty = torch.empty((2, 2, 0, 64), dtype=torch.bfloat16, device="cuda")
    o, lse = fa.fa_fwd_splitkv(tq, empty, empty)
    torch.cuda.synchronize()
    assert torch.all(o == 0) and torch.all(torch.isneginf(lse))


def test_splitkv_deterministic():
    import torch

    import exact_io_aware_flashattention_amd as fa
    q, k, v = draw(2, 4, 1, 8192, 128, 540)
    tq, tk, tv = (to_dev(x, "bf16") for x in (q, k, v))
    a = fa.fa_fwd_splitkv(tq, tk, tv)
    b = fa.fa_fwd_splitkv(tq, tk, tv)
    torch.cuda.synchronize()
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])


@pytest.mark.parametrize("which", ["decode", "prefill"])
def test_splitkv_full_size_sampled(which):
    """The benchmark shapes (decode: B16 H16 one query against 16384 keys;
    chunked prefill: the last 2048 queries of the 16384-token causal long
    context, B1 H16), d = 128, with the launch configuration the benchmark
    times; every row of decode, sampled rows of prefill."""
    w = SPLITKV_WORKLOADS[which]
    B, H, Nq, Nk, d, causal = w["B"], w["H"], w["Nq"], w["Nk"], w["d"], w["causal"]
    q, k, v = draw_split_qkv(B, H, Nq, Nk, d, w["sigma"], w["seed"])
    say(f"splitkv full size {which}: {w}")
    scale = 1 / np.sqrt(d)
    o, lse = run(q, k, v, scale, causal)
    rng = np.random.Generator(np.random.PCG64(551))
    rows = np.arange(Nq) if Nq <= 8 else np.unique(np.r_[0, Nq - 1, rng.integers(0, Nq, 40)])
    heads = [(b, h) for b in range(B) for h in range(H)]
    if len(heads) > 8:
        heads = [heads[i] for i in np.unique(np.r_[0, len(heads) - 1, rng.integers(0, len(heads), 8)])]
    O, L = oracle(q, k, v, scale, causal, None, rows, heads)
    got_o = np.stack([o[b, h][rows] for b, h in heads])
    got_l = np.stack([lse[b, h][rows] for b, h in heads])
    compare_forward(got_o, got_l, O, L, "bf16", f"splitkv {which}")


# ---------------------------------------------------------------- E4M3 key/value cache

def run_fp8kv(q, k8, v8, dk, dv, scale, causal=False, kv_len=None, num_splits=0):
    import torch

    import exact_io_aware_flashattention_amd as fa
    tq = to_dev(q, "bf16")
    tk, tv = (torch.from_numpy(np.ascontiguousarray(x)).cuda() for x in (k8, v8))
    kl = None if kv_len is None else torch.from_numpy(np.asarray(kv_len, np.int32)).cuda()
    o, lse = fa.fa_fwd_splitkv_fp8kv(tq, tk, tv, float(dk), float(dv), scale=scale, causal=causal, kv_len=kl,
                                     num_splits=num_splits)
    torch.cuda.synchronize()
    return host(o), lse.cpu().numpy().astype(np.float64)


FP8KV_CASES = [
    # B, H, Nq, Nk, d, causal, kv, num_splits
    (4, 8, 1, 5000, 128, False, False, 0),
    (3, 4, 3, 2500, 64, True, True, 0),
    (2, 2, 2, 3001, 256, True, False, 7),
    (1, 2, 4, 5, 128, True, False, 0),
]


@pytest.mark.parametrize("case", FP8KV_CASES, ids=lambda c: "B{}H{}q{}k{}d{}{}{}s{}".format(
    c[0], c[1], c[2], c[3], c[4], "c" if c[5] else "", "p" if c[6] else "", c[7]))
def test_fp8kv_decode_parity(case):
    """Decoding against an E4M3 K/V cache: the oracle is exact attention of the
    bf16 queries against the real values of the codes; every product is exact
    and the probabilities stay fp32, so the bf16 bounds apply."""
    from oracle import fp8 as ofp8
    from workloads import quantize_e4m3
    B, H, Nq, Nk, d, causal, kv, ns = case
    q, k, v = draw(B, H, Nq, Nk, d, 700 + Nq + Nk)
    (k8, dk), (v8, dv) = quantize_e4m3(k), quantize_e4m3(v)
    kv_len = None
    if kv:
        kv_len = draw_kv_len(B, 0, Nk, 710 + Nk)
        kv_len[0] = 0
    say(f"fp8kv decode {case}")
    scale = 1 / np.sqrt(d)
    o, lse = run_fp8kv(q, k8, v8, dk, dv, scale, causal, kv_len, ns)
    K, V = ofp8.dequantize(k8, dk), ofp8.dequantize(v8, dv)
    O, L = oracle(q, K, V, scale, causal, kv_len)
    compare_forward(o.reshape(B * H, Nq, d), lse.reshape(B * H, Nq), O, L, "bf16", f"fp8kv {case}")


def test_fp8kv_decode_full_size_sampled():
    """The decode benchmark shape (B16 H16, one query against 16384 keys) with
    the cache quantized per tensor, as bench.py --splitkv decode --fp8 times
    it, on sampled heads."""
    from oracle import fp8 as ofp8
    from workloads import quantize_e4m3
    w = SPLITKV_WORKLOADS["decode"]
    B, H, Nq, Nk, d = w["B"], w["H"], w["Nq"], w["Nk"], w["d"]
    q, k, v = draw_split_qkv(B, H, Nq, Nk, d, w["sigma"], w["seed"])
    (k8, dk), (v8, dv) = quantize_e4m3(k), quantize_e4m3(v)
    say("fp8kv decode full size")
    o, lse = run_fp8kv(q, k8, v8, dk, dv, 1 / np.sqrt(d))
    rng = np.random.Generator(np.random.PCG64(720))
    heads = [(int(x) // H, int(x) % H) for x in np.unique(np.r_[0, B * H - 1, rng.integers(0, B * H, 8)])]
    K = {bh: ofp8.dequantize(k8[bh], dk) for bh in heads}
    V = {bh: ofp8.dequantize(v8[bh], dv) for bh in heads}
    O = np.stack([attention.head_forward(q[b, h], K[(b, h)], V[(b, h)], 1 / np.sqrt(d))[0] for b, h in heads])
    L = np.stack([attention.head_forward(q[b, h], K[(b, h)], V[(b, h)], 1 / np.sqrt(d))[1] for b, h in heads])
    compare_forward(np.stack([o[b, h] for b, h in heads]), np.stack([lse[b, h] for b, h in heads]), O, L, "bf16",
                    "fp8kv decode full")
