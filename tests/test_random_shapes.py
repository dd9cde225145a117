"""GPU parity on seeded random shapes: forward and backward of the attention
kernels (plain and with dropout), the split-key forward and the FP8 forward,
against the fp64 oracles.

The hand-picked cases elsewhere pin the edges one at a time; these draw the
whole configuration at once (sizes on and off the 32/64/128 tile edges, every
head dimension, causal or not, key padding, block masks, fp32 and bf16, and
for the split-key forward Nq <= Nk and a range count), so that combinations
nobody wrote down -- a walk that passes from interior to edge steps at an odd
tile, a split range that starts inside a causal diagonal -- are covered too.
The draw is fixed (PCG64 seed), so every run checks the same cases."""
import numpy as np
import pytest

from oracle import attention
from workloads import draw_kv_len, draw_split_qkv

from gpu_cases import compare_forward, host, say, to_dev
from test_dropout import test_dropout_parity as dropout_parity
from test_fp8 import test_fp8_parity_within_e4m3_bound as fp8_parity
from test_parity import check_full, small_inputs

pytestmark = pytest.mark.gpu

SPECIAL_N = [1, 2, 31, 32, 33, 63, 64, 65, 96, 127, 128, 129, 191, 255, 256, 257, 383, 511, 513, 640, 767, 1023]


def draw_cases(n, seed):
    rng = np.random.Generator(np.random.PCG64(seed))
    cases = []
    for i in range(n):
        d = int(rng.choice([64, 64, 96, 128, 128, 160, 256]))
        N = int(rng.choice(SPECIAL_N)) if rng.random() < 0.5 else int(rng.integers(1, 1200))
        heads = 4 if N <= 600 else 2
        B = int(rng.integers(1, 3))
        H = max(1, min(3, heads // B))
        causal = bool(rng.random() < 0.5)
        kv = "rand" if rng.random() < 0.35 else None
        u = rng.random()
        mask = "bern" if u < 0.15 else ("band" if u < 0.3 else None)
        dtype = "f32" if (rng.random() < 0.1 and d <= 128) else "bf16"
        cases.append((B, H, N, d, dtype, causal, kv, mask, 7000 + i))
    return cases


CASES = draw_cases(32, 20261203)


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import exact_io_aware_flashattention_amd as fa
    fa.load_library()


@pytest.mark.parametrize("case", CASES, ids=lambda c: "B{}H{}N{}d{}{}{}{}{}".format(
    c[0], c[1], c[2], c[3], c[4], "c" if c[5] else "", "k" if c[6] else "", c[7] or ""))
def test_random_shape(case):
    B, H, N, d, dt, causal, kv, mask, seed = case
    check_full(small_inputs(B, H, N, d, dt, causal, kv, mask, seed=seed), f"random {case}")


def draw_split_cases(n, seed):
    rng = np.random.Generator(np.random.PCG64(seed))
    cases = []
    for i in range(n):
        d = int(rng.choice([64, 96, 128, 160, 256]))
        Nk = int(rng.choice(SPECIAL_N[4:])) if rng.random() < 0.5 else int(rng.integers(2, 3000))
        Nq = int(rng.choice([1, 2, 3, 4, 5, 64, 127, 128, 200, 257])) if rng.random() < 0.6 else int(rng.integers(1, 600))
        Nq = min(Nq, Nk)
        causal = bool(rng.random() < 0.6)
        kv = bool(rng.random() < 0.3)
        ns = int(rng.choice([0, 0, 1, 2, 3, 5]))
        cases.append((int(rng.integers(1, 3)), 2, Nq, Nk, d, causal, kv, ns, 8000 + i))
    return cases


SPLIT_CASES = draw_split_cases(20, 20261204)


@pytest.mark.parametrize("case", SPLIT_CASES, ids=lambda c: "B{}H{}q{}k{}d{}{}{}s{}".format(
    c[0], c[1], c[2], c[3], c[4], "c" if c[5] else "", "p" if c[6] else "", c[7]))
def test_random_split_key(case):
    import torch

    import exact_io_aware_flashattention_amd as fa
    B, H, Nq, Nk, d, causal, kv, ns, seed = case
    say(f"random split-key {case}")
    q, k, v = draw_split_qkv(B, H, Nq, Nk, d, 1.0, seed)
    kv_len = draw_kv_len(B, 0, Nk, seed + 1) if kv else None
    scale = 1 / np.sqrt(d)
    tq, tk, tv = (to_dev(x, "bf16") for x in (q, k, v))
    kl = None if kv_len is None else torch.from_numpy(np.asarray(kv_len, np.int32)).cuda()
    o, lse = fa.fa_fwd_splitkv(tq, tk, tv, scale=scale, causal=causal, kv_len=kl, num_splits=ns)
    torch.cuda.synchronize()
    O = np.zeros((B * H, Nq, d))
    L = np.zeros((B * H, Nq))
    for b in range(B):
        for h in range(H):
            n = b * H + h
            O[n], L[n] = attention.head_forward(q[b, h], k[b, h], v[b, h], scale, np.arange(Nq), causal, None,
                                                None if kv_len is None else int(kv_len[b]),
                                                causal_offset=Nk - Nq)
    compare_forward(host(o).reshape(B * H, Nq, d), lse.cpu().numpy().astype(np.float64).reshape(B * H, Nq),
                    O, L, "bf16", f"random split-key {case}")


def draw_dropout_cases(n, seed):
    rng = np.random.Generator(np.random.PCG64(seed))
    cases = []
    for _ in range(n):
        d = int(rng.choice([64, 96, 128, 160, 256]))
        N = int(rng.choice(SPECIAL_N[:-2])) if rng.random() < 0.5 else int(rng.integers(1, 600))
        u = rng.random()
        cases.append((int(rng.integers(1, 3)), int(rng.integers(1, 3)), N, d, bool(rng.random() < 0.5),
                      "rand" if rng.random() < 0.3 else None, "band" if u < 0.25 else None,
                      int(rng.integers(1, 256))))
    return cases


DROPOUT_CASES = draw_dropout_cases(12, 20261205)


@pytest.mark.parametrize("case", DROPOUT_CASES, ids=lambda c: "B{}H{}N{}d{}{}{}{}t{}".format(
    c[0], c[1], c[2], c[3], "c" if c[4] else "", "k" if c[5] else "", "m" if c[6] else "", c[7]))
def test_random_dropout(case):
    dropout_parity(case)


def draw_fp8_cases(n, seed):
    rng = np.random.Generator(np.random.PCG64(seed))
    cases = []
    for _ in range(n):
        N = int(rng.choice(SPECIAL_N)) if rng.random() < 0.5 else int(rng.integers(1, 1200))
        cases.append((int(rng.integers(1, 3)), int(rng.integers(1, 3)), N, int(rng.choice([64, 128])),
                      bool(rng.random() < 0.5), "rand" if rng.random() < 0.3 else None,
                      "band" if rng.random() < 0.25 else None))
    return cases


FP8_CASES = draw_fp8_cases(10, 20261206)


@pytest.mark.parametrize("case", FP8_CASES, ids=lambda c: "B{}H{}N{}d{}{}{}{}".format(
    c[0], c[1], c[2], c[3], "c" if c[4] else "", "k" if c[5] else "", "m" if c[6] else ""))
def test_random_fp8(case):
    fp8_parity(case)
