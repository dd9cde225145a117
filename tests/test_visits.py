"""The tile-skip walk: visited (query cell, key cell) pairs of the forward, dK/dV
and dQ kernels equal H x the expected set, bit for bit."""
import numpy as np
import pytest

from oracle.visits import expected_visits
from workloads import WORKLOADS, band_random_mask, draw_kv_len

from gpu_cases import say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def run_walks(B, H, N, d, causal, bm, kv, dtype=0):
    import torch

    import exact_io_aware_flashattention_amd as fa
    say(f"visits B={B} H={H} N={N} d={d} causal={causal} mask={bm is not None} kv={kv is not None}")
    tb = None if bm is None else torch.from_numpy(bm).cuda()
    tk = None if kv is None else torch.from_numpy(np.asarray(kv, np.int32)).cuda()
    want = H * expected_visits(B, N, causal, bm, kv)
    for which in (fa.WALK_FWD, fa.WALK_DKDV, fa.WALK_DQ):
        got = fa.fa_debug_visits(which, B, H, N, d, causal=causal, block_mask=tb, kv_len=tk, dtype=dtype)
        torch.cuda.synchronize()
        got = got.cpu().numpy().astype(np.int64)
        assert np.array_equal(got, want), f"walk {which}: {np.argwhere(got != want)[:5]}"


CASES = [
    (1, 1, 1, 64, False, None, None),
    (2, 3, 300, 64, True, None, None),
    (2, 2, 1000, 128, False, None, "rand"),
    (1, 2, 1024, 64, True, "band", None),
    (3, 1, 777, 128, True, "bern", "rand"),
    (2, 2, 2048, 64, False, "bern", [0, 2048]),
    # key columns 0 and 20 visited by every query cell: the dK/dV walk splits them
    (2, 2, 5083, 64, False, "split", [5083, 1000]),
    (1, 2, 5083, 128, True, "split", None),
    # the largest mask accepted: 2048 x 2048 cells
    (1, 1, 2048 * 128, 64, True, "band", None),
    # head dimension 256 (dK/dV computes in two passes; the walk is shared)
    (2, 2, 600, 256, True, "bern", "rand"),
    (1, 2, 5083, 256, False, "split", None),
    # head dimensions 96 and 160 (padded LDS rows; 160 computes dK/dV in two passes)
    (2, 2, 600, 96, True, "bern", "rand"),
    (1, 2, 5083, 160, False, "split", None),
]


@pytest.mark.parametrize("case", CASES)
def test_walk_matches_expected(case):
    B, H, N, d, causal, mask, kv = case
    T = -(-N // 128)
    bm = None
    if mask == "band":
        bm = band_random_mask(T, 11)
    elif mask == "bern":
        rng = np.random.Generator(np.random.PCG64(12))
        bm = (rng.random((T, T)) < 0.3).astype(np.uint8)
    elif mask == "split":
        bm = band_random_mask(T, 14, n_random=1)
        bm[:, 20] = 1
    if kv == "rand":
        kv = draw_kv_len(B, 1, N, 13)
    run_walks(B, H, N, d, causal, bm, kv)


@pytest.mark.parametrize("key", [2, 3, 4, 5, 6, 7, 8])
def test_walk_workloads(key):
    w = WORKLOADS[key]
    from workloads import make_inputs
    T = w.cells
    bm = band_random_mask(T, 2000 + key) if w.block_sparse else None
    kv = draw_kv_len(w.B, *w.kv_len_range, 1000 + key) if w.kv_len_range else None
    run_walks(w.B, w.H, w.N, w.d, w.causal, bm, kv)
    if bm is not None:
        say(f"  workload {key}: {int(bm.sum())} of {T * T} cells, s = {bm.sum() / T / T:.5f}")
