"""fa_fwd_splitkv_noalloc (fixed per-GPU scratch, no allocation in the call)
against fa_fwd_splitkv (caller's workspace) on the same inputs.

Both run the same kernels with the same range plan, so the outputs must be
identical bit for bit.  Two calls in a row share the scratch, the second with
a smaller input, so stale partial results of the first call would show in the
second.  Both the decoding kernel (Nq <= 4) and the matrix-core path run, and
the results are also checked against the oracle at the bf16 bounds.
"""
import numpy as np
import pytest

from oracle import attention
from workloads import draw_split_qkv

from gpu_cases import compare_forward, host, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import exact_io_aware_flashattention_amd as fa
    fa.load_library()


def one_call(B, H, Nq, Nk, d, seed, causal, kv, splits):
    import torch

    import exact_io_aware_flashattention_amd as fa
    say(f"noalloc vs workspace: B={B} H={H} Nq={Nq} Nk={Nk} d={d} causal={causal} kv={kv} splits={splits}")
    qa, ka, va = draw_split_qkv(B, H, Nq, Nk, d, 1.0, seed)
    q, k, v = (torch.from_numpy(x).to("cuda", torch.bfloat16) for x in (qa, ka, va))
    kl = None if kv is None else torch.tensor(kv, dtype=torch.int32, device="cuda")
    kw = dict(scale=d ** -0.5, causal=causal, kv_len=kl, num_splits=splits)
    o_ref, lse_ref = fa.fa_fwd_splitkv(q, k, v, **kw)
    o = torch.full_like(q, float("nan"))
    lse = torch.full((B, H, Nq), float("nan"), dtype=torch.float32, device="cuda")
    fa.fa_fwd_splitkv_noalloc(q, k, v, o, lse, **kw)
    torch.cuda.synchronize()
    assert torch.equal(o.view(torch.int16), o_ref.view(torch.int16))
    assert torch.equal(lse.view(torch.int32), lse_ref.view(torch.int32))
    O, L = np.zeros((B, H, Nq, d)), np.zeros((B, H, Nq))
    for b in range(B):
        for h in range(H):
            O[b, h], L[b, h] = attention.head_forward(qa[b, h], ka[b, h], va[b, h], d ** -0.5, None, causal, None,
                                                      None if kv is None else kv[b], causal_offset=Nk - Nq)
    compare_forward(host(o), lse.cpu().numpy().astype(np.float64), O, L, "bf16", "noalloc")


@pytest.mark.parametrize("first,second", [
    # decoding kernel: (B, H, Nq, Nk, d, seed, causal, kv_len, splits)
    ((4, 8, 1, 5000, 128, 1, True, [5000, 17, 4096, 1], 0), (2, 8, 3, 700, 128, 2, True, [700, 300], 0)),
    # matrix-core path, then a smaller decode-sized call
    ((2, 4, 300, 2000, 64, 3, True, None, 0), (1, 2, 37, 900, 64, 4, False, [500], 3)),
    ((1, 16, 2048, 4096, 128, 5, True, None, 0), (1, 4, 129, 1000, 256, 6, True, None, 0)),
])
def test_noalloc_matches_workspace_path_twice(first, second):
    one_call(*first)
    one_call(*second)


def test_noalloc_rejects_sizes_beyond_the_scratch():
    import torch

    import exact_io_aware_flashattention_amd as fa
    B, H, Nq, Nk, d = 8, 16, 4096, 4096, 128
    assert fa.fa_fwd_splitkv_workspace_bytes(B, H, Nq, Nk, d, 2) > fa.NOALLOC_SCRATCH_BYTES
    q = torch.zeros((B, H, Nq, d), dtype=torch.bfloat16, device="cuda")
    k = torch.zeros((B, H, Nk, d), dtype=torch.bfloat16, device="cuda")
    o = torch.empty_like(q)
    lse = torch.empty((B, H, Nq), dtype=torch.float32, device="cuda")
    with pytest.raises(fa.FAError, match="FA_ERR_SCRATCH"):
        fa.fa_fwd_splitkv_noalloc(q, k, k, o, lse, num_splits=2)
