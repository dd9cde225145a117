"""Guard bands around every output: no store lands outside its tensor.

Each output (O, lse, dQ, dK, dV, delta, the split-key O and lse, the FP8
forward's O and lse) and the caller-provided workspace is placed inside a larger buffer
whose bytes on both sides hold a sentinel pattern.  After the call the
sentinels must be unchanged, and the in-bounds results must equal those of
the same call on ordinary tensors bit for bit (the kernels are
deterministic).  Element-wise parity looks only at in-bounds elements, so an
out-of-bounds store from a ragged tail tile (N % 128 != 0, padded head
dimensions 96 and 160, split-key partial rows) would go unnoticed without
these bands.
"""
import numpy as np
import pytest

from workloads import draw_qkvdo, draw_split_qkv

from gpu_cases import say

pytestmark = pytest.mark.gpu

GUARD_BYTES = 256 << 10          # more than one 128-row tile of the widest head (128 x 256 x 2 bytes x 4)
SENTINEL = 0xA5


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import exact_io_aware_flashattention_amd as fa
    fa.load_library()


class Guarded:
    """A tensor of `shape` and `dtype` at offset GUARD_BYTES inside a byte buffer
    filled with SENTINEL."""

    def __init__(self, shape, dtype):
        import torch
        self.nbytes = int(np.prod(shape)) * torch.empty((), dtype=dtype).element_size()
        self.buf = torch.full((GUARD_BYTES * 2 + self.nbytes,), SENTINEL, dtype=torch.uint8, device="cuda")
        self.t = self.buf[GUARD_BYTES:GUARD_BYTES + self.nbytes].view(dtype).view(shape)
        assert self.t.data_ptr() % 256 == 0

    def check(self, what):
        import torch
        torch.cuda.synchronize()
        lo = self.buf[:GUARD_BYTES].cpu().numpy()
        hi = self.buf[GUARD_BYTES + self.nbytes:].cpu().numpy()
        bad_lo, bad_hi = np.flatnonzero(lo != SENTINEL), np.flatnonzero(hi != SENTINEL)
        assert bad_lo.size == 0, f"{what}: {bad_lo.size} bytes written before the tensor (first at -{GUARD_BYTES - bad_lo[0]})"
        assert bad_hi.size == 0, f"{what}: {bad_hi.size} bytes written past the end (first at +{bad_hi[0]})"


def dev(x, dtype):
    import torch
    return torch.from_numpy(np.ascontiguousarray(x)).to("cuda", dtype)


def same(a, b):
    import torch
    return bool(torch.equal(a.view(torch.uint8) if a.dtype != torch.uint8 else a,
                            b.view(torch.uint8) if b.dtype != torch.uint8 else b))


SQUARE = [(N, d) for N in (1, 63, 65, 129, 1000) for d in (64, 96, 128, 160, 256)]


@pytest.mark.parametrize("N,d", SQUARE, ids=[f"N{n}d{d}" for n, d in SQUARE])
def test_square_forward_backward_stay_in_bounds(N, d):
    import torch

    import exact_io_aware_flashattention_amd as fa
    B, H = 2, 2
    say(f"guard fa_fwd/fa_bwd B={B} H={H} N={N} d={d} bf16 causal, kv_len=[N, N//2+1]")
    q, k, v, do = (dev(x, torch.bfloat16) for x in draw_qkvdo(B, H, N, d, "bf16", 1.0, N + d))
    kl = torch.tensor([N, N // 2 + 1], dtype=torch.int32, device="cuda")
    kw = dict(scale=d ** -0.5, causal=True, kv_len=kl)
    o, lse = Guarded(q.shape, torch.bfloat16), Guarded((B, H, N), torch.float32)
    fa.fa_fwd(q, k, v, o.t, lse.t, **kw)
    o.check("O")
    lse.check("lse")
    o_ref, lse_ref = fa.fa_fwd(q, k, v, **kw)
    assert same(o.t, o_ref) and same(lse.t, lse_ref)

    grads = [Guarded(q.shape, torch.bfloat16) for _ in range(3)]
    need = max(fa.fa_bwd_workspace_bytes(B, H, N, d, fa.FA_BF16, False), 256)
    ws = Guarded((need,), torch.uint8)
    fa.fa_bwd(q, k, v, o_ref, do, lse_ref, *(g.t for g in grads), workspace=ws.t, **kw)
    for g, name in zip(grads, ("dQ", "dK", "dV")):
        g.check(name)
    ws.check("workspace")
    ref = fa.fa_bwd(q, k, v, o_ref, do, lse_ref, **kw)
    for g, r in zip(grads, ref):
        assert same(g.t, r)

    # the dQ stage that also writes delta: both outputs in guard bands; its dQ
    # is fa_bwd's (the same kernel on the same inputs)
    gdq, gdelta = Guarded(q.shape, torch.bfloat16), Guarded((B, H, N), torch.float32)
    fa.fa_bwd_dq_delta(q, k, v, o_ref, do, lse_ref, gdelta.t, gdq.t, **kw)
    gdq.check("dQ (dq_delta)")
    gdelta.check("delta (dq_delta)")
    assert same(gdq.t, ref[0])


@pytest.mark.parametrize("d", (64, 128, 256))
def test_block_mask_backward_stays_in_bounds(d):
    """A block mask with a long column: the dK/dV split stages write partial sums
    into the workspace, which must stay within the size the library asked for."""
    import torch

    import exact_io_aware_flashattention_amd as fa
    B, H, N = 1, 2, 1100
    T = -(-N // 128)
    say(f"guard fa_bwd block mask B={B} H={H} N={N} d={d}")
    q, k, v, do = (dev(x, torch.bfloat16) for x in draw_qkvdo(B, H, N, d, "bf16", 1.0, 77))
    bm = np.eye(T, dtype=np.uint8)
    bm[:, 0] = 1
    kw = dict(scale=d ** -0.5, causal=False, block_mask=torch.from_numpy(bm).cuda())
    o, lse = fa.fa_fwd(q, k, v, **kw)
    grads = [Guarded(q.shape, torch.bfloat16) for _ in range(3)]
    ws = Guarded((fa.fa_bwd_workspace_bytes(B, H, N, d, fa.FA_BF16, True),), torch.uint8)
    fa.fa_bwd(q, k, v, o, do, lse, *(g.t for g in grads), workspace=ws.t, **kw)
    for g, name in zip(grads, ("dQ", "dK", "dV")):
        g.check(name)
    ws.check("workspace")
    ref = fa.fa_bwd(q, k, v, o, do, lse, **kw)
    for g, r in zip(grads, ref):
        assert same(g.t, r)


def test_fp32_and_dropout_stay_in_bounds():
    import torch

    import exact_io_aware_flashattention_amd as fa
    for N, d in ((65, 64), (129, 128)):
        say(f"guard fp32 N={N} d={d}")
        q, k, v, do = (dev(x, torch.float32) for x in draw_qkvdo(1, 2, N, d, "f32", 1.0, N))
        o, lse = Guarded(q.shape, torch.float32), Guarded((1, 2, N), torch.float32)
        fa.fa_fwd(q, k, v, o.t, lse.t, causal=True)
        o.check("O fp32")
        lse.check("lse fp32")
        grads = [Guarded(q.shape, torch.float32) for _ in range(3)]
        fa.fa_bwd(q, k, v, o.t, do, lse.t, *(g.t for g in grads), causal=True)
        for g, name in zip(grads, ("dQ", "dK", "dV")):
            g.check(name + " fp32")
    for N, d in ((63, 64), (1000, 128), (129, 256)):
        say(f"guard dropout N={N} d={d}")
        q, k, v, do = (dev(x, torch.bfloat16) for x in draw_qkvdo(1, 2, N, d, "bf16", 1.0, N))
        kw = dict(causal=True, dropout_p=0.1, seed=5)
        o, lse = Guarded(q.shape, torch.bfloat16), Guarded((1, 2, N), torch.float32)
        fa.fa_fwd(q, k, v, o.t, lse.t, **kw)
        o.check("O dropout")
        lse.check("lse dropout")
        grads = [Guarded(q.shape, torch.bfloat16) for _ in range(3)]
        fa.fa_bwd(q, k, v, o.t, do, lse.t, *(g.t for g in grads), **kw)
        for g, name in zip(grads, ("dQ", "dK", "dV")):
            g.check(name + " dropout")


SPLIT = [(nq, nk, d) for nq, nk in ((1, 1), (3, 65), (4, 1000), (37, 1000), (129, 300)) for d in (64, 96, 160, 256)]


@pytest.mark.parametrize("Nq,Nk,d", SPLIT, ids=[f"q{a}k{b}d{c}" for a, b, c in SPLIT])
def test_split_key_forward_stays_in_bounds(Nq, Nk, d):
    import torch

    import exact_io_aware_flashattention_amd as fa
    B, H = 2, 3
    say(f"guard fa_fwd_splitkv B={B} H={H} Nq={Nq} Nk={Nk} d={d}")
    qa, ka, va = draw_split_qkv(B, H, Nq, Nk, d, 1.0, Nq + Nk + d)
    q, k, v = (dev(x, torch.bfloat16) for x in (qa, ka, va))
    kl = torch.tensor([Nk, max(Nk // 3, 1)], dtype=torch.int32, device="cuda")
    for splits in (0, 3):
        kw = dict(scale=d ** -0.5, causal=True, kv_len=kl, num_splits=splits)
        o, lse = Guarded(q.shape, torch.bfloat16), Guarded((B, H, Nq), torch.float32)
        ws = Guarded((fa.fa_fwd_splitkv_workspace_bytes(B, H, Nq, Nk, d, splits),), torch.uint8)
        fa.fa_fwd_splitkv(q, k, v, o.t, lse.t, workspace=ws.t, **kw)
        o.check(f"split O ({splits} ranges)")
        lse.check(f"split lse ({splits} ranges)")
        ws.check(f"split workspace ({splits} ranges)")
        o_ref, lse_ref = fa.fa_fwd_splitkv(q, k, v, **kw)
        assert same(o.t, o_ref) and same(lse.t, lse_ref)


@pytest.mark.parametrize("N,d", [(1, 64), (65, 128), (1000, 64), (129, 128)])
def test_fp8_forward_stays_in_bounds(N, d):
    import torch

    import exact_io_aware_flashattention_amd as fa
    from workloads import quantize_e4m3
    B, H = 1, 2
    say(f"guard fa_fwd_fp8 B={B} H={H} N={N} d={d}")
    q, k, v, _ = draw_qkvdo(B, H, N, d, "bf16", 1.0, 9 + N)
    (q8, dq), (k8, dk), (v8, dv) = (quantize_e4m3(x) for x in (q, k, v))
    t8 = [torch.from_numpy(x).cuda() for x in (q8, k8, v8)]
    o, lse = Guarded((B, H, N, d), torch.bfloat16), Guarded((B, H, N), torch.float32)
    fa.fa_fwd_fp8(*t8, float(dq), float(dk), float(dv), o.t, lse.t, causal=True)
    o.check("fp8 O")
    lse.check("fp8 lse")
