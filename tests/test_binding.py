"""The Python binding rejects bad arguments before any library call.

The C ABI receives bare pointers and cannot see allocation sizes, so a tensor
of the wrong shape, dtype or device would become an out-of-bounds device
access.  These tests use CPU tensors only, with the library loader replaced by
one that fails the test, so each check is shown to fire before anything
reaches libfa.so or the GPU.
"""
import pytest

torch = pytest.importorskip("torch")

import exact_io_aware_flashattention_amd as fa  # noqa: E402

B, H, N, D = 2, 3, 200, 64
T = -(-N // 128)


@pytest.fixture(autouse=True)
def no_library(monkeypatch):
    def fail(*a, **k):
        raise AssertionError("the binding called into libfa.so before rejecting its arguments")
    monkeypatch.setattr(fa, "load_library", fail)


def t(*shape, dtype=torch.bfloat16):
    return torch.zeros(shape, dtype=dtype)


def qkv(dtype=torch.bfloat16):
    return t(B, H, N, D, dtype=dtype), t(B, H, N, D, dtype=dtype), t(B, H, N, D, dtype=dtype)


def test_host_tensors_are_rejected():
    q, k, v = qkv()
    with pytest.raises(ValueError, match="GPU tensor"):
        fa.fa_fwd(q, k, v)
    with pytest.raises(ValueError, match="GPU tensor"):
        fa.fa_bwd(q, k, v, t(B, H, N, D), t(B, H, N, D), t(B, H, N, dtype=torch.float32))


@pytest.mark.parametrize("which", ["k", "v"])
def test_forward_operand_shape(which):
    q, k, v = qkv()
    bad = t(B, H, N + 1, D)
    args = dict(k=k, v=v)
    args[which] = bad
    with pytest.raises(ValueError, match=f"{which} must have shape"):
        fa.fa_fwd(q, args["k"], args["v"])


def test_forward_operand_dtype():
    q, k, v = qkv()
    with pytest.raises(TypeError, match="v must be torch.bfloat16"):
        fa.fa_fwd(q, k, v.float())
    with pytest.raises(TypeError, match="unsupported dtype"):
        fa.fa_fwd(q.half(), k.half(), v.half())


def test_forward_outputs():
    q, k, v = qkv()
    with pytest.raises(ValueError, match="o must have shape"):
        fa.fa_fwd(q, k, v, o=t(B, H, N, D // 2))
    with pytest.raises(TypeError, match="lse must be torch.float32"):
        fa.fa_fwd(q, k, v, lse=t(B, H, N))
    with pytest.raises(ValueError, match="lse must have shape"):
        fa.fa_fwd(q, k, v, lse=t(B, H, N - 1, dtype=torch.float32))


def test_masks():
    q, k, v = qkv()
    with pytest.raises(ValueError, match="block_mask must have shape"):
        fa.fa_fwd(q, k, v, block_mask=t(T + 1, T + 1, dtype=torch.uint8))
    with pytest.raises(TypeError, match="block_mask must be torch.uint8"):
        fa.fa_fwd(q, k, v, block_mask=t(T, T, dtype=torch.bool))
    with pytest.raises(TypeError, match="kv_len must be torch.int32"):
        fa.fa_fwd(q, k, v, kv_len=t(B, dtype=torch.int64))
    with pytest.raises(ValueError, match="kv_len must have shape"):
        fa.fa_fwd(q, k, v, kv_len=t(B + 1, dtype=torch.int32))
    with pytest.raises(ValueError, match="block_mask must have shape"):
        fa.fa_fwd_fp8(*(x.to(torch.uint8) for x in qkv()), 1.0, 1.0, 1.0, block_mask=t(1, 1, dtype=torch.uint8))


def test_backward_arguments():
    q, k, v = qkv()
    o, do = t(B, H, N, D), t(B, H, N, D)
    lse = t(B, H, N, dtype=torch.float32)
    with pytest.raises(ValueError, match="dO must have shape"):
        fa.fa_bwd(q, k, v, o, t(B, H, N, D + 32), lse)
    with pytest.raises(TypeError, match="lse must be torch.float32"):
        fa.fa_bwd(q, k, v, o, do, lse.double())
    with pytest.raises(ValueError, match="dq must have shape"):
        fa.fa_bwd(q, k, v, o, do, lse, dq=t(B, H, N - 1, D))
    with pytest.raises(TypeError, match="dk must be torch.bfloat16"):
        fa.fa_bwd(q, k, v, o, do, lse, dk=t(B, H, N, D, dtype=torch.float32))
    with pytest.raises(ValueError, match="workspace must be a 1-D"):
        fa.fa_bwd(q, k, v, o, do, lse, workspace=t(4, 4, dtype=torch.uint8))
    with pytest.raises(TypeError, match="workspace must be torch.uint8"):
        fa.fa_bwd(q, k, v, o, do, lse, workspace=t(16, dtype=torch.float32))
    with pytest.raises(ValueError, match="delta must have shape"):
        fa.fa_bwd_preprocess(o, do, delta=t(B, H, 1, dtype=torch.float32))
    with pytest.raises(ValueError, match="delta must have shape"):
        fa.fa_bwd_dkdv(q, k, v, do, lse, t(B, H, 1, dtype=torch.float32))
    with pytest.raises(TypeError, match="delta must be torch.float32"):
        fa.fa_bwd_dq(q, k, v, do, lse, t(B, H, N))
    with pytest.raises(ValueError, match="o must have shape"):
        fa.fa_bwd_dq_delta(q, k, v, t(B, H, N, D // 2), do, lse)
    with pytest.raises(ValueError, match="delta must have shape"):
        fa.fa_bwd_dq_delta(q, k, v, o, do, lse, delta=t(B, H, N + 1, dtype=torch.float32))
    with pytest.raises(ValueError, match="GPU tensor"):
        fa.fa_bwd_dq_delta(q, k, v, o, do, lse)


def test_split_key_arguments():
    q = t(B, H, 3, D)
    k, v = t(B, H, 500, D), t(B, H, 500, D)
    with pytest.raises(ValueError, match="v must have shape"):
        fa.fa_fwd_splitkv(q, k, t(B, H, 499, D))
    with pytest.raises(ValueError, match="k must have shape"):
        fa.fa_fwd_splitkv(q, t(B, H, 500, D + 32), v)
    with pytest.raises(TypeError, match="bfloat16 queries"):
        fa.fa_fwd_splitkv(q.float(), k.float(), v.float())
    with pytest.raises(ValueError, match="lse must have shape"):
        fa.fa_fwd_splitkv(q, k, v, lse=t(B, H, 500, dtype=torch.float32))
    with pytest.raises(TypeError, match="k must be torch.uint8"):
        fa.fa_fwd_splitkv_fp8kv(q, k, v, 1.0, 1.0)
    with pytest.raises(ValueError, match="GPU tensor"):
        fa.fa_fwd_splitkv(q, k, v)


def test_fp8_arguments():
    q8, k8, v8 = (x.to(torch.uint8) for x in qkv())
    with pytest.raises(TypeError, match="E4M3 codes"):
        fa.fa_fwd_fp8(q8.bfloat16(), k8, v8, 1.0, 1.0, 1.0)
    with pytest.raises(ValueError, match="k8 must have shape"):
        fa.fa_fwd_fp8(q8, k8[:, :, :-1].contiguous(), v8, 1.0, 1.0, 1.0)
    with pytest.raises(TypeError, match="o must be torch.bfloat16"):
        fa.fa_fwd_fp8(q8, k8, v8, 1.0, 1.0, 1.0, o=t(B, H, N, D, dtype=torch.float32))
    with pytest.raises(ValueError, match="GPU tensor"):
        fa.fa_fwd_fp8(q8, k8, v8, 1.0, 1.0, 1.0)
