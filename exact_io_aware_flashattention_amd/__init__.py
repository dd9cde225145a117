"""Python binding of libfa.so, the gfx950 exact IO-aware attention library.

Argument marshalling only: every step of the computation runs in the HIP
kernels behind the C ABI declared in include/fa.h.  PyTorch supplies device
memory and the current stream; tensors are passed as raw device pointers.
The functions keep the C names (fa_fwd, fa_bwd, ...), take torch tensors of
layout [B, H, N, d] and raise FAError when the library returns a non-zero
status.  There is no fallback: if libfa.so is missing, loading fails loudly.
"""
from __future__ import annotations

import ctypes
import math
import os
from typing import Optional

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libfa.so")

FA_BF16, FA_F32 = 0, 1
WALK_FWD, WALK_DKDV, WALK_DQ = 0, 1, 2
CELL = 128

EXPORTS = ("fa_fwd", "fa_bwd_workspace_bytes", "fa_bwd_dkdv_workspace_bytes", "fa_bwd", "fa_bwd_preprocess",
           "fa_bwd_dkdv", "fa_bwd_dq", "fa_bwd_dq_delta", "fa_fwd_dropout", "fa_bwd_dropout", "fa_fwd_splitkv_workspace_bytes",
           "fa_fwd_splitkv_num_splits", "fa_fwd_splitkv", "fa_fwd_splitkv_noalloc", "fa_fwd_splitkv_fp8kv", "fa_fwd_fp8", "fa_debug_visits", "fa_status_str")


class FAError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {fa_status_str(status)} (status {status})")


_lib = None


def load_library(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load libfa.so (built by __graft_entry__.build()).  torch is imported first
    so the library binds to the HIP runtime torch already loaded."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"libfa.so not found at {path}; build it with __graft_entry__.build()")
    try:
        import torch  # noqa: F401  (HIP runtime first)
    except ImportError:
        pass
    lib = ctypes.CDLL(path)
    P, I, F, S, U64 = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t, ctypes.c_uint64
    sig = {
        "fa_fwd": [P, P, P, P, P, I, I, I, I, F, I, P, P, I, P],
        "fa_bwd_workspace_bytes": [I, I, I, I, I, I],
        "fa_bwd_dkdv_workspace_bytes": [I, I, I, I],
        "fa_bwd": [P, P, P, P, P, P, P, P, P, I, I, I, I, F, I, P, P, I, P, S, P],
        "fa_bwd_preprocess": [P, P, P, I, I, I, I, I, P],
        "fa_bwd_dkdv": [P, P, P, P, P, P, P, P, I, I, I, I, F, I, P, P, I, P, S, P],
        "fa_bwd_dq": [P, P, P, P, P, P, P, I, I, I, I, F, I, P, P, I, P],
        "fa_bwd_dq_delta": [P, P, P, P, P, P, P, P, I, I, I, I, F, I, P, P, I, P],
        "fa_fwd_dropout": [P, P, P, P, P, I, I, I, I, F, I, P, P, I, F, U64, P],
        "fa_bwd_dropout": [P, P, P, P, P, P, P, P, P, I, I, I, I, F, I, P, P, I, F, U64, P, S, P],
        "fa_fwd_splitkv_workspace_bytes": [I, I, I, I, I, I],
        "fa_fwd_splitkv_num_splits": [I, I, I, I, I],
        "fa_fwd_splitkv": [P, P, P, P, P, I, I, I, I, I, F, I, P, I, I, P, S, P],
        "fa_fwd_splitkv_noalloc": [P, P, P, P, P, I, I, I, I, I, F, I, P, I, I, P],
        "fa_fwd_fp8": [P, P, P, P, P, I, I, I, I, F, I, P, P, F, F, F, P],
        "fa_fwd_splitkv_fp8kv": [P, P, P, P, P, I, I, I, I, I, F, I, P, F, F, I, P, S, P],
        "fa_debug_visits": [I, I, I, I, I, I, P, P, I, P, P, S, P],
        "fa_status_str": [I],
    }
    for name, args in sig.items():
        fn = getattr(lib, name)
        fn.argtypes = args
        fn.restype = ctypes.c_int
    lib.fa_bwd_workspace_bytes.restype = ctypes.c_size_t
    lib.fa_bwd_dkdv_workspace_bytes.restype = ctypes.c_size_t
    lib.fa_fwd_splitkv_workspace_bytes.restype = ctypes.c_size_t
    lib.fa_status_str.restype = ctypes.c_char_p
    _lib = lib
    return lib


def fa_status_str(status: int) -> str:
    return load_library().fa_status_str(int(status)).decode()


# ---------------------------------------------------------------- marshalling helpers

def _ptr(t) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _stream(stream) -> Optional[int]:
    import torch
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def _dtype_code(t) -> int:
    import torch
    if t.dtype == torch.bfloat16:
        return FA_BF16
    if t.dtype == torch.float32:
        return FA_F32
    raise TypeError(f"unsupported dtype {t.dtype}; use bfloat16 or float32")


def _shape(t):
    if t.dim() != 4:
        raise ValueError("expected a [B, H, N, d] tensor")
    return tuple(int(x) for x in t.shape)


# The C ABI receives bare pointers and cannot see how large an allocation is:
# every tensor is checked here, before any library call, for the device, the
# dtype, the shape and the layout the kernels assume.  A mismatch raises
# TypeError (dtype) or ValueError (anything else).

def _on_gpu(name, t, ref):
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor (got device {t.device})")
    if t.device != ref.device:
        raise ValueError(f"{name} is on {t.device}, expected {ref.device}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _like(name, t, shape, dtype):
    import torch
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")


def _validate(ref, specs):
    """specs: (name, tensor or None, shape, dtype).  Dtypes and shapes are
    checked first, then that every tensor (and ref) is a contiguous GPU tensor
    on ref's device."""
    live = [(n, t, s, dt) for n, t, s, dt in specs if t is not None]
    for n, t, s, dt in live:
        _like(n, t, s, dt)
    for n, t, _, _ in live:
        _on_gpu(n, t, ref)


def _mask_specs(B, N, block_mask, kv_len):
    import torch
    T = -(-N // CELL)
    return [("block_mask", block_mask, (T, T), torch.uint8), ("kv_len", kv_len, (B,), torch.int32)]


def _workspace_spec(workspace):
    import torch
    if workspace is not None and workspace.dim() != 1:
        raise ValueError("workspace must be a 1-D uint8 tensor")
    return [("workspace", workspace, tuple(workspace.shape) if workspace is not None else (), torch.uint8)]


def _check_square(q, named, B, H, N, block_mask=None, kv_len=None, stats=(), workspace=None):
    """q: [B,H,N,d] bf16/f32 on the GPU; every tensor of ``named`` has q's shape
    and dtype; every tensor of ``stats`` is float32 [B,H,N]."""
    import torch
    _dtype_code(q)
    specs = [("q", q, q.shape, q.dtype)] + [(n, t, q.shape, q.dtype) for n, t in named]
    specs += [(n, t, (B, H, N), torch.float32) for n, t in stats]
    _validate(q, specs + _mask_specs(B, N, block_mask, kv_len) + _workspace_spec(workspace))


def _call(name, *args):
    st = getattr(load_library(), name)(*args)
    if st != 0:
        raise FAError(st, name)


def _mask_args(block_mask, kv_len):
    return _ptr(block_mask), _ptr(kv_len)


def _scale(scale, d):
    return float(1.0 / math.sqrt(d) if scale is None else scale)


# ---------------------------------------------------------------- entry points

def _new(shape, dtype, ref):
    import torch
    return torch.empty(shape, dtype=dtype, device=ref.device)


def fa_fwd(q, k, v, o=None, lse=None, *, scale=None, causal=False, block_mask=None, kv_len=None,
           dropout_p=0.0, seed=0, stream=None):
    """O, lse = attention forward.  q, k, v: [B,H,N,d] bf16 or float32 on the GPU;
    block_mask: uint8 [T,T] (T = ceil(N/128)) or None; kv_len: int32 [B] or None;
    dropout_p > 0 applies dropout on P (bf16 only; rate rounded to a multiple
    of 1/256) with the Philox stream of `seed`."""
    import torch
    B, H, N, d = _shape(q)
    _check_square(q, [("k", k), ("v", v), ("o", o)], B, H, N, block_mask, kv_len, [("lse", lse)])
    o = _new(q.shape, q.dtype, q) if o is None else o
    lse = _new((B, H, N), torch.float32, q) if lse is None else lse
    mb, kl = _mask_args(block_mask, kv_len)
    if dropout_p:
        _call("fa_fwd_dropout", _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), B, H, N, d, _scale(scale, d),
              int(bool(causal)), mb, kl, _dtype_code(q), float(dropout_p), int(seed), _stream(stream))
    else:
        _call("fa_fwd", _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), B, H, N, d, _scale(scale, d),
              int(bool(causal)), mb, kl, _dtype_code(q), _stream(stream))
    return o, lse


NOALLOC_SCRATCH_BYTES = 64 << 20     # FA_NOALLOC_SCRATCH_BYTES of include/fa.h


def fa_fwd_splitkv_noalloc(q, k, v, o, lse, *, scale=None, causal=False, kv_len=None, num_splits=0, stream=None):
    """fa_fwd_splitkv into caller-provided o and lse, with the partial results in
    the library's fixed per-GPU scratch instead of a workspace (for callers
    that cannot allocate; nothing is allocated here either)."""
    import torch
    if o is None or lse is None:
        raise ValueError("fa_fwd_splitkv_noalloc writes into caller-provided o and lse")
    B, H, Nq, Nk, d = _check_split(q, k, v, o, lse, kv_len, torch.bfloat16, None)
    _call("fa_fwd_splitkv_noalloc", _ptr(q), _ptr(k) if Nk else None, _ptr(v) if Nk else None, _ptr(o), _ptr(lse),
          B, H, Nq, Nk, d, _scale(scale, d), int(bool(causal)), _ptr(kv_len), _dtype_code(q), int(num_splits),
          _stream(stream))
    return o, lse


def _check_split(q, k, v, o, lse, kv_len, kv_dtype, workspace):
    """q: bf16 [B,H,Nq,d]; k, v: kv_dtype [B,H,Nk,d]; o like q; lse f32 [B,H,Nq]."""
    import torch
    B, H, Nq, d = _shape(q)
    _, _, Nk, _ = _shape(k)
    if q.dtype != torch.bfloat16:
        raise TypeError("the split-key forward takes bfloat16 queries")
    _validate(q, [("q", q, q.shape, q.dtype), ("k", k, (B, H, Nk, d), kv_dtype), ("v", v, (B, H, Nk, d), kv_dtype),
                  ("o", o, q.shape, q.dtype), ("lse", lse, (B, H, Nq), torch.float32),
                  ("kv_len", kv_len, (B,), torch.int32)] + _workspace_spec(workspace))
    return B, H, Nq, Nk, d


def fa_fwd_splitkv_fp8kv(q, k8, v8, k_descale, v_descale, o=None, lse=None, *, scale=None, causal=False,
                         kv_len=None, num_splits=0, workspace=None, stream=None):
    """Decoding (at most 4 bf16 queries [B,H,Nq,d]) against E4M3 K and V codes
    (uint8 [B,H,Nk,d]; real value = code * descale), keys split over ranges
    as fa_fwd_splitkv."""
    import torch
    B, H, Nq, Nk, d = _check_split(q, k8, v8, o, lse, kv_len, torch.uint8, workspace)
    o = _new(q.shape, q.dtype, q) if o is None else o
    lse = _new((B, H, Nq), torch.float32, q) if lse is None else lse
    ws, nbytes = _workspace(workspace, fa_fwd_splitkv_workspace_bytes(B, H, Nq, Nk, d, num_splits), q.device)
    _call("fa_fwd_splitkv_fp8kv", _ptr(q), _ptr(k8) if Nk else None, _ptr(v8) if Nk else None, _ptr(o), _ptr(lse),
          B, H, Nq, Nk, d, _scale(scale, d), int(bool(causal)), _ptr(kv_len), float(k_descale), float(v_descale),
          int(num_splits), _ptr(ws), nbytes, _stream(stream))
    return o, lse


def fa_fwd_fp8(q8, k8, v8, q_descale, k_descale, v_descale, o=None, lse=None, *, scale=None, causal=False,
               block_mask=None, kv_len=None, stream=None):
    """O (bf16), lse for E4M3 inputs: q8, k8, v8 are uint8 [B,H,N,d] tensors of
    OCP E4M3 codes whose real values are code * descale (one float per tensor)."""
    import torch
    B, H, N, d = _shape(q8)
    if q8.dtype != torch.uint8:
        raise TypeError("FP8 inputs are uint8 tensors of E4M3 codes")
    _validate(q8, [("q8", q8, q8.shape, torch.uint8), ("k8", k8, q8.shape, torch.uint8),
                   ("v8", v8, q8.shape, torch.uint8), ("o", o, q8.shape, torch.bfloat16),
                   ("lse", lse, (B, H, N), torch.float32)] + _mask_specs(B, N, block_mask, kv_len))
    o = _new((B, H, N, d), torch.bfloat16, q8) if o is None else o
    lse = _new((B, H, N), torch.float32, q8) if lse is None else lse
    mb, kl = _mask_args(block_mask, kv_len)
    _call("fa_fwd_fp8", _ptr(q8), _ptr(k8), _ptr(v8), _ptr(o), _ptr(lse), B, H, N, d, _scale(scale, d),
          int(bool(causal)), mb, kl, float(q_descale), float(k_descale), float(v_descale), _stream(stream))
    return o, lse


def fa_bwd_workspace_bytes(B, H, N, d, dtype=FA_BF16, has_block_mask=False) -> int:
    return int(load_library().fa_bwd_workspace_bytes(B, H, N, d, dtype, int(bool(has_block_mask))))


def fa_bwd_dkdv_workspace_bytes(N, d, dtype=FA_BF16, has_block_mask=False) -> int:
    return int(load_library().fa_bwd_dkdv_workspace_bytes(N, d, dtype, int(bool(has_block_mask))))


def _workspace(workspace, need, device):
    import torch
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=device)
    if workspace is None:
        return None, 0
    return workspace, workspace.numel() * workspace.element_size()


def fa_fwd_splitkv_workspace_bytes(B, H, Nq, Nk, d, num_splits=0) -> int:
    return int(load_library().fa_fwd_splitkv_workspace_bytes(B, H, Nq, Nk, d, num_splits))


def fa_fwd_splitkv_num_splits(B, H, Nq, Nk, num_splits=0) -> int:
    return int(load_library().fa_fwd_splitkv_num_splits(B, H, Nq, Nk, num_splits))


def fa_fwd_splitkv(q, k, v, o=None, lse=None, *, scale=None, causal=False, kv_len=None, num_splits=0,
                   workspace=None, stream=None):
    """O, lse for Nq queries [B,H,Nq,d] against Nk keys k, v [B,H,Nk,d] (bf16),
    with the keys split over num_splits ranges (0 = chosen from the sizes)
    whose partial results are merged.  causal aligns the queries with the
    last Nq key positions (key j allowed for query i iff j <= i + Nk - Nq)."""
    import torch
    B, H, Nq, Nk, d = _check_split(q, k, v, o, lse, kv_len, torch.bfloat16, workspace)
    o = _new(q.shape, q.dtype, q) if o is None else o
    lse = _new((B, H, Nq), torch.float32, q) if lse is None else lse
    ws, nbytes = _workspace(workspace, fa_fwd_splitkv_workspace_bytes(B, H, Nq, Nk, d, num_splits), q.device)
    _call("fa_fwd_splitkv", _ptr(q), _ptr(k) if Nk else None, _ptr(v) if Nk else None, _ptr(o), _ptr(lse), B, H,
          Nq, Nk, d, _scale(scale, d), int(bool(causal)), _ptr(kv_len), _dtype_code(q), int(num_splits), _ptr(ws),
          nbytes, _stream(stream))
    return o, lse


def fa_bwd(q, k, v, o, dO, lse, dq=None, dk=None, dv=None, *, scale=None, causal=False, block_mask=None,
           kv_len=None, dropout_p=0.0, seed=0, workspace=None, stream=None):
    """dQ, dK, dV for the loss gradient dO, from the forward's O and lse (with
    the same dropout_p and seed as the forward)."""
    B, H, N, d = _shape(q)
    _check_square(q, [("k", k), ("v", v), ("o", o), ("dO", dO), ("dq", dq), ("dk", dk), ("dv", dv)],
                  B, H, N, block_mask, kv_len, [("lse", lse)], workspace)
    dq = _new(q.shape, q.dtype, q) if dq is None else dq
    dk = _new(q.shape, q.dtype, q) if dk is None else dk
    dv = _new(q.shape, q.dtype, q) if dv is None else dv
    need = fa_bwd_workspace_bytes(B, H, N, d, _dtype_code(q), block_mask is not None)
    workspace, ws_bytes = _workspace(workspace, max(need, 256), q.device)
    mb, kl = _mask_args(block_mask, kv_len)
    if dropout_p:
        _call("fa_bwd_dropout", _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(dO), _ptr(lse), _ptr(dq), _ptr(dk),
              _ptr(dv), B, H, N, d, _scale(scale, d), int(bool(causal)), mb, kl, _dtype_code(q),
              float(dropout_p), int(seed), _ptr(workspace), ws_bytes, _stream(stream))
    else:
        _call("fa_bwd", _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(dO), _ptr(lse), _ptr(dq), _ptr(dk), _ptr(dv),
              B, H, N, d, _scale(scale, d), int(bool(causal)), mb, kl, _dtype_code(q), _ptr(workspace),
              ws_bytes, _stream(stream))
    return dq, dk, dv


def fa_bwd_preprocess(o, dO, delta=None, *, stream=None):
    import torch
    B, H, N, d = _shape(o)
    _dtype_code(o)
    _validate(o, [("o", o, o.shape, o.dtype), ("dO", dO, o.shape, o.dtype), ("delta", delta, (B, H, N), torch.float32)])
    delta = _new((B, H, N), torch.float32, o) if delta is None else delta
    _call("fa_bwd_preprocess", _ptr(o), _ptr(dO), _ptr(delta), B, H, N, d, _dtype_code(o), _stream(stream))
    return delta


def fa_bwd_dkdv(q, k, v, dO, lse, delta, dk=None, dv=None, *, scale=None, causal=False, block_mask=None,
                kv_len=None, workspace=None, stream=None):
    B, H, N, d = _shape(q)
    _check_square(q, [("k", k), ("v", v), ("dO", dO), ("dk", dk), ("dv", dv)], B, H, N,
                  block_mask, kv_len, [("lse", lse), ("delta", delta)], workspace)
    dk = _new(q.shape, q.dtype, q) if dk is None else dk
    dv = _new(q.shape, q.dtype, q) if dv is None else dv
    need = fa_bwd_dkdv_workspace_bytes(N, d, _dtype_code(q), block_mask is not None)
    workspace, ws_bytes = _workspace(workspace, need, q.device)
    mb, kl = _mask_args(block_mask, kv_len)
    _call("fa_bwd_dkdv", _ptr(q), _ptr(k), _ptr(v), _ptr(dO), _ptr(lse), _ptr(delta), _ptr(dk), _ptr(dv),
          B, H, N, d, _scale(scale, d), int(bool(causal)), mb, kl, _dtype_code(q), _ptr(workspace), ws_bytes,
          _stream(stream))
    return dk, dv


def fa_bwd_dq(q, k, v, dO, lse, delta, dq=None, *, scale=None, causal=False, block_mask=None, kv_len=None,
              stream=None):
    B, H, N, d = _shape(q)
    _check_square(q, [("k", k), ("v", v), ("dO", dO), ("dq", dq)], B, H, N, block_mask, kv_len,
                  [("lse", lse), ("delta", delta)])
    dq = _new(q.shape, q.dtype, q) if dq is None else dq
    mb, kl = _mask_args(block_mask, kv_len)
    _call("fa_bwd_dq", _ptr(q), _ptr(k), _ptr(v), _ptr(dO), _ptr(lse), _ptr(delta), _ptr(dq),
          B, H, N, d, _scale(scale, d), int(bool(causal)), mb, kl, _dtype_code(q), _stream(stream))
    return dq


def fa_bwd_dq_delta(q, k, v, o, dO, lse, delta=None, dq=None, *, scale=None, causal=False, block_mask=None,
                    kv_len=None, stream=None):
    """dq and delta = rowsum(dO * O) in one stage (fa_bwd_preprocess + fa_bwd_dq
    for bf16 in one kernel).  Returns (dq, delta)."""
    import torch
    B, H, N, d = _shape(q)
    _check_square(q, [("k", k), ("v", v), ("o", o), ("dO", dO), ("dq", dq)], B, H, N, block_mask, kv_len,
                  [("lse", lse), ("delta", delta)])
    dq = _new(q.shape, q.dtype, q) if dq is None else dq
    delta = _new((B, H, N), torch.float32, q) if delta is None else delta
    mb, kl = _mask_args(block_mask, kv_len)
    _call("fa_bwd_dq_delta", _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(dO), _ptr(lse), _ptr(delta), _ptr(dq),
          B, H, N, d, _scale(scale, d), int(bool(causal)), mb, kl, _dtype_code(q), _stream(stream))
    return dq, delta


def fa_debug_visits(which, B, H, N, d, *, causal=False, block_mask=None, kv_len=None, dtype=FA_BF16,
                    device="cuda", workspace=None, stream=None):
    """Visit counters [B, T, T] (uint32 stored in int32) of the forward (0),
    dK/dV (1) or dQ (2) tile walk."""
    import torch
    T = -(-N // CELL)
    counts = torch.zeros((B, T, T), dtype=torch.int32, device=device)
    _validate(counts, _mask_specs(B, N, block_mask, kv_len) + _workspace_spec(workspace))
    need = fa_bwd_dkdv_workspace_bytes(N, d, dtype, block_mask is not None) if which == WALK_DKDV else 0
    workspace, ws_bytes = _workspace(workspace, need, device)
    mb, kl = _mask_args(block_mask, kv_len)
    _call("fa_debug_visits", int(which), B, H, N, d, int(bool(causal)), mb, kl, int(dtype), _ptr(counts),
          _ptr(workspace), ws_bytes, _stream(stream))
    return counts
