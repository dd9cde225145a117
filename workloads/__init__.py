"""Seeded synthetic workloads for the attention hot path.

This module only draws random numbers and arranges them into the shapes of the
workloads; it holds none of the attention arithmetic.  Both the CPU oracle
(through the tests and the bench) and the HIP library receive exactly the
arrays produced here.

Workload shapes follow the pages: the GPT-2 shape N=1024, d=64 (bornlex.github.io
"Flash Attention", section "Standard Attention"), BERT-large at sequence length
512 and the 16K / 64K block-sparse long sequences (FlashAttention reading guide,
xyznot.com, section "Hasil"), and head dimension 256 at the 16K shape (datacamp
"Penjelasan Flash Attention", Flash Attention 2, "Dukungan untuk dimensi head
yang lebih besar").  No dataset item is used: values are i.i.d.
normals.

Recipe (all randomness is numpy PCG64):
  * workload k draws fp32 standard normals from PCG64(k) in the order
    Q, K, V, dO, each multiplied by sigma; bf16 workloads are then rounded
    to the nearest bf16 (ties to even), so the CPU and the GPU see the
    same values;
  * key-padding lengths come from PCG64(1000 + k), uniform integers in
    [lo, hi] inclusive;
  * the random cells of the block mask come from PCG64(2000 + k).
"""
from __future__ import annotations

import dataclasses
import hashlib
import math
from typing import Optional

import numpy as np

CELL = 128  # block-mask cell edge (queries x keys), fixed by the 64K workload


@dataclasses.dataclass(frozen=True)
class Workload:
    key: int
    name: str
    B: int
    H: int
    N: int
    d: int
    dtype: str            # "bf16" or "f32"
    causal: bool
    scale: float
    sigma: float          # standard deviation of Q, K, V
    kv_len_range: Optional[tuple] = None   # (lo, hi) inclusive, per batch entry
    block_sparse: bool = False

    @property
    def cells(self) -> int:
        return -(-self.N // CELL)


WORKLOADS = {
    1: Workload(1, "tiny-exact", 1, 2, 128, 64, "f32", False, 1.0 / 8.0, 1.0),
    2: Workload(2, "gpt2-train", 8, 12, 1024, 64, "bf16", True, 1.0 / 8.0, 1.0),
    3: Workload(3, "bert-large-padded", 32, 16, 512, 64, "bf16", False, 1.0 / 8.0, 1.0,
                kv_len_range=(128, 512)),
    # "N(0, 0.5)" read as variance 0.5
    4: Workload(4, "long-context", 1, 16, 16384, 128, "bf16", True, 1.0 / math.sqrt(128.0),
                math.sqrt(0.5)),
    5: Workload(5, "block-sparse-64k", 1, 8, 65536, 64, "bf16", False, 1.0 / 8.0, 1.0,
                block_sparse=True),
    # head dimension 256 (the FA2 extension): the long-context shape with the
    # same H * d and flops as workload 4
    6: Workload(6, "long-context-d256", 1, 8, 16384, 256, "bf16", True, 1.0 / 16.0, math.sqrt(0.5)),
    # head dimensions 96 and 160 (not powers of two): the long-context shape
    # with d changed
    7: Workload(7, "long-context-d96", 1, 16, 16384, 96, "bf16", True, 1.0 / math.sqrt(96.0), math.sqrt(0.5)),
    8: Workload(8, "long-context-d160", 1, 16, 16384, 160, "bf16", True, 1.0 / math.sqrt(160.0), math.sqrt(0.5)),
}


def bf16_round(x: np.ndarray):
    """Round fp32 values to bf16, nearest with ties to even.

    Returns (values as float32, raw bf16 bit patterns as uint16)."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    r = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)
    return (r.astype(np.uint32) << 16).view(np.float32), r


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def draw_qkvdo(B, H, N, d, dtype="bf16", sigma=1.0, seed=0):
    """Q, K, V, dO as fp32 arrays [B,H,N,d] (bf16-exact when dtype is bf16)."""
    rng = np.random.Generator(np.random.PCG64(seed))
    out = []
    for _ in range(4):
        a = rng.standard_normal((B, H, N, d), dtype=np.float32)
        if sigma != 1.0:
            a *= np.float32(sigma)
        if dtype == "bf16":
            a, _ = bf16_round(a)
        out.append(a)
    return tuple(out)


# Split-key forward workloads: few queries against a long key/value sequence
# (the small-batch, long-prompt inference case of the sequence-parallel
# discussion).  Values as the long-context workload: N(0, 0.5), bf16.
SPLITKV_WORKLOADS = {
    "decode": dict(B=16, H=16, Nq=1, Nk=16384, d=128, causal=False, sigma=math.sqrt(0.5), seed=21,
                   desc="decode: B=16 H=16, one query against 16384 keys, d=128 bf16, scale 1/sqrt(128)"),
    "prefill": dict(B=1, H=16, Nq=2048, Nk=16384, d=128, causal=True, sigma=math.sqrt(0.5), seed=22,
                    desc="chunked prefill: the last 2048 queries of the 16384-token causal long context, "
                         "B=1 H=16 d=128 bf16, scale 1/sqrt(128)"),
}


def draw_split_qkv(B, H, Nq, Nk, d, sigma=1.0, seed=0):
    """Q [B,H,Nq,d], K and V [B,H,Nk,d] as bf16-exact fp32 arrays.  Batch entry
    b of tensor t (0 = Q, 1 = K, 2 = V) is fp32 standard normals drawn from
    PCG64(seed) jumped 3 b + t + 1 times, times sigma, rounded to bf16
    (nearest, ties to even).  Entries are drawn on parallel threads."""
    import os
    from concurrent.futures import ThreadPoolExecutor
    base = np.random.PCG64(seed)
    out = [np.empty((B, H, n, d), np.float32) for n in (Nq, Nk, Nk)]

    def fill(job):
        b, t = job
        rng = np.random.Generator(base.jumped(3 * b + t + 1))
        x = rng.standard_normal(out[t].shape[1:], dtype=np.float32)
        if sigma != 1.0:
            x *= np.float32(sigma)
        out[t][b] = _bf16_round_finite(x)

    workers = max(1, min(8, len(os.sched_getaffinity(0))))
    with ThreadPoolExecutor(workers) as ex:
        list(ex.map(fill, [(b, t) for b in range(B) for t in range(3)]))
    return tuple(out)


def _bf16_round_finite(x: np.ndarray) -> np.ndarray:
    """bf16_round's values for finite fp32 input, in 32-bit integer arithmetic
    (no carry leaves 32 bits for finite values)."""
    u = np.ascontiguousarray(x, np.float32).view(np.uint32)
    r = (u + np.uint32(0x7FFF) + ((u >> 16) & np.uint32(1))) >> 16
    return (r << 16).view(np.float32)


def quantize_e4m3(x):
    """Per-tensor quantization to OCP E4M3 codes: descale = max|x| / 448 (1 if
    x is all zero), codes = E4M3(x / descale) rounded to nearest even by
    torch's float8_e4m3fn conversion.  Returns (uint8 codes, float32 descale)."""
    import torch
    x = np.asarray(x, np.float32)
    amax = float(np.abs(x).max()) if x.size else 0.0
    descale = np.float32(amax / 448.0 if amax > 0 else 1.0)
    y = np.clip(x / descale, -448.0, 448.0).astype(np.float32)
    codes = torch.from_numpy(y).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    return codes, descale


def draw_qkv_fp8(B, H, N, d, sigma=1.0, seed=0):
    """Q, K, V as E4M3 codes with their descale factors: fp32 normals times
    sigma from PCG64(seed) (drawn as draw_qkvdo draws Q, K, V), each tensor
    quantized by quantize_e4m3.  Returns ((q8, dq), (k8, dk), (v8, dv))."""
    rng = np.random.Generator(np.random.PCG64(seed))
    out = []
    for _ in range(3):
        a = rng.standard_normal((B, H, N, d), dtype=np.float32)
        if sigma != 1.0:
            a *= np.float32(sigma)
        out.append(quantize_e4m3(a))
    return tuple(out)


def draw_kv_len(B, lo, hi, seed):
    rng = np.random.Generator(np.random.PCG64(seed))
    return rng.integers(lo, hi, size=B, endpoint=True).astype(np.int32)


def band_random_mask(T, seed, below=2, above=1, n_random=2, global_col=True):
    """{0,1} mask of T x T cells: a band of cells j in [i-below, i+above],
    the first cell column (global keys) and n_random extra cells per row drawn
    without replacement from the row's remaining zero cells."""
    rng = np.random.Generator(np.random.PCG64(seed))
    m = np.zeros((T, T), dtype=np.uint8)
    for i in range(T):
        m[i, max(0, i - below):min(T, i + above + 1)] = 1
    if global_col:
        m[:, 0] = 1
    for i in range(T):
        free = np.flatnonzero(m[i] == 0)
        if n_random and free.size:
            pick = rng.choice(free, size=min(n_random, free.size), replace=False)
            m[i, pick] = 1
    return m


def make_inputs(w: Workload, seed: Optional[int] = None, N: Optional[int] = None,
                B: Optional[int] = None, H: Optional[int] = None):
    """All arrays of one workload. N/B/H may be overridden (smaller parity cases
    with the same value distribution and structure)."""
    seed = w.key if seed is None else seed
    B = w.B if B is None else B
    H = w.H if H is None else H
    N = w.N if N is None else N
    q, k, v, do = draw_qkvdo(B, H, N, w.d, w.dtype, w.sigma, seed)
    kv_len = None
    if w.kv_len_range is not None:
        lo, hi = w.kv_len_range
        kv_len = draw_kv_len(B, min(lo, N), min(hi, N), 1000 + seed)
    mask = None
    if w.block_sparse:
        mask = band_random_mask(-(-N // CELL), 2000 + seed)
    return dict(q=q, k=k, v=v, do=do, kv_len=kv_len, block_mask=mask,
                B=B, H=H, N=N, d=w.d, dtype=w.dtype, causal=w.causal, scale=w.scale)


def digest(*arrays) -> str:
    h = hashlib.sha256()
    for a in arrays:
        if a is not None:
            h.update(np.ascontiguousarray(a).tobytes())
    return h.hexdigest()[:16]
