"""The C ABI without a GPU: the library loads, exports every declared entry point,
and rejects bad arguments synchronously (no call here reaches a launch)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fa.h")

fa = pytest.importorskip("exact_io_aware_flashattention_amd")

if not os.path.exists(fa.LIB_PATH):
    pytest.skip("libfa.so not built (run __graft_entry__.build())", allow_module_level=True)


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(fa_[a-z_0-9]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    return fa.load_library()


def test_exports_every_declared_symbol(lib):
    names = declared_functions()
    assert set(names) == set(fa.EXPORTS)
    for n in names:
        assert hasattr(lib, n), n


def test_status_strings(lib):
    for s in range(9):
        assert fa.fa_status_str(s).startswith("FA_")
    assert "unknown" in fa.fa_status_str(99)


def test_workspace_is_linear_in_n(lib):
    w1 = lib.fa_bwd_workspace_bytes(1, 16, 16384, 128, 0, 0)
    w2 = lib.fa_bwd_workspace_bytes(1, 16, 32768, 128, 0, 0)
    assert w1 >= 16 * 16384 * 4 and w2 == 2 * w1
    assert lib.fa_bwd_workspace_bytes(0, 1, 1, 64, 0, 0) == 0


def test_split_workspace_size(lib):
    """The dK/dV split workspace: only bf16 with a block mask, bounded slot pool
    (1024 chunks x 128 keys x d x {dK, dV} x fp32) plus a mask-sized count table."""
    for d in (64, 128):
        pool = 1024 * 2 * 128 * d * 4
        T = 512
        w = lib.fa_bwd_dkdv_workspace_bytes(T * 128, d, 0, 1)
        assert pool <= w <= pool + 64 * 1024 + (T // 64) * T * 4 + 1024
        assert lib.fa_bwd_dkdv_workspace_bytes(T * 128, d, 0, 0) == 0
        assert lib.fa_bwd_dkdv_workspace_bytes(T * 128, d, 1, 1) == 0      # float32 path: none
        full = lib.fa_bwd_workspace_bytes(2, 3, T * 128, d, 0, 1)
        assert full == lib.fa_bwd_workspace_bytes(2, 3, T * 128, d, 0, 0) + w
        # independent of B and H
        assert lib.fa_bwd_dkdv_workspace_bytes(T * 128, d, 0, 1) == w


FAKE = 1 << 20          # an aligned, never-dereferenced address


def fwd(lib, **kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, o=FAKE, lse=FAKE, B=1, H=1, N=128, d=64, scale=0.125, causal=0,
             mask=None, kv=None, dtype=0, stream=None)
    a.update(kw)
    return lib.fa_fwd(a["q"], a["k"], a["v"], a["o"], a["lse"], a["B"], a["H"], a["N"], a["d"],
                      a["scale"], a["causal"], a["mask"], a["kv"], a["dtype"], a["stream"])


def test_forward_validation(lib):
    assert fwd(lib, q=None) == 1                       # FA_ERR_NULL
    assert fwd(lib, lse=None) == 1
    for d in (32, 80, 192, 320):
        assert fwd(lib, d=d) == 2                      # FA_ERR_SHAPE
    for d in (96, 160, 256):
        assert fwd(lib, d=d, dtype=1) == 2             # bf16 only
        assert fwd(lib, d=d, scale=-1.0) == 7          # bf16 passes the shape check
    # d = 96, 160: padded LDS rows need a head of at most 2^31 bytes (N d <= 2^30)
    n_max = (1 << 30) // 96
    assert fwd(lib, d=96, N=n_max, scale=-1.0) == 7
    assert fwd(lib, d=96, N=n_max + 1, scale=-1.0) == 2
    assert fwd(lib, d=128, N=n_max + 1, scale=-1.0) == 7
    assert fwd(lib, d=160, N=(1 << 30) // 160 + 1, scale=-1.0) == 2
    assert fwd(lib, N=-1) == 2
    assert fwd(lib, dtype=7) == 3                      # FA_ERR_DTYPE
    assert fwd(lib, k=FAKE + 8) == 4                   # FA_ERR_ALIGN
    assert fwd(lib, kv=FAKE + 2) == 4
    assert fwd(lib, scale=0.0) == 7                    # FA_ERR_ARG
    assert fwd(lib, scale=float("nan")) == 7
    assert fwd(lib, scale=-1.0) == 7
    assert fwd(lib, N=2049 * 128, mask=FAKE, scale=-1.0) == 2   # more than 2048 mask cells
    # empty problems succeed without touching the device (pointers may be NULL)
    assert fwd(lib, N=0, q=None, k=None) == 0
    assert fwd(lib, B=0) == 0


def test_backward_validation(lib):
    P = FAKE

    def bwd(ws_bytes=1 << 30, ws=P, scale=0.125, dq=P):
        return lib.fa_bwd(P, P, P, P, P, P, dq, P, P, 2, 4, 1000, 128, scale, 1, None, None, 0,
                          ws, ws_bytes, None)

    need = lib.fa_bwd_workspace_bytes(2, 4, 1000, 128, 0, 0)
    assert bwd(ws_bytes=need - 1) == 5                 # FA_ERR_WORKSPACE
    assert bwd(ws=None) == 1
    assert bwd(dq=None) == 1
    assert bwd(scale=float("inf")) == 7

    def bwd_masked(ws_bytes):
        return lib.fa_bwd(P, P, P, P, P, P, P, P, P, 2, 4, 1000, 128, 0.125, 1, P, None, 0, P, ws_bytes, None)

    # with a block mask the workspace grows by the dK/dV split part
    need_m = lib.fa_bwd_workspace_bytes(2, 4, 1000, 128, 0, 1)
    assert need_m > need
    assert bwd_masked(need) == 5
    assert bwd_masked(need_m - 1) == 5

    def dkdv(ws, ws_bytes, scale=0.125):
        return lib.fa_bwd_dkdv(P, P, P, P, P, P, P, P, 1, 1, 300, 64, scale, 0, P, None, 0, ws, ws_bytes, None)

    w = lib.fa_bwd_dkdv_workspace_bytes(300, 64, 0, 1)
    assert dkdv(None, w) == 1                          # bf16 + mask: FA_ERR_NULL
    assert dkdv(P + 8, w) == 4                         # FA_ERR_ALIGN
    assert dkdv(P, w - 1) == 5                         # FA_ERR_WORKSPACE
    assert dkdv(P, w, scale=-1.0) == 7
    assert lib.fa_bwd_dq(P, P, P, P, None, P, P, 1, 1, 100, 64, 0.1, 0, None, None, 0, None) == 1
    assert lib.fa_bwd_preprocess(P, P, P, 1, 1, 100, 80, 0, None) == 2


def test_dropout_validation(lib):
    def fwd_drop(p, dtype=0, seed=1):
        return lib.fa_fwd_dropout(FAKE, FAKE, FAKE, FAKE, FAKE, 1, 1, 128, 64, 0.125, 0, None, None, dtype, p, seed,
                                  None)
    # checks run before any launch: a rate outside [0, 1), or one that rounds to 256/256
    assert fwd_drop(-0.1) == 7 and fwd_drop(1.0) == 7 and fwd_drop(float("nan")) == 7
    assert fwd_drop(0.999) == 7          # rounds to t = 256
    assert fwd_drop(0.5, dtype=1) == 3   # the float32 path has no dropout
    P = FAKE
    r = lib.fa_bwd_dropout(P, P, P, P, P, P, P, P, P, 1, 1, 128, 64, 0.125, 0, None, None, 1, 0.25, 7, P, 1 << 20,
                           None)
    assert r == 3
    r = lib.fa_bwd_dropout(P, P, P, P, P, P, P, P, P, 1, 1, 128, 64, 0.125, 0, None, None, 0, 2.0, 7, P, 1 << 20, None)
    assert r == 7


def test_splitkv_plan_and_validation(lib):
    # At most 4 queries: one wave per (range, b, h), ranges of whole 64-key
    # tiles, when chosen as many as give one wave per SIMD (1024 = 256
    # compute units x 4).  More queries: one work-group per (range, b, h, 128
    # queries), ranges of whole 128-key cells, 512 resident work-groups.
    assert lib.fa_fwd_splitkv_num_splits(1, 1, 1, 16384, 0) == 256       # one tile each
    assert lib.fa_fwd_splitkv_num_splits(16, 16, 1, 16384, 0) == 4
    assert lib.fa_fwd_splitkv_num_splits(4, 16, 4, 16384, 0) == 16
    assert lib.fa_fwd_splitkv_num_splits(3, 16, 1, 16384, 0) == 20       # 21 asked, 13 tiles each
    assert lib.fa_fwd_splitkv_num_splits(1, 1, 1, 1000, 3) == 3
    assert lib.fa_fwd_splitkv_num_splits(1, 1, 1, 300, 64) == 5          # clamped to the tiles
    assert lib.fa_fwd_splitkv_num_splits(1, 1, 5, 300, 64) == 3          # clamped to the cells
    assert lib.fa_fwd_splitkv_num_splits(1, 16, 2048, 16384, 0) == 2
    assert lib.fa_fwd_splitkv_num_splits(3, 16, 5, 16384, 0) == 10       # 480 work-groups, not 528
    assert lib.fa_fwd_splitkv_num_splits(8, 16, 4096, 16384, 0) == 1     # 4096 groups already
    assert lib.fa_fwd_splitkv_num_splits(1, 1, 1, 0, 0) == 1
    assert lib.fa_fwd_splitkv_num_splits(1, 1, 1, 100, 1025) == 0
    assert lib.fa_fwd_splitkv_workspace_bytes(2, 3, 5, 1000, 64, 3) == 3 * 2 * 3 * 5 * (64 + 2) * 4
    assert lib.fa_fwd_splitkv_workspace_bytes(2, 3, 0, 1000, 64, 3) == 0
    P = FAKE
    need = lib.fa_fwd_splitkv_workspace_bytes(1, 2, 10, 500, 128, 0)

    def call(ws=P, nbytes=need, dtype=0, ns=0, d=128, scale=0.1, Nk=500, k=P):
        return lib.fa_fwd_splitkv(P, k, P, P, P, 1, 2, 10, Nk, d, scale, 1, None, dtype, ns, ws, nbytes, None)
    assert call(dtype=1) == 3                         # bf16 only
    assert call(d=80) == 2
    assert call(d=96, scale=0.0) == 7 and call(d=160, scale=0.0) == 7   # shapes accepted
    assert call(d=96, Nk=(1 << 30) // 96 + 1) == 2
    assert call(ns=1025) == 7 and call(ns=-1) == 7
    assert call(scale=0.0) == 7
    assert call(ws=None) == 1
    assert call(ws=P + 8) == 4
    assert call(nbytes=need - 1) == 5
    assert call(k=None) == 1
    assert lib.fa_fwd_splitkv(P, P, P, P, P, 1, 2, 0, 500, 128, 0.1, 0, None, 0, 0, None, 0, None) == 0


def test_fp8_validation(lib):
    P = FAKE

    def f8(d=128, scale=0.1, dq=1.0, dk=1.0, dv=1.0, q=P, N=128):
        return lib.fa_fwd_fp8(q, P, P, P, P, 1, 1, N, d, scale, 0, None, None, dq, dk, dv, None)
    assert f8(d=256) == 2 and f8(d=96) == 2            # d = 64 or 128
    assert f8(q=None) == 1
    assert f8(dq=0.0) == 7 and f8(dv=float("inf")) == 7 and f8(dk=-1.0) == 7
    assert f8(scale=1e30, dq=1e30) == 7               # scale * dq * dk overflows float32
    assert f8(N=0, q=None) == 0


def test_fp8kv_decode_validation(lib):
    P = FAKE
    need = lib.fa_fwd_splitkv_workspace_bytes(1, 2, 3, 500, 128, 0)

    def call(Nq=3, dk=1.0, dv=1.0, d=128, ns=0):
        return lib.fa_fwd_splitkv_fp8kv(P, P, P, P, P, 1, 2, Nq, 500, d, 0.1, 0, None, dk, dv, ns, P, need, None)
    assert call(Nq=5) == 2                              # decoding only: at most 4 queries
    assert call(dk=0.0) == 7 and call(dv=float("nan")) == 7
    assert call(d=80) == 2 and call(ns=2000) == 7
    assert call(d=160, dk=0.0) == 7                     # d = 160 passes the shape check


def test_debug_visits_validation(lib):
    assert lib.fa_debug_visits(3, 1, 1, 128, 64, 0, None, None, 0, FAKE, None, 0, None) == 7
    assert lib.fa_debug_visits(0, 1, 1, 128, 64, 0, None, None, 0, None, None, 0, None) == 1
    assert lib.fa_debug_visits(0, 1, 1, 0, 64, 0, None, None, 0, None, None, 0, None) == 0
    # the dK/dV walk under a block mask needs the split workspace
    assert lib.fa_debug_visits(1, 1, 1, 128, 64, 0, FAKE, None, 0, FAKE, None, 0, None) == 1
    assert lib.fa_debug_visits(1, 1, 1, 128, 64, 0, FAKE, None, 0, FAKE, FAKE, 1, None) == 5


def test_library_links_only_hip_runtime():
    """The product library must not pull in torch or the oracle."""
    import subprocess
    out = subprocess.run(["readelf", "-d", fa.LIB_PATH], capture_output=True, text=True).stdout
    needed = re.findall(r"\[(.*?)\]", "\n".join(l for l in out.splitlines() if "NEEDED" in l))
    assert any("amdhip64" in n for n in needed)
    assert not any("torch" in n or "python" in n for n in needed)


def test_noalloc_splitkv_validation(lib):
    """fa_fwd_splitkv_noalloc checks its arguments like fa_fwd_splitkv and
    refuses, before anything is launched, sizes whose partial results would
    not fit the fixed scratch (64 MiB)."""
    P = FAKE
    assert fa.NOALLOC_SCRATCH_BYTES == 64 << 20
    text = open(HEADER).read()
    assert "#define FA_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)" in text

    def call(B=1, H=2, Nq=10, Nk=500, d=128, dtype=0, ns=0, scale=0.1, k=P, q=P):
        return lib.fa_fwd_splitkv_noalloc(q, k, P, P, P, B, H, Nq, Nk, d, scale, 1, None, dtype, ns, None)
    big = dict(B=8, H=16, Nq=4096, Nk=16384, d=128, ns=2)
    assert lib.fa_fwd_splitkv_workspace_bytes(8, 16, 4096, 16384, 128, 2) > fa.NOALLOC_SCRATCH_BYTES
    assert call(**big) == 8
    assert "FA_ERR_SCRATCH" in fa.fa_status_str(8)
    assert call(dtype=1) == 3 and call(d=80) == 2 and call(ns=1025) == 7 and call(scale=0.0) == 7
    assert call(k=None) == 1 and call(q=P + 8) == 4
    assert call(Nq=0) == 0                  # nothing to compute
