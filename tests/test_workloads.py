"""The seeded input generators: determinism, rounding and structure."""
import numpy as np

from workloads import (WORKLOADS, band_random_mask, bf16_bits_to_f32, bf16_round,
                       digest, draw_kv_len, draw_qkvdo, make_inputs)


def test_bf16_round_to_nearest_even():
    one = np.float32(1.0)
    vals = np.array([1.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, 1.0 + 2 ** -9, -2.5, 0.0,
                     3.0e38, 1.0 + 2 ** -8 + 2 ** -20], dtype=np.float32)
    r, bits = bf16_round(vals)
    # 1 + 2^-8 is a tie between 1 and 1 + 2^-7: even mantissa -> 1
    # 1 + 3*2^-8 is a tie between 1 + 2^-7 and 1 + 2^-6: even -> 1 + 2^-6
    want = [1.0, 1.0, 1.0 + 2 ** -6, 1.0, -2.5, 0.0, None, 1.0 + 2 ** -7]
    for got, w in zip(r, want):
        if w is not None:
            assert got == np.float32(w)
    assert np.array_equal(bf16_bits_to_f32(bits), r)
    assert bits[0] == 0x3F80 and one == r[0]


def test_generators_are_deterministic():
    a = draw_qkvdo(1, 2, 64, 8, "bf16", 1.0, seed=3)
    b = draw_qkvdo(1, 2, 64, 8, "bf16", 1.0, seed=3)
    c = draw_qkvdo(1, 2, 64, 8, "bf16", 1.0, seed=4)
    assert digest(*a) == digest(*b) != digest(*c)
    for x in a:
        assert np.array_equal(bf16_round(x)[0], x)       # already bf16-exact


def test_kv_len_range():
    L = draw_kv_len(32, 128, 512, 1003)
    assert L.min() >= 128 and L.max() <= 512 and L.dtype == np.int32
    assert np.array_equal(L, draw_kv_len(32, 128, 512, 1003))


def test_block_sparse_mask_structure():
    T = 512
    m = band_random_mask(T, 2005)
    assert int(m.sum()) == 3577                              # 2044 band + 509 column + 1024 random
    for i in range(T):
        assert all(m[i, j] for j in range(max(0, i - 2), min(T, i + 2)))
        assert m[i, 0] == 1
    band = np.zeros_like(m)
    for i in range(T):
        band[i, max(0, i - 2):min(T, i + 2)] = 1
    band[:, 0] = 1
    assert np.all((m - band).sum(axis=1) == 2)


def test_workload_table():
    assert WORKLOADS[4].N == 16384 and WORKLOADS[4].d == 128 and WORKLOADS[4].causal
    assert abs(WORKLOADS[4].sigma ** 2 - 0.5) < 1e-12
    x = make_inputs(WORKLOADS[3], N=256, B=4, H=2)
    assert x["kv_len"].shape == (4,) and x["kv_len"].max() <= 256
    x = make_inputs(WORKLOADS[5], N=1024, H=1)
    assert x["block_mask"].shape == (8, 8)
