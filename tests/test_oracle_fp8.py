"""Pins of the FP8 oracle (oracle/fp8.py): the E4M3 decoder against values the
OCP 8-bit floating point specification fixes and against torch's own
float8_e4m3fn conversion (an independent implementation), and the placement
of the descale factors."""
import numpy as np
import pytest

from oracle import attention, fp8
from workloads import draw_qkv_fp8, quantize_e4m3

# (code, value) pairs fixed by the E4M3 definition: bias 7, 3 mantissa bits,
# subnormals at exponent field 0, largest finite 448, S.1111.111 = NaN.
TABLE = [(0x00, 0.0), (0x80, -0.0), (0x38, 1.0), (0x40, 2.0), (0x3C, 1.5), (0x39, 1.125), (0xB8, -1.0),
         (0x7E, 448.0), (0xFE, -448.0), (0x08, 2.0 ** -6), (0x01, 2.0 ** -9), (0x07, 7 * 2.0 ** -9),
         (0x30, 0.5), (0x77, 240.0), (0x78, 256.0)]


@pytest.mark.parametrize("code,value", TABLE)
def test_decode_table(code, value):
    got = fp8.decode_e4m3(np.array([code], np.uint8))[0]
    assert got == value and np.signbit(got) == np.signbit(value)


def test_nan_codes():
    assert np.isnan(fp8.decode_e4m3(np.array([0x7F, 0xFF], np.uint8))).all()


def test_all_codes_match_torch():
    torch = pytest.importorskip("torch")
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = fp8.decode_e4m3(codes)
    both_nan = np.isnan(ref) & np.isnan(got)
    assert np.array_equal(got[~both_nan], ref[~both_nan]) and np.array_equal(np.isnan(got), np.isnan(ref))


def test_positive_codes_increase():
    v = fp8.decode_e4m3(np.arange(0x7F, dtype=np.uint8))
    assert np.all(np.diff(v) > 0)


def test_descales_enter_scores_and_values():
    """O(dq, dk, dv, scale) = dv O(1, 1, 1, scale dq dk) and lse likewise: the
    query and key descales scale the scores, the value descale the output."""
    (q8, dq), (k8, dk), (v8, dv) = draw_qkv_fp8(1, 2, 37, 16, 1.0, 70)
    O, lse = fp8.forward(q8, k8, v8, dq, dk, dv, 0.25, causal=True)
    O1, lse1 = fp8.forward(q8, k8, v8, 1.0, 1.0, 1.0, 0.25 * float(dq) * float(dk), causal=True)
    assert np.allclose(O, float(dv) * O1, rtol=1e-13, atol=1e-13)
    assert np.allclose(lse, lse1, rtol=1e-13, atol=1e-13)


def test_quantization_round_trip():
    """Codes decode to within half an E4M3 step of the scaled input, the
    largest magnitude maps to 448, and every code is finite."""
    rng = np.random.Generator(np.random.PCG64(71))
    x = rng.standard_normal(4096).astype(np.float32)
    codes, descale = quantize_e4m3(x)
    back = fp8.decode_e4m3(codes)
    assert np.isfinite(back).all() and np.abs(back).max() == 448.0
    y = x.astype(np.float64) / float(descale)
    step = np.where(np.abs(y) >= 2.0 ** -6, 2.0 ** (np.floor(np.log2(np.maximum(np.abs(y), 1e-300))) - 3), 2.0 ** -9)
    assert np.all(np.abs(back - y) <= step / 2 + 1e-12 * np.abs(y))


def test_forward_is_attention_of_the_real_values():
    (q8, dq), (k8, dk), (v8, dv) = draw_qkv_fp8(1, 1, 20, 8, 1.0, 72)
    O, _ = fp8.forward(q8, k8, v8, dq, dk, dv, 0.3)
    Q, K, V = (fp8.decode_e4m3(c)[0, 0] * float(s) for c, s in ((q8, dq), (k8, dk), (v8, dv)))
    S = 0.3 * Q @ K.T
    P = np.exp(S - S.max(axis=1, keepdims=True))
    P /= P.sum(axis=1, keepdims=True)
    assert np.allclose(O[0, 0], P @ V, rtol=1e-12, atol=1e-12)
