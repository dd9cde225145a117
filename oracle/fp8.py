"""Attention on FP8 (E4M3) inputs -- test infrastructure only.

The pages state that FlashAttention-3 supports 8-bit floating point natively,
halving the memory traffic of bf16 (datacamp "Penjelasan Flash Attention",
Flash Attention 3, "Presisi FP8 native"), and give no format, scaling or
rounding rule.  The reading used here and by the kernel:

  * Q, K and V are stored as OCP E4M3 codes (Open Compute Project, "OCP 8-bit
    Floating Point Specification (OFP8)", 2023): 1 sign bit, 4 exponent bits
    with bias 7, 3 mantissa bits; exponent field 0 encodes subnormals
    (mantissa / 8 * 2^-6); S.1111.111 is NaN; there are no infinities and the
    largest finite magnitude is 448;
  * each tensor carries one float32 descale factor: the real value of a code
    c is decode(c) * descale;
  * the result is exact attention (the definition in ``attention``) of the
    real values: O = softmax(scale (dq Q8)(dk K8)^T) (dv V8), lse likewise.

Everything here is float64, and nothing is rounded: what the FP8 path
computes approximately (its probabilities pass through E4M3 on the matrix
cores) is compared against this exact result with a bound derived from the
E4M3 rounding (see the tests).
"""
from __future__ import annotations

import numpy as np

from . import attention


def decode_e4m3(codes):
    """float64 values of OCP E4M3 codes (uint8 array); NaN codes give NaN."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = c & 0x7
    normal = sign * (1.0 + m / 8.0) * np.exp2(e - 7.0)
    subnormal = sign * (m / 8.0) * 2.0 ** -6
    v = np.where(e == 0, subnormal, normal)
    return np.where((c & 0x7F) == 0x7F, np.nan, v)


def dequantize(codes, descale):
    return decode_e4m3(codes) * float(descale)


def forward(q8, k8, v8, q_descale, k_descale, v_descale, scale, causal=False, block_mask=None, kv_len=None):
    """O [B,H,N,d] and lse [B,H,N] (float64) of exact attention on the real
    values of the E4M3 inputs."""
    return attention.forward(dequantize(q8, q_descale), dequantize(k8, k_descale), dequantize(v8, v_descale), scale,
                             causal=causal, block_mask=block_mask, kv_len=kv_len)
