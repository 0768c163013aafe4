"""Plain CPU oracle of the FP8 (e4m3) paged-cache baseline (TEST INFRASTRUCTURE).

Only the test suite may import this module.  It shares no code, tables or
constants with the GPU library.

The pages list FP8 KV as a fallback format of the engine ("FreeToken" issue
#141, Proposed Solution: FP8 / int4 KV fallback) without fixing its encoding;
the reading here is the OCP 8-bit floating point format E4M3 ("fn": no
infinities), the usual FP8 KV-cache format:

* 1 sign bit, 4 exponent bits with bias 7, 3 mantissa bits;
* exponent field 1..15: value 2^(e - 7) (1 + m / 8); exponent field 0:
  subnormal m 2^-9; S.1111.111 is NaN, so the largest finite value is
  0x7E = 1.75 * 2^8 = 448;
* encoding a real: round to the nearest representable value, ties to the
  even mantissa, saturating at +-448 (the cache never holds NaN).

A cache stores byte = e4m3(float32(x) * float32(1 / scale)) with one scale per
tensor (K or V) and cache, and reads back e4m3 * scale.
"""

from __future__ import annotations

import numpy as np

from oracle import isoquant_oracle as O

E4M3_MAX = 448.0


def e4m3_decode(b) -> np.ndarray:
    """Byte(s) -> float64 value (NaN for S.1111.111)."""
    b = np.asarray(b, dtype=np.int64)
    s = np.where(b & 0x80, -1.0, 1.0)
    e = (b >> 3) & 15
    m = b & 7
    val = np.where(e == 0, m * 2.0 ** -9, (1.0 + m / 8.0) * np.exp2(e - 7.0))
    val = np.where((e == 15) & (m == 7), np.nan, val)
    return s * val


def e4m3_encode(x) -> np.ndarray:
    """float(s) -> byte(s): nearest e4m3 value, ties to even, saturating."""
    x = np.asarray(x, dtype=np.float64)
    sign = np.where(np.signbit(x), 0x80, 0).astype(np.int64)
    a = np.minimum(np.abs(x), E4M3_MAX)
    # spacing of the representable values around a: 2^-9 below 2^-6, else
    # 2^(floor(log2 a) - 3)
    with np.errstate(divide="ignore"):
        ex = np.floor(np.log2(np.where(a > 0, a, 1.0)))
    ex = np.maximum(ex, -6.0)
    q = np.exp2(ex - 3.0)
    n = a / q                              # exact: q is a power of two
    r = np.floor(n)
    frac = n - r
    up = (frac > 0.5) | ((frac == 0.5) & (r % 2 == 1))
    r = r + up                             # r in 0..16 (16: the next binade)
    val = r * q
    val = np.minimum(val, E4M3_MAX)
    # bits of val
    e_field = np.where(val >= 2.0 ** -6, np.floor(np.log2(np.where(val > 0, val, 1.0))) + 7, 0)
    e_field = e_field.astype(np.int64)
    m_field = np.where(e_field == 0, np.round(val / 2.0 ** -9),
                       np.round((val / np.exp2(e_field - 7.0) - 1.0) * 8.0)).astype(np.int64)
    return (sign | (e_field << 3) | m_field).astype(np.uint8)


def quantize_rows(x, scale: float) -> np.ndarray:
    """Bytes of float32(x) * float32(1 / scale)."""
    inv = np.float32(1.0) / np.float32(scale)
    y = np.asarray(x, dtype=np.float32) * inv
    return e4m3_encode(y.astype(np.float64))


def dequantize_rows(b, scale: float) -> np.ndarray:
    return e4m3_decode(b) * float(np.float32(scale))


def decode_attention_fp8(k, v, q, starts, hkv, k_scale=1.0, v_scale=1.0, scale=None):
    """Plain fp64 attention over the e4m3-rounded rows: k, v [n_tok][Hkv][128]
    (the appended inputs, token t of sequence b at row starts[b] + t), q
    [B][Hq][128].  Returns [B][Hq][128]."""
    kq = dequantize_rows(quantize_rows(k, k_scale), k_scale)
    vq = dequantize_rows(quantize_rows(v, v_scale), v_scale)
    q = np.asarray(q, dtype=np.float64)
    bsz, hq, _ = q.shape
    grp = hq // hkv
    out = np.zeros((bsz, hq, O.HEAD_DIM))
    for b in range(bsz):
        s, e = starts[b], starts[b + 1]
        if e == s:
            continue
        for g in range(hkv):
            out[b, g * grp:(g + 1) * grp] = O.reference_attention(q[b, g * grp:(g + 1) * grp],
                                                                  kq[s:e, g], vq[s:e, g], scale)
    return out
