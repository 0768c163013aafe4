"""Pins of the FP8 (E4M3) oracle (oracle/fp8_oracle.py) against torch's own
float8_e4m3fn conversions (an independent implementation of the OCP format),
the format's defining values, and plain attention."""

import numpy as np
import torch

from oracle import fp8_oracle as F
from oracle import isoquant_oracle as O


def test_decode_table_matches_torch():
    b = np.arange(256, dtype=np.uint8)
    ours = F.e4m3_decode(b)
    theirs = torch.from_numpy(b).view(torch.float8_e4m3fn).double().numpy()
    assert np.array_equal(np.isnan(ours), np.isnan(theirs))
    ok = ~np.isnan(ours)
    assert np.array_equal(ours[ok], theirs[ok])
    assert np.sum(np.isnan(ours)) == 2                       # S.1111.111 only


def test_defining_values():
    assert F.e4m3_decode(0x7E) == 448.0                       # largest finite
    assert F.e4m3_decode(0x01) == 2.0 ** -9                   # smallest subnormal
    assert F.e4m3_decode(0x08) == 2.0 ** -6                   # smallest normal
    assert F.e4m3_decode(0x38) == 1.0 and F.e4m3_decode(0xB8) == -1.0
    # ties go to the even mantissa: 1 + 1/16 -> 1, 1 + 3/16 -> 1.25
    assert F.e4m3_encode(1.0625) == 0x38 and F.e4m3_encode(1.1875) == 0x3A
    # saturation (the cache never holds NaN)
    assert F.e4m3_encode(1000.0) == 0x7E and F.e4m3_encode(-1e9) == 0xFE
    assert F.e4m3_encode(0.0) == 0x00 and F.e4m3_encode(-0.0) == 0x80


def test_encode_matches_torch_on_float32_inputs():
    rng = np.random.default_rng(2)
    x = np.concatenate([rng.standard_normal(200_000) * 4.0,
                        rng.standard_normal(50_000) * 1e-2,          # subnormal range
                        rng.uniform(-448, 448, 50_000),
                        F.e4m3_decode(np.arange(256))[np.isfinite(F.e4m3_decode(np.arange(256)))],
                        # every midpoint between adjacent positive values (exact ties)
                        ]).astype(np.float32)
    vals = np.unique(F.e4m3_decode(np.arange(0, 0x7F)))
    mids = ((vals[:-1] + vals[1:]) / 2).astype(np.float32)
    x = np.concatenate([x, mids, -mids])
    ours = F.e4m3_encode(x.astype(np.float64))
    theirs = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(ours, theirs)


def test_round_trip_and_nearest():
    b = np.arange(256)
    v = F.e4m3_decode(b)
    fin = np.isfinite(v)
    assert np.array_equal(F.e4m3_decode(F.e4m3_encode(v[fin])), v[fin])
    # the encoding is a nearest representable value
    x = np.random.default_rng(3).uniform(-448, 448, 20_000)
    got = F.e4m3_decode(F.e4m3_encode(x))
    grid = np.unique(v[fin])
    best = np.min(np.abs(x[:, None] - grid[None, :]), axis=1)
    assert np.allclose(np.abs(got - x), best, rtol=0, atol=0)


def test_scaled_rows_and_attention():
    rng = np.random.default_rng(4)
    k = rng.standard_normal((100, 2, 128)) * 30.0
    v = rng.standard_normal((100, 2, 128))
    q = rng.standard_normal((2, 4, 128))
    # a scale of 2 halves every stored magnitude (before rounding)
    b1 = F.quantize_rows(k, 2.0)
    assert np.array_equal(b1, F.e4m3_encode((k.astype(np.float32) * np.float32(0.5)).astype(np.float64)))
    starts = np.array([0, 37, 100])
    out = F.decode_attention_fp8(k, v, q, starts, 2, k_scale=2.0, v_scale=0.5)
    kq = F.e4m3_decode(F.quantize_rows(k, 2.0)) * 2.0
    vq = F.e4m3_decode(F.quantize_rows(v, 0.5)) * 0.5
    ref = O.reference_attention(q[1, 2:4], kq[37:100, 1], vq[37:100, 1])
    assert np.max(np.abs(out[1, 2:4] - ref)) < 1e-12
    # fp8 rounding of N(0,1) values keeps attention within a few percent
    plain = O.reference_attention(q[0, 0:2], k[:37, 0], v[:37, 0])
    assert np.max(np.abs(out[0, 0:2] - plain)) < 0.1 * np.max(np.abs(plain))
