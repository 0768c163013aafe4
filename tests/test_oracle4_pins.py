"""Pins of the 4-bit oracle (oracle/isoquant4_oracle.py) against mathematics
it does not share code with: the 3-bit levels the specification of this path
fixes (four digits each; the pages print no codebook), numerical
integration of the Gaussian (scipy), brute force on tiny inputs, and a
hand-worked packing example (tests/golden/pack4_worked_example.txt)."""

import math
import os

import numpy as np
import pytest
from scipy import integrate, stats

from oracle import isoquant4_oracle as O4
from oracle import isoquant_oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "pack4_worked_example.txt")


def test_lloyd_iteration_reproduces_specified_3bit_codebook():
    """The 3-bit Gaussian Lloyd-Max levels of the specification are given to
    four digits: the same iteration with 8 levels must land on them."""
    c8 = O4.lloyd_max_gaussian(8)
    specified = np.array([-2.1520, -1.3440, -0.7560, -0.2451, 0.2451, 0.7560, 1.3440, 2.1520])
    # four significant digits each (2.152, 1.344, 0.7560, 0.2451): half a unit
    # of the fourth digit
    half_ulp = 0.5 * 10.0 ** (np.floor(np.log10(np.abs(specified))) - 3)
    assert np.all(np.abs(c8 - specified) <= half_ulp + 1e-12)
    assert abs(O4.gaussian_mse(c8) - 0.034548) < 5e-7


def test_16_levels_are_a_lloyd_max_fixed_point():
    c = O4.centroids4()
    assert np.all(np.diff(c) > 0)
    assert np.array_equal(c, -c[::-1])
    t = np.concatenate([[-np.inf], (c[:-1] + c[1:]) / 2, [np.inf]])
    pdf = stats.norm.pdf
    for i in range(16):
        num, _ = integrate.quad(lambda x: x * pdf(x), t[i], t[i + 1], epsabs=1e-14, epsrel=1e-13)
        den, _ = integrate.quad(pdf, t[i], t[i + 1], epsabs=1e-14, epsrel=1e-13)
        assert abs(num / den - c[i]) < 1e-10, i
    th = O4.thresholds4_f32()
    assert th[7] == 0.0
    assert np.array_equal(th, -th[::-1])
    assert np.array_equal(th, ((c[:-1] + c[1:]) / 2).astype(np.float32))


def test_mse_closed_form_matches_integration_and_sampling():
    c = O4.centroids4()
    t = np.concatenate([[-np.inf], (c[:-1] + c[1:]) / 2, [np.inf]])
    by_quad = sum(integrate.quad(lambda x, ci=ci: (x - ci) ** 2 * stats.norm.pdf(x), t[i], t[i + 1],
                                 epsabs=1e-14)[0] for i, ci in enumerate(c))
    mse = O4.gaussian_mse(c)
    assert abs(mse - by_quad) < 1e-10
    x = np.random.default_rng(3).standard_normal(2_000_000)
    q = c[np.searchsorted(t[1:-1], x)]
    est = float(np.mean((x - q) ** 2))
    assert abs(est - mse) < 4 * np.std((x - q) ** 2) / math.sqrt(x.size)
    assert mse < O4.gaussian_mse(O4.lloyd_max_gaussian(8)) / 3.5


def test_decision_rule_is_nearest_level_and_symmetric():
    c = O4.centroids4()
    th = O4.thresholds4_f32().astype(np.float64)
    u = np.linspace(-4, 4, 80001)
    u = u[np.min(np.abs(u[:, None] - th[None, :]), axis=1) > 1e-6]
    codes = np.array([int(np.sum(np.float32(v) >= O4.thresholds4_f32())) for v in u])
    assert np.array_equal(codes, np.argmin(np.abs(u[:, None] - c[None, :]), axis=1))
    neg = np.array([int(np.sum(np.float32(-v) >= O4.thresholds4_f32())) for v in u])
    assert np.array_equal(neg, 15 - codes)


def test_quantize4_zero_vector_and_closed_form():
    blocks = O.rotation_matrices(np.tile(np.array([1.0, 0, 0, 0]), (1, 32, 2, 1)))[0]
    out = O4.quantize4(np.zeros((1, 128)), blocks)
    assert np.all(out["codes"] == 8) and out["norm16"][0] == 0
    # with identity blocks T = H / sqrt(d): x = row 0 of H gives T x = sqrt(d) e_0,
    # n = sqrt(d), u = d * e_0 / sqrt(d) ... u_0 = sqrt(128) > every threshold
    x = O.sylvester_hadamard()[0:1]
    q = O4.quantize4(x, blocks)
    assert q["codes"][0, 0] == 15 and np.all(q["codes"][0, 1:] == 8)


def test_nibbles_are_sign_magnitude():
    codes = np.arange(16)
    nib = O4.nibble_of_code(codes)
    assert sorted(nib.tolist()) == list(range(16))
    assert np.array_equal(O4.code_of_nibble(nib), codes)
    c = O4.centroids4()
    for k in range(16):
        sign_neg = nib[k] >= 8
        assert sign_neg == (c[k] < 0)
        mag_index = nib[k] & 7
        assert abs(c[k]) == np.sort(np.abs(c[8:]))[mag_index]


def test_pack4_worked_example_and_round_trip():
    want = np.zeros(64, dtype=np.uint8)
    for line in open(GOLDEN):
        if line.strip() and not line.startswith("#"):
            off, val = line.split()
            want[int(off)] = int(val, 16)
    codes = np.full((1, 128), 8, dtype=np.uint8)
    codes[0, :16] = np.arange(16)
    assert np.array_equal(O4.pack4(codes)[0], want)
    rnd = np.random.default_rng(1).integers(0, 16, size=(50, 128)).astype(np.uint8)
    assert np.array_equal(O4.unpack4(O4.pack4(rnd)), rnd)


def test_v4_positions_are_a_bijection_with_one_token_per_byte():
    off, sh = O4.v4_offsets()
    keys = off * 2 + sh // 4
    assert len(np.unique(keys)) == 64 * 128 and keys.min() == 0 and keys.max() == 8191
    owner = np.full(4096, -1)
    for t in range(64):
        for c in range(128):
            b = off[t, c]
            assert owner[b] in (-1, t)
            owner[b] = t


def _v_block_from_layout(slot_codes):
    """The 4,096-byte V block of a page from the layout statement, walked byte
    by byte (region n + 16 jq, dword 4p + 2 th + q, byte r: token slot 32 th +
    16 q + 4 jq + r; low nibble coordinate 32 (n // 4) + 4p + n % 4, high
    nibble that + 16).  slot_codes: [64][128] codes."""
    nib = O4.nibble_of_code(slot_codes)
    blk = np.zeros(4096, dtype=np.uint8)
    for jq in range(4):
        for n in range(16):
            for p in range(4):
                for th in range(2):
                    for q in range(2):
                        for r in range(4):
                            t = 32 * th + 16 * q + 4 * jq + r
                            c = 32 * (n // 4) + 4 * p + n % 4
                            blk[(n + 16 * jq) * 64 + 4 * (4 * p + 2 * th + q) + r] = \
                                nib[t, c] | (nib[t, c + 16] << 4)
    return blk


def test_v4_store_matches_layout_and_round_trips():
    """Every byte carries two codes of one token: storing tokens one at a
    time, in any order, must leave both nibbles (the block equals the
    byte-by-byte construction) and read back the codes."""
    rng = np.random.default_rng(5)
    codes = rng.integers(0, 16, size=(64, 128)).astype(np.uint8)
    cache = O4.PagedCache4(2, 1)
    order = rng.permutation(64)
    for t in order:                                  # one token per call
        cache.store("v", np.array([1]), 0, np.array([t]), codes[t:t + 1])
    assert np.array_equal(cache.v_codes[1, 0].reshape(-1), _v_block_from_layout(codes))
    assert np.array_equal(cache.codes("v", np.full(64, 1), 0, np.arange(64)), codes)
    assert not cache.v_codes[0].any()
    # overwriting a slot changes only that token's nibbles
    new = rng.integers(0, 16, size=(1, 128)).astype(np.uint8)
    cache.store("v", np.array([1]), 0, np.array([37]), new)
    codes[37] = new[0]
    assert np.array_equal(cache.v_codes[1, 0].reshape(-1), _v_block_from_layout(codes))


def test_decode4_equals_plain_attention_on_materialised_kv():
    rng = np.random.default_rng(7)
    hkv, hq, lens = 2, 4, [1, 70, 130]
    quats = rng.standard_normal((hkv, 32, 2, 4))
    blocks = O.rotation_matrices(quats)
    pages = [-(-n // 64) for n in lens]
    bt = np.zeros((3, max(pages)), dtype=np.int64)
    nxt = 0
    for b, p in enumerate(pages):
        bt[b, :p] = np.arange(nxt, nxt + p)
        nxt += p
    cache = O4.PagedCache4(nxt, hkv)
    k = rng.standard_normal((sum(lens), hkv, 128))
    v = rng.standard_normal((sum(lens), hkv, 128))
    seq = np.concatenate([np.full(n, b) for b, n in enumerate(lens)])
    pos = np.concatenate([np.arange(n) for n in lens])
    O4.quantize_append4(cache, blocks, k, v, seq, pos, bt)
    q = rng.standard_normal((3, hq, 128))
    out = O4.decode_attention4(cache, blocks, q, bt, lens)
    for b, n in enumerate(lens):
        for g in range(hkv):
            kc, kn = cache.gather(bt, b, n, g, "k")
            vc, vn = cache.gather(bt, b, n, g, "v")
            kk = O.inverse_rotate(O4.dequantize_rotated4(kc, kn), blocks[g])
            vv = O.inverse_rotate(O4.dequantize_rotated4(vc, vn), blocks[g])
            ref = O.reference_attention(q[b, 2 * g:2 * g + 2], kk, vv)
            assert np.max(np.abs(out[b, 2 * g:2 * g + 2] - ref)) < 1e-12
    # context 1: the output is the dequantised value
    vc, vn = cache.gather(bt, 0, 1, 0, "v")
    assert np.allclose(out[0, 0], O.inverse_rotate(O4.dequantize_rotated4(vc, vn), blocks[0])[0], atol=1e-12)
    # the stored records hold the quantiser's codes
    kc, _ = cache.gather(bt, 2, 130, 1, "k")
    assert np.array_equal(kc, O4.quantize4(k[sum(lens[:2]):, 1], blocks[1])["codes"])
    vc, _ = cache.gather(bt, 2, 130, 1, "v")
    assert np.array_equal(vc, O4.quantize4(v[sum(lens[:2]):, 1], blocks[1])["codes"])


def test_prefill4_rows_equal_causal_plain_attention():
    """Each query row equals plain softmax attention of the unrotated query
    over the dequantised keys and values up to its own position."""
    rng = np.random.default_rng(9)
    hkv, hq, n_ctx, q_start = 2, 8, 150, 100
    quats = rng.standard_normal((hkv, 32, 2, 4))
    blocks = O.rotation_matrices(quats)
    bt = rng.permutation(4).reshape(1, 4)
    cache = O4.PagedCache4(4, hkv)
    k = rng.standard_normal((n_ctx, hkv, 128))
    v = rng.standard_normal((n_ctx, hkv, 128))
    O4.quantize_append4(cache, blocks, k, v, np.zeros(n_ctx, int), np.arange(n_ctx), bt)
    q = rng.standard_normal((n_ctx - q_start, hq, 128))
    out = O4.prefill_attention4(cache, blocks, q, q_start, bt[0])
    for g in range(hkv):
        kc, kn = cache.gather(bt, 0, n_ctx, g, "k")
        vc, vn = cache.gather(bt, 0, n_ctx, g, "v")
        kk = O.inverse_rotate(O4.dequantize_rotated4(kc, kn), blocks[g])
        vv = O.inverse_rotate(O4.dequantize_rotated4(vc, vn), blocks[g])
        for i in (0, 7, 49):
            for h in range(g * 4, g * 4 + 4):
                ref = O.reference_attention(q[i, h:h + 1], kk[:q_start + i + 1], vv[:q_start + i + 1])
                assert np.max(np.abs(out[i, h] - ref[0])) < 1e-12
    # the first query sees exactly q_start + 1 keys: a later key does not move it
    k2 = k.copy()
    k2[q_start + 1:] *= -3.0
    cache2 = O4.PagedCache4(4, hkv)
    O4.quantize_append4(cache2, blocks, k2, v, np.zeros(n_ctx, int), np.arange(n_ctx), bt)
    out2 = O4.prefill_attention4(cache2, blocks, q[:1], q_start, bt[0])
    assert np.array_equal(out2[0], out[0])
