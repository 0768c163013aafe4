"""Pins of the CPU oracle against what the pages and mathematics fix.

Each test checks the oracle against something other than itself: a textbook
or library special case (scipy's Sylvester Hadamard and 3-D rotations), a
closed form, an invariant, or brute force on tiny inputs.  Sources:
"RotaryQuant: Fitting 120B MoE Models on Consumer Hardware via Fused
Compressed-Space Attention", abstract (WHT then block-diagonal SO(4), 3-bit
scalar quantisation, 256 parameters per head, attention on packed tensors);
FreeToken issue #141, Proposed Solution (quaternion rotations, GQA).
"""

import math
import os

import numpy as np
import pytest
import scipy.linalg
import scipy.stats
from scipy.spatial.transform import Rotation

from oracle import isoquant_oracle as O
from compressed_space_attention_amd import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def random_blocks(seed, hkv=1):
    return O.rotation_matrices(synth.quaternions(seed, hkv))


# ---------------------------------------------------------------- Hadamard --
def test_hadamard_is_sylvester_and_orthogonal():
    h = O.sylvester_hadamard()
    assert np.array_equal(h @ h.T, 128.0 * np.eye(128))
    assert np.array_equal(h, h.T)
    # textbook Sylvester construction (scipy builds it by Kronecker doubling)
    assert np.array_equal(h, scipy.linalg.hadamard(128).astype(np.float64))


def test_identity_quaternions_give_normalised_hadamard():
    blocks = O.rotation_matrices(synth.identity_quaternions(1))[0]
    assert np.allclose(blocks, np.eye(4)[None], atol=0, rtol=0)
    t = O.dense_rotation(blocks)
    assert np.allclose(t, scipy.linalg.hadamard(128) / math.sqrt(128), atol=1e-15)


# ------------------------------------------------------------------- SO(4) --
def test_blocks_are_special_orthogonal():
    for blocks in random_blocks(7, hkv=4):
        for m in blocks:
            assert np.max(np.abs(m.T @ m - np.eye(4))) < 1e-12
            assert abs(np.linalg.det(m) - 1.0) < 1e-12


def test_double_cover_and_normalisation():
    g = np.random.default_rng(3)
    for _ in range(20):
        ql, qr = g.standard_normal(4), g.standard_normal(4)
        m = O.so4_block(ql, qr)
        assert np.allclose(O.so4_block(-ql, -qr), m, atol=1e-14)
        assert np.allclose(O.so4_block(3.5 * ql, 0.25 * qr), m, atol=1e-14)


def _left_matrix(a):
    """Textbook matrix of v -> a v (quaternion left multiplication)."""
    w, x, y, z = a
    return np.array([[w, -x, -y, -z], [x, w, -z, y], [y, z, w, -x], [z, -y, x, w]])


def _right_matrix(r):
    """Textbook matrix of v -> v r (quaternion right multiplication)."""
    w, x, y, z = r
    return np.array([[w, -x, -y, -z], [x, w, z, -y], [y, -z, w, x], [z, y, -x, w]])


def test_block_equals_left_times_right_isoclinic_closed_form():
    g = np.random.default_rng(5)
    for _ in range(20):
        ql, qr = g.standard_normal(4), g.standard_normal(4)
        a = ql / np.linalg.norm(ql)
        p = qr / np.linalg.norm(qr)
        pbar = np.array([p[0], -p[1], -p[2], -p[3]])
        want = _left_matrix(a) @ _right_matrix(pbar)
        assert np.max(np.abs(O.so4_block(ql, qr) - want)) < 1e-14


def test_conjugation_matches_scipy_3d_rotation():
    """With q_L = q_R = q the block is v -> q v q*, which fixes the real part
    and rotates (v1, v2, v3) by the 3-D rotation of q (scipy: scalar-last)."""
    g = np.random.default_rng(11)
    for _ in range(20):
        q = g.standard_normal(4)
        q /= np.linalg.norm(q)
        m = O.so4_block(q, q)
        r = Rotation.from_quat([q[1], q[2], q[3], q[0]]).as_matrix()
        assert abs(m[0, 0] - 1.0) < 1e-14
        assert np.max(np.abs(m[0, 1:])) < 1e-14 and np.max(np.abs(m[1:, 0])) < 1e-14
        assert np.max(np.abs(m[1:, 1:] - r)) < 1e-13


def test_parameter_count_and_rate():
    assert O.PARAMS_PER_HEAD == 256 and synth.quaternions(0, 1)[0].size == 256
    assert O.DENSE_PARAMS_PER_HEAD == 16384
    bits = (O.CODE_BYTES + O.NORM_BYTES) * 8 / O.HEAD_DIM
    assert bits == 3.125
    assert (2 * O.HEAD_DIM) / (O.CODE_BYTES + O.NORM_BYTES) == 5.12


# --------------------------------------------------------------- transform --
def test_round_trip_dot_products_and_dense_equivalence():
    blocks = random_blocks(21)[0]
    x = np.random.default_rng(1).standard_normal((64, 128))
    y = np.random.default_rng(2).standard_normal((64, 128))
    tx = O.forward_rotate(x, blocks)
    assert np.max(np.abs(O.inverse_rotate(tx, blocks) - x)) <= 1e-12
    ty = O.forward_rotate(y, blocks)
    assert np.allclose(np.sum(tx * ty, 1), np.sum(x * y, 1), rtol=1e-12, atol=1e-12)
    t = O.dense_rotation(blocks)
    assert np.max(np.abs(x @ t.T - tx)) < 1e-13
    assert np.max(np.abs(t @ t.T - np.eye(128))) < 1e-13


def _quats_block0(ql, qr):
    q = synth.identity_quaternions(1).astype(np.float64)
    q[0, 0, 0] = ql
    q[0, 0, 1] = qr
    return O.rotation_matrices(q)[0]


@pytest.mark.parametrize("side", ["left", "right"])
def test_quantiser_closed_form_orientation(side):
    """x = all-ones has H x / sqrt(d) = sqrt(d) e_0, so u = sqrt(d) * (block 0
    applied to e_0).  A left rotation by e^{i th} sends e_0 to (cos, sin, 0, 0);
    a right factor conj(e^{i th}) sends it to (cos, -sin, 0, 0).  With
    sin(th) = 0.05, u_1 = +-0.5657: code 5 or code 2 — the sign pins the
    orientation of the blocks and the conjugation of q_R."""
    th = math.asin(0.05)
    rot = np.array([math.cos(th), math.sin(th), 0.0, 0.0])
    one = np.array([1.0, 0, 0, 0])
    blocks = _quats_block0(rot, one) if side == "left" else _quats_block0(one, rot)
    # 0.5 is a power of two, so the Hadamard sums cancel exactly to 0
    q = O.quantize(np.full((1, 128), 0.5), blocks)
    codes = q["codes"][0]
    assert codes[0] == 7                          # u_0 = sqrt(128) cos th = 11.30
    assert codes[1] == (5 if side == "left" else 2)
    assert np.all(codes[2:] == 4)                 # u = 0 -> code 4 (ties go up)
    assert q["near"][0, 2:].all()                 # exactly on the 0 boundary
    assert q["norm16"][0] == np.float16(0.5 * math.sqrt(128)).view(np.uint16)


def test_quantiser_hadamard_column_and_basis_vector():
    blocks = O.rotation_matrices(synth.identity_quaternions(1))[0]
    h = scipy.linalg.hadamard(128).astype(np.float64)
    # x = column k of H: H x = 128 e_k, so u_k = sqrt(128) (code 7), others 0 (code 4)
    q = O.quantize(h[:, 37][None] * 0.25, blocks)   # power of two: exact sums
    want = np.full(128, 4)
    want[37] = 7
    assert np.array_equal(q["codes"][0], want)
    # x = e_0: H e_0 = all ones, u_i = 1 for every i -> code 5 (1.0 in [0.50055, 1.05))
    e0 = np.zeros((1, 128))
    e0[0, 0] = 3.0
    assert np.all(O.quantize(e0, blocks)["codes"] == 5)
    # -e_0 -> u = -1 -> code 2
    assert np.all(O.quantize(-e0, blocks)["codes"] == 2)


def test_zero_vector_and_scale_invariance_and_norm_saturation():
    blocks = random_blocks(4)[0]
    z = O.quantize(np.zeros((1, 128)), blocks)
    assert np.all(z["codes"] == 4) and z["norm16"][0] == 0
    x = np.random.default_rng(9).standard_normal((16, 128))
    a = O.quantize(x, blocks)
    b = O.quantize(x * 8.0, blocks)             # power of two: exact scaling
    assert np.array_equal(a["codes"], b["codes"])
    bits = O.fp16_bits_saturating(np.array([1.0, 65504.0, 65519.0, 65520.0, 1e6, 0.0]))
    assert list(bits) == [0x3C00, 0x7BFF, 0x7BFF, 0x7BFF, 0x7BFF, 0x0000]
    # 2049 is the midpoint between fp16 values 2048 and 2050: RNE -> 2048
    assert O.fp16_bits_saturating(np.array([2049.0]))[0] == np.float16(2048).view(np.uint16)
    assert O.fp16_midpoint_near(np.array([2049.0, 2048.0]))[0]
    assert not O.fp16_midpoint_near(np.array([2049.0, 2048.0]))[1]


# ---------------------------------------------------------------- codebook --
def test_centroids_are_gaussian_lloyd_max():
    c = O.CENTROIDS
    edges = np.concatenate([[-np.inf], (c[:-1] + c[1:]) / 2, [np.inf]])
    lo, hi = edges[:-1], edges[1:]
    mass = scipy.stats.norm.cdf(hi) - scipy.stats.norm.cdf(lo)
    cond_mean = (scipy.stats.norm.pdf(lo) - scipy.stats.norm.pdf(hi)) / mass
    assert np.max(np.abs(cond_mean - c)) < 4e-5
    # closed-form MSE of the quantiser on N(0,1): E[X^2] - sum mass*c^2 at the optimum
    mse = 1.0 - np.sum(mass * cond_mean ** 2)
    assert abs(mse - 0.034548) < 2e-5
    assert np.allclose(c, -c[::-1])


def test_threshold_rule_is_nearest_centroid():
    u = np.linspace(-4, 4, 200001)
    uf = u.astype(np.float32)
    by_threshold = np.sum(uf[:, None] >= O.THRESHOLDS_F32[None, :], axis=1)
    nearest = np.argmin(np.abs(u[:, None] - O.CENTROIDS[None, :]), axis=1)
    mid = np.min(np.abs(u[:, None] - O.THRESHOLDS_F32.astype(np.float64)[None]), axis=1) < 1e-6
    assert np.array_equal(by_threshold[~mid], nearest[~mid])
    neg = np.sum((-uf)[:, None] >= O.THRESHOLDS_F32[None, :], axis=1)
    assert np.array_equal(neg[~mid], 7 - by_threshold[~mid])


def test_distortion_sanity_on_gaussian_vectors():
    blocks = random_blocks(8)[0]
    x = np.random.default_rng(12).standard_normal((4000, 128))
    q = O.quantize(x, blocks)
    xh = O.dequantize(q["codes"], q["norm16"], blocks)
    rel = np.sum((x - xh) ** 2, 1) / np.sum(x * x, 1)
    assert 0.030 < rel.mean() < 0.036


# ----------------------------------------------------------------- packing --
def _golden_pack_cases():
    cases = []
    with open(os.path.join(GOLDEN, "pack_worked_example.txt")) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            name, codes, bytes_ = (p.strip() for p in line.split(";"))
            c = np.zeros(128, dtype=np.uint8)
            for kv in codes.split():
                k, v = kv.split("=")
                c[int(k)] = int(v)
            b = np.zeros(48, dtype=np.uint8)
            for kv in bytes_.split():
                k, v = kv.split("=")
                b[int(k)] = int(v, 16)
            cases.append((name, c, b))
    return cases


@pytest.mark.parametrize("name,codes,want", _golden_pack_cases())
def test_pack_worked_examples(name, codes, want):
    got = O.pack_codes(codes[None])[0]
    assert np.array_equal(got, want), name
    assert np.array_equal(O.unpack_codes(want[None])[0], codes)


def test_pack_round_trip_and_saturation():
    c = np.random.default_rng(0).integers(0, 8, size=(300, 128)).astype(np.uint8)
    assert np.array_equal(O.unpack_codes(O.pack_codes(c)), c)
    assert np.all(O.pack_codes(np.full((1, 128), 7, np.uint8)) == 0xFF)


def test_v_block_permutation():
    """V blocks are a fixed byte permutation of the 64 records (reading R9b).
    Hand-derived offsets: slot 5 (chunk 0, quad 1, lane 1), record byte 0
    (group 0, dword 0, byte lane 0 -> region 0 + 16) -> 16*48 + 1 = 769;
    slot 63, byte 47 (group 3, dword 2, byte lane 3 -> region 15 + 48) ->
    63*48 + 12*3 + 8 + 3 = 3071; slot 16 (chunk 1), byte 13 (group 1, dword 0,
    byte lane 1 -> region 5) -> 5*48 + 12 = 252."""
    off = O.v_block_offsets()
    assert sorted(off.ravel().tolist()) == list(range(3072))
    assert off[5, 0] == 769 and off[63, 47] == 3071 and off[16, 13] == 252 and off[0, 0] == 0
    c = O.PagedCache(3, 2)
    recs = np.random.default_rng(4).integers(0, 256, (70, 48), dtype=np.uint8)
    page = np.array([1] * 64 + [2] * 6)
    slot = np.concatenate([np.arange(64), np.arange(6)])
    c.store("v", page, 1, slot, recs)
    assert np.array_equal(c.records("v", page, 1, slot), recs)
    assert np.all(c.v_codes[0] == 0) and np.all(c.v_codes[:, 0] == 0)
    # region (n=6, q=2) chunk 1 byte lane 3 holds slot 16+8+3=27's byte lane 2 of group 1
    blk = c.v_codes[1, 1].reshape(3072)
    region = blk[(6 + 32) * 48:(6 + 32) * 48 + 48]
    for i in range(3):
        assert region[12 * 1 + 4 * i + 3] == recs[27, 12 * 1 + 4 * i + 2]


# --------------------------------------------------------------- attention --
def _small_cache(seed, lens, hkv, pages_extra=3):
    pages = [-(-int(n) // 64) for n in lens]
    bt, total = synth.block_table(seed, pages, shuffle=True, extra_pages=pages_extra)
    cache = O.PagedCache(total, hkv)
    blocks = random_blocks(seed + 1, hkv)
    for b, n in enumerate(lens):
        k = synth.normal(seed + 10 + b, (n, hkv, 128)).astype(np.float64)
        v = synth.normal(seed + 20 + b, (n, hkv, 128)).astype(np.float64)
        O.quantize_append(cache, blocks, k, v, np.full(n, b), np.arange(n), bt)
    return cache, blocks, bt


def test_decode_equals_plain_attention_on_materialised_kv():
    """Brute force: dequantise every key and value back to the original
    space (T^T), run plain softmax attention with the unrotated query."""
    lens = [1, 150, 300]
    hkv, hq = 2, 6
    cache, blocks, bt = _small_cache(40, lens, hkv)
    q = np.random.default_rng(41).standard_normal((len(lens), hq, 128))
    got = O.decode_attention(cache, blocks, q, bt, lens)
    for b, n in enumerate(lens):
        for h in range(hq):
            g = h // (hq // hkv)
            kc, kn = cache.gather(bt, b, n, g, "k")
            vc, vn = cache.gather(bt, b, n, g, "v")
            kf = O.dequantize(kc, kn, blocks[g])
            vf = O.dequantize(vc, vn, blocks[g])
            s = (kf @ q[b, h]) / math.sqrt(128)
            p = np.exp(s - s.max())
            want = p @ vf / p.sum()
            assert np.max(np.abs(got[b, h] - want)) <= 1e-12 * max(1.0, np.max(np.abs(want)))


def test_decode_special_cases():
    hkv, hq = 1, 4
    cache, blocks, bt = _small_cache(50, [1, 97], hkv)
    q = np.random.default_rng(51).standard_normal((2, hq, 128))
    out = O.decode_attention(cache, blocks, q, bt, [1, 97])
    # context 1: the output is the dequantised value of token 0
    vc, vn = cache.gather(bt, 0, 1, 0, "v")
    v0 = O.dequantize(vc, vn, blocks[0])[0]
    assert np.allclose(out[0], v0[None], atol=1e-12)
    # empty context: zeros, never NaN
    assert np.all(O.decode_attention(cache, blocks, q, bt, [0, 0]) == 0)
    # identical queries in a group give identical outputs
    qq = np.repeat(q[:, :1], hq, axis=1)
    o2 = O.decode_attention(cache, blocks, qq, bt, [1, 97])
    assert np.allclose(o2, o2[:, :1], atol=0)


def test_equal_keys_give_mean_of_values():
    n, hkv = 70, 1
    bt, total = synth.block_table(0, [2], shuffle=False)
    cache = O.PagedCache(total, hkv)
    blocks = random_blocks(60, hkv)
    k = np.repeat(np.random.default_rng(1).standard_normal((1, 1, 128)), n, axis=0)
    v = np.random.default_rng(2).standard_normal((n, 1, 128))
    O.quantize_append(cache, blocks, k, v, np.zeros(n, int), np.arange(n), bt)
    q = np.random.default_rng(3).standard_normal((1, 1, 128))
    out = O.decode_attention(cache, blocks, q, bt, [n])
    vc, vn = cache.gather(bt, 0, n, 0, "v")
    assert np.allclose(out[0, 0], O.dequantize(vc, vn, blocks[0]).mean(0), atol=1e-12)


def test_prefill_rows_equal_causal_plain_attention():
    n, hkv, hq = 200, 2, 4
    cache, blocks, bt = _small_cache(70, [n], hkv)
    n_q, q_start = 9, n - 9
    q = np.random.default_rng(71).standard_normal((n_q, hq, 128))
    got = O.prefill_attention(cache, blocks, q, q_start, bt[0])
    dec = np.stack([O.decode_attention(cache, blocks, q[i:i + 1], bt, [q_start + i + 1])[0]
                    for i in range(n_q)])
    assert np.max(np.abs(got - dec)) < 1e-12
    for g in range(hkv):
        kc, kn = cache.gather(bt, 0, n, g, "k")
        vc, vn = cache.gather(bt, 0, n, g, "v")
        kf, vf = O.dequantize(kc, kn, blocks[g]), O.dequantize(vc, vn, blocks[g])
        for h in range(g * 2, g * 2 + 2):
            want = O.reference_attention(q[:, h], kf, vf, visible=q_start + np.arange(n_q) + 1)
            assert np.max(np.abs(got[:, h] - want)) < 1e-12


def test_row_error_metric():
    ref = np.array([[1.0, -2.0, 0.0]])
    assert O.row_relative_error(ref + np.array([[0.0, 0.002, 0.0]]), ref)[0] == pytest.approx(1e-3)
    assert O.row_cosine(ref, 2 * ref)[0] == pytest.approx(1.0)
