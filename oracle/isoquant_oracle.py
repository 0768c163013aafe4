"""Plain CPU oracle for IsoQuant compressed-space attention (TEST INFRASTRUCTURE).

This module is the slow, obviously-correct reference that the HIP kernels are
checked against.  Only the test suite, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import it.  It shares no code, tables
or constants with the GPU library (``compressed_space_attention_amd``): every
constant below is derived here from its definition.

Arithmetic: float64 for the transform and for attention; float32 for the
quantiser's threshold decisions (both sides decide in fp32); IEEE fp16
round-to-nearest-even for the stored norm.

Sources (cited by page title and section):

* [RQ] "RotaryQuant: Fitting 120B MoE Models on Consumer Hardware via Fused
  Compressed-Space Attention", abstract.  IsoQuant applies a Walsh-Hadamard
  transform, then block-diagonal SO(4) rotations, then 3-bit scalar
  quantisation; it stores 256 parameters per head (versus 16,384 for a dense
  d x d rotation) and attention runs on the packed 3-bit tensors directly.
* [FT141] FreeToken issue #141 ("unified KV cache backend"), Proposed
  Solution: the RotorQuant family (IsoQuant/PlanarQuant) uses quaternion
  rotations at 3 bits; GQA/MQA is listed as an architectural KV reduction.
* [FTREL] FreeToken v0.2.0 release notes, Kernels section: decode attention
  split by context length (#729); softmax chunks that start at -inf must not
  produce NaN (#654).

Where the pages leave a step open, the reading taken is stated at the
function that implements it (readings R1-R18 of the design notes).

Parity pins: every function here is pinned by a ``-m "not gpu"`` test against
mathematics the pages fix (closed forms, library special cases, brute force).
None is "parity unpinned" except the items the pages themselves never define
(RotaryQuant's own codebook, packing and quaternion convention), for which the
readings below are used and stated.
"""

from __future__ import annotations

import math
from functools import lru_cache

import numpy as np

# ----------------------------------------------------------------------------
# Fixed sizes.  d = 128 per head: 32 SO(4) blocks x 2 quaternions x 4 = 256
# stored parameters per head, the count [RQ] gives.
# ----------------------------------------------------------------------------
HEAD_DIM = 128
N_BLOCKS = HEAD_DIM // 4            # 32 blocks of 4 coordinates (R2)
PAGE_TOKENS = 64                    # tokens per cache page (R9)
CODE_BYTES = HEAD_DIM * 3 // 8      # 48 bytes of 3-bit codes per vector
NORM_BYTES = 2                      # fp16 norm per vector
PARAMS_PER_HEAD = N_BLOCKS * 2 * 4  # 256, [RQ]
DENSE_PARAMS_PER_HEAD = HEAD_DIM * HEAD_DIM  # 16,384, [RQ]

# The 8 Gaussian Lloyd-Max reconstruction levels; code k maps to CENTROIDS[k]
# in ascending order.  The pages fix only "3-bit scalar quantization" [RQ];
# the level values are the ones the specification of this path fixes.
CENTROIDS = np.array([-2.1520, -1.3440, -0.7560, -0.2451,
                      0.2451, 0.7560, 1.3440, 2.1520], dtype=np.float64)

# Nearest-centroid decision boundaries = midpoints of adjacent levels,
# rounded once to fp32: the decision itself is an fp32 compare (R7).
THRESHOLDS_F32 = ((CENTROIDS[:-1] + CENTROIDS[1:]) / 2.0).astype(np.float32)

NEAR_EPS = 1e-6                     # boundary exemption width (R17)
FP16_MAX = 65504.0


# ----------------------------------------------------------------------------
# Walsh-Hadamard transform (R1): Sylvester natural order, built entry by entry
# from its definition H[i, j] = (-1)^popcount(i & j), applied as a dense
# product (deliberately O(d^2), not a butterfly).
# ----------------------------------------------------------------------------
@lru_cache(maxsize=None)
def sylvester_hadamard(d: int = HEAD_DIM) -> np.ndarray:
    """Unnormalised Sylvester Hadamard matrix, entries +-1 ([RQ] first stage)."""
    h = np.empty((d, d), dtype=np.float64)
    for i in range(d):
        for j in range(d):
            h[i, j] = -1.0 if bin(i & j).count("1") % 2 else 1.0
    h.setflags(write=False)
    return h


# ----------------------------------------------------------------------------
# Quaternions and SO(4) blocks (R3): components (w, x, y, z) with w real.
# A 4-vector block (v0, v1, v2, v3) is read as v0 + v1 i + v2 j + v3 k, and the
# block rotation is v -> a * v * conj(p), with a = q_L/|q_L|, p = q_R/|q_R|.
# Left and right multiplication by unit quaternions are both rotations of R^4
# with determinant +1, so the product is in SO(4) ([FT141]: quaternion
# rotations; [RQ]: block-diagonal SO(4) rotations).
# ----------------------------------------------------------------------------
def quat_mul(a, b) -> np.ndarray:
    """Hamilton product a*b with i^2 = j^2 = k^2 = ijk = -1."""
    aw, ax, ay, az = (float(t) for t in a)
    bw, bx, by, bz = (float(t) for t in b)
    return np.array([
        aw * bw - ax * bx - ay * by - az * bz,
        aw * bx + ax * bw + ay * bz - az * by,
        aw * by - ax * bz + ay * bw + az * bx,
        aw * bz + ax * by - ay * bx + az * bw,
    ], dtype=np.float64)


def quat_conj(q) -> np.ndarray:
    return np.array([q[0], -q[1], -q[2], -q[3]], dtype=np.float64)


def quat_normalize(q) -> np.ndarray:
    q = np.asarray(q, dtype=np.float64)
    n = math.sqrt(float(np.dot(q, q)))
    if not math.isfinite(n) or n == 0.0:
        raise ValueError("quaternion with zero or non-finite norm")
    return q / n


def so4_block(q_left, q_right) -> np.ndarray:
    """4x4 matrix of v -> a v conj(p): column j is the image of basis e_j."""
    a = quat_normalize(q_left)
    p_conj = quat_conj(quat_normalize(q_right))
    m = np.empty((4, 4), dtype=np.float64)
    for j in range(4):
        e = np.zeros(4)
        e[j] = 1.0
        m[:, j] = quat_mul(quat_mul(a, e), p_conj)
    return m


def rotation_matrices(quats) -> np.ndarray:
    """[Hkv][32][2][4] quaternions ([..][b][0] = q_L, [..][b][1] = q_R) ->
    [Hkv][32][4][4] fp64 block matrices (one rotation per kv head, shared by
    K, V and that head's query group: R5)."""
    quats = np.asarray(quats, dtype=np.float64)
    hkv = quats.shape[0]
    assert quats.shape == (hkv, N_BLOCKS, 2, 4)
    out = np.empty((hkv, N_BLOCKS, 4, 4), dtype=np.float64)
    for h in range(hkv):
        for b in range(N_BLOCKS):
            out[h, b] = so4_block(quats[h, b, 0], quats[h, b, 1])
    return out


# ----------------------------------------------------------------------------
# The orthogonal map T = B * (H / sqrt(d)) (R4: Hadamard first, then SO(4)).
# ----------------------------------------------------------------------------
def forward_rotate(x, blocks) -> np.ndarray:
    """T x for x[..., 128] with one head's blocks [32][4][4] ([RQ])."""
    x = np.asarray(x, dtype=np.float64)
    y = x @ sylvester_hadamard().T / math.sqrt(HEAD_DIM)
    yb = y.reshape(y.shape[:-1] + (N_BLOCKS, 4))
    z = np.einsum("bij,...bj->...bi", blocks, yb)
    return z.reshape(x.shape)


def inverse_rotate(z, blocks) -> np.ndarray:
    """T^T z = (H / sqrt(d)) * B^T z."""
    z = np.asarray(z, dtype=np.float64)
    zb = z.reshape(z.shape[:-1] + (N_BLOCKS, 4))
    y = np.einsum("bji,...bj->...bi", blocks, zb).reshape(z.shape)
    return y @ sylvester_hadamard().T / math.sqrt(HEAD_DIM)


def dense_rotation(blocks) -> np.ndarray:
    """T as an explicit 128x128 matrix (the O(d^2) form [RQ] compares with)."""
    b = np.zeros((HEAD_DIM, HEAD_DIM))
    for k in range(N_BLOCKS):
        b[4 * k:4 * k + 4, 4 * k:4 * k + 4] = blocks[k]
    return b @ sylvester_hadamard() / math.sqrt(HEAD_DIM)


# ----------------------------------------------------------------------------
# fp16 norm storage (R6): round-to-nearest-even, saturating at 65504.
# ----------------------------------------------------------------------------
def fp16_bits_saturating(n) -> np.ndarray:
    n = np.asarray(n, dtype=np.float64)
    with np.errstate(over="ignore"):
        h = n.astype(np.float16)
    h = np.where(np.isinf(h), np.float16(FP16_MAX), h)
    return h.view(np.uint16)


def fp16_bits_to_float(bits) -> np.ndarray:
    return np.asarray(bits, dtype=np.uint16).view(np.float16).astype(np.float64)


def fp16_midpoint_near(n, rel_eps: float = NEAR_EPS) -> np.ndarray:
    """True where n lies within rel_eps (relative) of a point where fp16
    rounding changes value; such norms may legitimately round differently
    when computed in fp32 instead of fp64 (R6/R17)."""
    n = np.asarray(n, dtype=np.float64)
    h = np.minimum(n, FP16_MAX).astype(np.float16)
    with np.errstate(over="ignore"):
        up = np.nextafter(h, np.float16(np.inf)).astype(np.float64)
    dn = np.nextafter(h, np.float16(0)).astype(np.float64)
    hv = h.astype(np.float64)
    mids = np.stack([(hv + up) / 2.0, (hv + dn) / 2.0])
    with np.errstate(invalid="ignore"):
        dist = np.min(np.abs(mids - n), axis=0)
    return dist <= rel_eps * np.maximum(n, 1e-30)


# ----------------------------------------------------------------------------
# Quantiser.  [RQ] (abstract) names a 3-bit scalar quantisation after the
# rotation and leaves its details open; they are fixed here as:
#   n = ||x||_2 of the unrotated input (fp64),
#   u = (T x) * sqrt(d) / n,
#   code_i = #{ j : float32(u_i) >= THRESHOLDS_F32[j] }  (ties go up; R7),
#   stored norm = fp16(n), and the zero vector gets codes 4 and norm 0.
# ----------------------------------------------------------------------------
def quantize(x, blocks):
    """x[N][128] (values exactly as the GPU receives them) -> dict with
    codes uint8[N][128], norm16 uint16[N], near bool[N][128] (a coordinate
    within 1e-6 of a boundary), norm_near bool[N], and u float64[N][128]."""
    x = np.asarray(x, dtype=np.float64).reshape(-1, HEAD_DIM)
    n = np.sqrt(np.sum(x * x, axis=1))
    z = forward_rotate(x, blocks)
    safe = np.where(n > 0, n, 1.0)
    u = z * math.sqrt(HEAD_DIM) / safe[:, None]
    uf = u.astype(np.float32)
    codes = np.zeros(u.shape, dtype=np.uint8)
    for t in THRESHOLDS_F32:
        codes += (uf >= t).astype(np.uint8)
    dist = np.full(u.shape, np.inf)
    for t in THRESHOLDS_F32.astype(np.float64):
        dist = np.minimum(dist, np.abs(u - t))
    near = dist < NEAR_EPS
    zero = n == 0
    codes[zero] = 4
    u[zero] = 0.0
    near[zero] = False
    return {
        "codes": codes,
        "norm16": fp16_bits_saturating(n),
        "near": near,
        "norm_near": fp16_midpoint_near(n),
        "u": u,
        "norm": n,
    }


# ----------------------------------------------------------------------------
# Bit packing (R8, GPU-oriented reading; the pages fix only "packed 3-bit").
# A 48-byte record holds the 128 codes of one vector as four 12-byte groups;
# group g covers coordinates 32g .. 32g+31.  A group is three little-endian
# bytes planes: for byte lane b in 0..3, the bytes at offsets b, 4+b and 8+b
# form a 24-bit little-endian integer, and the code of coordinate
# 32g + 4s + b (s = 0..7) occupies bits 3s .. 3s+2 of that integer.
# Written here bit by bit from that description.
# ----------------------------------------------------------------------------
def _bit_position(coord: int):
    """(byte offset in the record, bit position 0..23 in the byte lane)."""
    g, r = divmod(coord, 32)
    s, b = divmod(r, 4)
    return g, b, 3 * s


def pack_codes(codes) -> np.ndarray:
    codes = np.asarray(codes, dtype=np.uint8).reshape(-1, HEAD_DIM)
    if np.any(codes > 7):
        raise ValueError("codes must be 3-bit")
    out = np.zeros((codes.shape[0], CODE_BYTES), dtype=np.uint8)
    for coord in range(HEAD_DIM):
        g, b, bit = _bit_position(coord)
        c = codes[:, coord].astype(np.uint32)
        for k in range(3):
            pos = bit + k                 # 0..23 within the byte lane
            byte = 12 * g + 4 * (pos // 8) + b
            out[:, byte] |= (((c >> k) & 1) << (pos % 8)).astype(np.uint8)
    return out


def unpack_codes(packed) -> np.ndarray:
    packed = np.asarray(packed, dtype=np.uint8).reshape(-1, CODE_BYTES)
    codes = np.zeros((packed.shape[0], HEAD_DIM), dtype=np.uint8)
    for coord in range(HEAD_DIM):
        g, b, bit = _bit_position(coord)
        for k in range(3):
            pos = bit + k
            byte = 12 * g + 4 * (pos // 8) + b
            codes[:, coord] |= (((packed[:, byte] >> (pos % 8)) & 1) << k).astype(np.uint8)
    return codes


def dequantize_rotated(codes, norm16) -> np.ndarray:
    """Rotated-space reconstruction: fp16(n)/sqrt(d) * C[code] (fp64)."""
    n = fp16_bits_to_float(norm16)
    return CENTROIDS[np.asarray(codes)] * (n / math.sqrt(HEAD_DIM))[..., None]


def dequantize(codes, norm16, blocks) -> np.ndarray:
    """Full-precision reconstruction in the original space: T^T of the above.
    Used only by the brute-force cross-check; the attention path never forms it."""
    return inverse_rotate(dequantize_rotated(codes, norm16), blocks)


# ----------------------------------------------------------------------------
# Paged cache (R9): pages of 64 tokens; per (page, kv head) a 3072-byte block
# of codes and 64 fp16 norms, separately for K and V; token t of sequence s
# lives in page block_table[s][t // 64], slot t % 64.
#
# K blocks hold the 64 records in slot order (slot t at bytes 48t..48t+47).
# V blocks hold the same 48-byte records with their bytes permuted into the
# order the decode matrix cores read them (reading R9b): the block is 64
# regions of 48 bytes; region n + 16q (n = 0..15, q = 0..3) is four 12-byte
# chunks c = 0..3; byte lane r (bytes r, 4+r, 8+r) of chunk c of region
# (n, q) is the 24-bit byte lane n % 4 of group n // 4 of the record in slot
# 16c + 4q + r.  Nothing is lost or added: it is a fixed byte permutation.
# ----------------------------------------------------------------------------
def v_block_offsets() -> np.ndarray:
    """int[64][48]: physical byte offset in a V block of (slot, record byte)."""
    off = np.empty((PAGE_TOKENS, CODE_BYTES), dtype=np.int64)
    for t in range(PAGE_TOKENS):
        c, q, r = t // 16, (t % 16) // 4, t % 4
        for j in range(CODE_BYTES):
            g, k = divmod(j, 12)          # group and byte within the group
            i, b = divmod(k, 4)           # dword w_i of the group, byte lane b
            n = 4 * g + b
            off[t, j] = (n + 16 * q) * 48 + 12 * c + 4 * i + r
    return off


class PagedCache:
    def __init__(self, num_pages: int, n_kv_heads: int):
        self.num_pages = num_pages
        self.n_kv_heads = n_kv_heads
        shape = (num_pages, n_kv_heads, PAGE_TOKENS)
        self.k_codes = np.zeros(shape + (CODE_BYTES,), dtype=np.uint8)
        self.v_codes = np.zeros(shape + (CODE_BYTES,), dtype=np.uint8)
        self.k_norms = np.zeros(shape, dtype=np.uint16)
        self.v_norms = np.zeros(shape, dtype=np.uint16)

    @classmethod
    def from_arrays(cls, k_codes, k_norms, v_codes, v_norms):
        c = cls.__new__(cls)
        c.k_codes, c.k_norms = np.asarray(k_codes), np.asarray(k_norms)
        c.v_codes, c.v_norms = np.asarray(v_codes), np.asarray(v_norms)
        c.num_pages, c.n_kv_heads = c.k_codes.shape[0], c.k_codes.shape[1]
        return c

    def locate(self, block_table, seq: int, pos):
        pos = np.asarray(pos)
        return np.asarray(block_table)[seq, pos // PAGE_TOKENS], pos % PAGE_TOKENS

    def records(self, which: str, page, head: int, slot) -> np.ndarray:
        """48-byte records (K-format byte order) of the given slots."""
        page, slot = np.asarray(page), np.asarray(slot)
        if which == "k":
            return self.k_codes[page, head, slot]
        blocks = self.v_codes[page, head].reshape(np.shape(page) + (PAGE_TOKENS * CODE_BYTES,))
        return np.take_along_axis(blocks, v_block_offsets()[slot], axis=-1)

    def store(self, which: str, page, head: int, slot, recs):
        page, slot = np.asarray(page), np.asarray(slot)
        if which == "k":
            self.k_codes[page, head, slot] = recs
            return
        flat = self.v_codes.reshape(self.num_pages, self.n_kv_heads, PAGE_TOKENS * CODE_BYTES)
        offs = v_block_offsets()[slot]
        for i in range(len(page)):
            flat[page[i], head, offs[i]] = recs[i]

    def gather(self, block_table, seq: int, length: int, head: int, which: str):
        """(codes uint8[length][128], norm16 uint16[length]) of tokens 0..length-1."""
        page, slot = self.locate(block_table, seq, np.arange(length))
        codes = self.records(which, page, head, slot)
        norms = getattr(self, which + "_norms")[page, head, slot]
        return unpack_codes(codes), norms


def quantize_append(cache: PagedCache, blocks_all, k, v, seq_idx, pos, block_table):
    """Quantise each (token, kv head) K and V vector and store it in its slot.
    k, v: [n_tokens][Hkv][128] (exact input values).  Returns the per-vector
    quantiser outputs for K and V (for boundary bookkeeping)."""
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    n_tok, hkv, _ = k.shape
    info = {}
    for name, x in (("k", k), ("v", v)):
        per_head = []
        for h in range(hkv):
            q = quantize(x[:, h, :], blocks_all[h])
            per_head.append(q)
            packed = pack_codes(q["codes"])
            pos_a = np.asarray(pos, dtype=np.int64)
            page = np.asarray(block_table)[np.asarray(seq_idx, dtype=np.int64),
                                           pos_a // PAGE_TOKENS]
            slot = pos_a % PAGE_TOKENS
            cache.store(name, page, h, slot, packed)
            getattr(cache, name + "_norms")[page, h, slot] = q["norm16"]
        info[name] = per_head
    return info


# ----------------------------------------------------------------------------
# Attention in the rotated space (R10).  q' = T q; scores use the rotated,
# dequantised keys; the value accumulator stays rotated and is mapped back
# once with T^T.  Because T is orthogonal, this equals ordinary attention on
# the dequantised K and V ([RQ]: attention on the packed tensors without
# materialising full-precision KV).
# ----------------------------------------------------------------------------
def default_scale(scale: float | None) -> float:
    return 1.0 / math.sqrt(HEAD_DIM) if scale is None or scale <= 0 else float(scale)


def _softmax_weighted(scores: np.ndarray, values: np.ndarray) -> np.ndarray:
    """softmax(scores) @ values in fp64, max-subtracted.  An empty key set
    gives zeros (never NaN: [FTREL] #654)."""
    if scores.shape[-1] == 0:
        return np.zeros(scores.shape[:-1] + values.shape[-1:])
    m = np.max(scores, axis=-1, keepdims=True)
    p = np.exp(scores - m)
    return (p @ values) / np.sum(p, axis=-1, keepdims=True)


def decode_attention(cache: PagedCache, blocks_all, q, block_table, seq_lens, scale=None):
    """q[B][Hq][128] -> out[B][Hq][128] fp64: every query head of sequence b
    attends the seq_lens[b] cached tokens of its kv head h // (Hq/Hkv)."""
    q = np.asarray(q, dtype=np.float64)
    bsz, hq, _ = q.shape
    hkv = cache.n_kv_heads
    if hq % hkv:
        raise ValueError("query heads must be a multiple of kv heads")
    grp = hq // hkv
    sc = default_scale(scale)
    out = np.zeros_like(q)
    for b in range(bsz):
        length = int(seq_lens[b])
        for g in range(hkv):
            kc, kn = cache.gather(block_table, b, length, g, "k")
            vc, vn = cache.gather(block_table, b, length, g, "v")
            k_rot = dequantize_rotated(kc, kn)
            v_rot = dequantize_rotated(vc, vn)
            qr = forward_rotate(q[b, g * grp:(g + 1) * grp], blocks_all[g])
            o_rot = _softmax_weighted(sc * qr @ k_rot.T, v_rot)
            out[b, g * grp:(g + 1) * grp] = inverse_rotate(o_rot, blocks_all[g])
    return out


def prefill_attention(cache: PagedCache, blocks_all, q, q_start, block_table_row, scale=None,
                      rows=None):
    """Causal attention of one sequence's query chunk: q[n_q][Hq][128]; query i
    sits at position q_start + i and attends keys 0 .. q_start + i (R10).
    ``rows`` optionally restricts the computation to a list of query indices."""
    q = np.asarray(q, dtype=np.float64)
    n_q, hq, _ = q.shape
    hkv = cache.n_kv_heads
    grp = hq // hkv
    sc = default_scale(scale)
    rows = np.arange(n_q) if rows is None else np.asarray(rows)
    kv_len = int(q_start + rows.max() + 1)
    bt = np.asarray(block_table_row).reshape(1, -1)
    out = np.zeros((len(rows), hq, HEAD_DIM))
    for g in range(hkv):
        kc, kn = cache.gather(bt, 0, kv_len, g, "k")
        vc, vn = cache.gather(bt, 0, kv_len, g, "v")
        k_rot = dequantize_rotated(kc, kn)
        v_rot = dequantize_rotated(vc, vn)
        for ri, i in enumerate(rows):
            visible = int(q_start + i + 1)
            qr = forward_rotate(q[i, g * grp:(g + 1) * grp], blocks_all[g])
            o_rot = _softmax_weighted(sc * qr @ k_rot[:visible].T, v_rot[:visible])
            out[ri, g * grp:(g + 1) * grp] = inverse_rotate(o_rot, blocks_all[g])
    return out


def reference_attention(q, k, v, scale=None, visible=None):
    """Uncompressed fp64 attention for one head: q[R][128], k, v[L][128];
    row r sees keys 0 .. visible[r]-1 (all if None).  Used for the cosine
    similarity of compressed vs uncompressed attention."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    sc = default_scale(scale)
    if visible is None:
        return _softmax_weighted(sc * q @ k.T, v)
    out = np.zeros((q.shape[0], HEAD_DIM))
    for r in range(q.shape[0]):
        n = int(visible[r])
        out[r] = _softmax_weighted(sc * q[r:r + 1] @ k[:n].T, v[:n])[0]
    return out


def row_relative_error(got, ref) -> np.ndarray:
    """Per output row: max_i |got - ref| / max_i |ref| (R11)."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    num = np.max(np.abs(got - ref), axis=-1)
    den = np.max(np.abs(ref), axis=-1)
    return np.where(den > 0, num / np.where(den > 0, den, 1.0), num)


def row_cosine(a, b) -> np.ndarray:
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    na = np.linalg.norm(a, axis=-1)
    nb = np.linalg.norm(b, axis=-1)
    return np.sum(a * b, axis=-1) / np.maximum(na * nb, 1e-300)
