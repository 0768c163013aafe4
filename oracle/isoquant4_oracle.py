"""Plain CPU oracle for the 4-bit IsoQuant variant (TEST INFRASTRUCTURE).

Only the test suite may import this module (with ``isoquant_oracle``, of which
it reuses the rotation, the fp16 norm rules and the softmax); it shares no
code, tables or constants with the GPU library.

Sources (cited by page title and section):

* [RQ] "RotaryQuant: Fitting 120B MoE Models on Consumer Hardware via Fused
  Compressed-Space Attention", abstract: Walsh-Hadamard transform, then
  block-diagonal SO(4) rotations, then low-bit scalar quantisation; attention
  runs on the packed tensors.
* [FT141] FreeToken issue #141 ("unified KV cache backend"), Proposed
  Solution: the rotation-based KV quantisers it lists span 3 and 4 bits (the
  TurboQuant line); this is the 4-bit member of the same pipeline.

Readings (the pages fix the pipeline, not the 4-bit codebook or packing):

* R4-1 Codebook: the 16-level Lloyd-Max quantiser of N(0, 1), computed here
  by Lloyd's iteration (decision thresholds at the midpoints of adjacent
  levels, each level the conditional mean of its cell).  The same iteration
  with 8 levels reproduces, to their four digits, the 3-bit levels the
  specification of this path fixes (the pages print no codebook), which pins
  the iteration.
* R4-2 Decision: code = #{j : float32(u) >= fp32 midpoint j} (ties go up),
  u = (T x) sqrt(d) / n as for 3 bits; the zero vector gets code 8.
* R4-3 Stored nibble: sign-magnitude, nib = c - 8 for c >= 8 (levels >= 0)
  and nib = 8 + (7 - c) for c < 8: bit 3 marks the negative side, bits 0-2
  the magnitude index (0 = smallest).  A bijection of the 16 codes.
* R4-4 Record: 64 bytes of nibbles + fp16 norm (66 B per vector).  Dword d
  (d = 0..15) holds coordinates 8 d .. 8 d + 7: byte b of it carries
  coordinate 8 d + b in its low nibble and 8 d + 4 + b in its high one.
* R4-5 V blocks: the 4,096 bytes of (page, kv head) are 64 regions of 64 B;
  region n + 16 jq (n < 16, jq < 4) is 16 dwords, dword 4 p + 2 th + q
  (p < 4, th < 2, q < 2); byte r of it belongs to the token in slot
  32 th + 16 q + 4 jq + r and carries coordinate c = 32 (n // 4) + 4 p +
  n % 4 in its low nibble and c + 16 in its high one.  Every byte holds two
  codes of one token.
"""

from __future__ import annotations

import math
from functools import lru_cache

import numpy as np

from oracle import isoquant_oracle as O

HEAD_DIM = O.HEAD_DIM
PAGE_TOKENS = O.PAGE_TOKENS
CODE_BYTES4 = HEAD_DIM // 2         # 64 bytes of 4-bit codes per vector
NEAR_EPS = O.NEAR_EPS


# ----------------------------------------------------------------------------
# R4-1: Lloyd's iteration for the standard normal.
# ----------------------------------------------------------------------------
def _phi(x: float) -> float:
    return 0.0 if math.isinf(x) else math.exp(-0.5 * x * x) / math.sqrt(2.0 * math.pi)


def _cdf(x: float) -> float:
    if math.isinf(x):
        return 0.0 if x < 0 else 1.0
    return 0.5 * (1.0 + math.erf(x / math.sqrt(2.0)))


def lloyd_max_gaussian(levels: int, tol: float = 1e-15, max_iter: int = 200000) -> np.ndarray:
    """Ascending reconstruction levels of the `levels`-level Lloyd-Max
    quantiser of N(0, 1): alternate (a) thresholds = midpoints of adjacent
    levels and (b) levels = E[X | cell] = (phi(a) - phi(b)) / (Phi(b) - Phi(a)),
    from evenly spaced levels, until no level moves by more than `tol`."""
    c = np.linspace(-2.0, 2.0, levels)
    for _ in range(max_iter):
        t = np.concatenate([[-math.inf], (c[:-1] + c[1:]) / 2.0, [math.inf]])
        new = np.array([(_phi(t[i]) - _phi(t[i + 1])) / (_cdf(t[i + 1]) - _cdf(t[i]))
                        for i in range(levels)])
        moved = float(np.max(np.abs(new - c)))
        c = new
        if moved < tol:
            break
    return c


@lru_cache(maxsize=None)
def centroids4() -> np.ndarray:
    """The 16 levels, symmetrised (the Lloyd-Max codebook of a symmetric
    density is symmetric; the iteration leaves ~1e-16 of rounding asymmetry,
    which would move the middle threshold off 0)."""
    c = lloyd_max_gaussian(16)
    c = (c - c[::-1]) / 2.0
    c.setflags(write=False)
    return c


@lru_cache(maxsize=None)
def thresholds4_f32() -> np.ndarray:
    c = centroids4()
    t = ((c[:-1] + c[1:]) / 2.0).astype(np.float32)
    t.setflags(write=False)
    return t


def gaussian_mse(levels: np.ndarray) -> float:
    """E[(X - Q(X))^2] for N(0,1) with nearest-level quantisation, from the
    closed form of the truncated moments of each cell."""
    c = np.asarray(levels, dtype=np.float64)
    t = np.concatenate([[-math.inf], (c[:-1] + c[1:]) / 2.0, [math.inf]])
    mse = 0.0
    for i, ci in enumerate(c):
        a, b = t[i], t[i + 1]
        p = _cdf(b) - _cdf(a)
        m1 = _phi(a) - _phi(b)                                   # int x phi
        m2 = p + ((a * _phi(a)) if not math.isinf(a) else 0.0) - ((b * _phi(b)) if not math.isinf(b) else 0.0)
        mse += m2 - 2.0 * ci * m1 + ci * ci * p
    return mse


# ----------------------------------------------------------------------------
# R4-2 / R4-3: quantiser and stored nibbles.
# ----------------------------------------------------------------------------
def nibble_of_code(c) -> np.ndarray:
    c = np.asarray(c, dtype=np.int64)
    return np.where(c >= 8, c - 8, 15 - c).astype(np.uint8)


def code_of_nibble(nib) -> np.ndarray:
    nib = np.asarray(nib, dtype=np.int64)
    return np.where(nib < 8, nib + 8, 15 - nib).astype(np.uint8)


def quantize4(x, blocks):
    """As isoquant_oracle.quantize with the 16-level codebook (codes 0..15)."""
    x = np.asarray(x, dtype=np.float64).reshape(-1, HEAD_DIM)
    n = np.sqrt(np.sum(x * x, axis=1))
    z = O.forward_rotate(x, blocks)
    safe = np.where(n > 0, n, 1.0)
    u = z * math.sqrt(HEAD_DIM) / safe[:, None]
    uf = u.astype(np.float32)
    codes = np.zeros(u.shape, dtype=np.uint8)
    for t in thresholds4_f32():
        codes += (uf >= t).astype(np.uint8)
    dist = np.full(u.shape, np.inf)
    for t in thresholds4_f32().astype(np.float64):
        dist = np.minimum(dist, np.abs(u - t))
    near = dist < NEAR_EPS
    zero = n == 0
    codes[zero] = 8
    u[zero] = 0.0
    near[zero] = False
    return {"codes": codes, "norm16": O.fp16_bits_saturating(n), "near": near,
            "norm_near": O.fp16_midpoint_near(n), "u": u, "norm": n}


# ----------------------------------------------------------------------------
# R4-4: record packing, from the layout description.
# ----------------------------------------------------------------------------
def record_position(coord: int):
    """(byte offset in the 64-byte record, nibble shift 0 or 4)."""
    d, e = divmod(coord, 8)
    return 4 * d + (e % 4), 4 * (e // 4)


def pack4(codes) -> np.ndarray:
    codes = np.asarray(codes, dtype=np.uint8).reshape(-1, HEAD_DIM)
    if np.any(codes > 15):
        raise ValueError("codes must be 4-bit")
    nib = nibble_of_code(codes)
    out = np.zeros((codes.shape[0], CODE_BYTES4), dtype=np.uint8)
    for coord in range(HEAD_DIM):
        off, sh = record_position(coord)
        out[:, off] |= (nib[:, coord] << sh).astype(np.uint8)
    return out


def unpack4(packed) -> np.ndarray:
    packed = np.asarray(packed, dtype=np.uint8).reshape(-1, CODE_BYTES4)
    nib = np.zeros((packed.shape[0], HEAD_DIM), dtype=np.uint8)
    for coord in range(HEAD_DIM):
        off, sh = record_position(coord)
        nib[:, coord] = (packed[:, off] >> sh) & 15
    return code_of_nibble(nib)


# ----------------------------------------------------------------------------
# R4-5: V block nibble positions.
# ----------------------------------------------------------------------------
def v4_position(slot: int, coord: int):
    """(byte offset in the 4,096-byte V block, nibble shift) of (slot, coord)."""
    th, rest = divmod(slot, 32)
    q, rest = divmod(rest, 16)
    jq, r = divmod(rest, 4)
    a, rest = divmod(coord, 32)
    m, b = divmod(rest, 4)            # coordinate 32 a + 4 m + b, m = 0..7
    high, p = divmod(m, 4)
    region = (4 * a + b) + 16 * jq
    return region * 64 + 4 * (4 * p + 2 * th + q) + r, 4 * high


@lru_cache(maxsize=None)
def v4_offsets():
    off = np.empty((PAGE_TOKENS, HEAD_DIM), dtype=np.int64)
    sh = np.empty((PAGE_TOKENS, HEAD_DIM), dtype=np.int64)
    for t in range(PAGE_TOKENS):
        for c in range(HEAD_DIM):
            off[t, c], sh[t, c] = v4_position(t, c)
    return off, sh


class PagedCache4:
    """Cache of 4-bit records: k_codes [pages][Hkv][64][64] (slot-ordered
    records), v_codes [pages][Hkv][64][64] (a 4,096-byte block in the R4-5
    order, shaped like the K block), fp16 norms as for 3 bits."""

    def __init__(self, num_pages: int, n_kv_heads: int):
        self.num_pages, self.n_kv_heads = num_pages, n_kv_heads
        shape = (num_pages, n_kv_heads, PAGE_TOKENS)
        self.k_codes = np.zeros(shape + (CODE_BYTES4,), dtype=np.uint8)
        self.v_codes = np.zeros(shape + (CODE_BYTES4,), dtype=np.uint8)
        self.k_norms = np.zeros(shape, dtype=np.uint16)
        self.v_norms = np.zeros(shape, dtype=np.uint16)

    @classmethod
    def from_arrays(cls, k_codes, k_norms, v_codes, v_norms):
        c = cls.__new__(cls)
        c.k_codes, c.k_norms = np.asarray(k_codes), np.asarray(k_norms)
        c.v_codes, c.v_norms = np.asarray(v_codes), np.asarray(v_norms)
        c.num_pages, c.n_kv_heads = c.k_codes.shape[0], c.k_codes.shape[1]
        return c

    def codes(self, which: str, page, head: int, slot) -> np.ndarray:
        """Codes (0..15) [len][128] of the given slots."""
        page, slot = np.asarray(page), np.asarray(slot)
        if which == "k":
            return unpack4(self.k_codes[page, head, slot])
        off, sh = v4_offsets()
        blocks = self.v_codes[page, head].reshape(len(page), PAGE_TOKENS * CODE_BYTES4)
        nib = (np.take_along_axis(blocks, off[slot], axis=1) >> sh[slot]) & 15
        return code_of_nibble(nib)

    def store(self, which: str, page, head: int, slot, codes):
        page, slot = np.asarray(page), np.asarray(slot)
        if which == "k":
            self.k_codes[page, head, slot] = pack4(codes)
            return
        off, sh = v4_offsets()
        nib = nibble_of_code(codes).astype(np.uint8)
        flat = self.v_codes.reshape(self.num_pages, self.n_kv_heads, PAGE_TOKENS * CODE_BYTES4)
        for i in range(len(page)):
            # two coordinates share each byte: clear and set nibble by nibble
            # (ufunc.at applies repeated byte indices one after another)
            o, s = off[slot[i]], sh[slot[i]].astype(np.uint8)
            row = flat[int(page[i]), head]
            np.bitwise_and.at(row, o, ~(np.uint8(15) << s))
            np.bitwise_or.at(row, o, nib[i] << s)

    def gather(self, block_table, seq: int, length: int, head: int, which: str):
        pos = np.arange(length)
        page, slot = np.asarray(block_table)[seq, pos // PAGE_TOKENS], pos % PAGE_TOKENS
        return self.codes(which, page, head, slot), getattr(self, which + "_norms")[page, head, slot]


def quantize_append4(cache: PagedCache4, blocks_all, k, v, seq_idx, pos, block_table):
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    info = {}
    for name, x in (("k", k), ("v", v)):
        per_head = []
        for h in range(x.shape[1]):
            q = quantize4(x[:, h, :], blocks_all[h])
            per_head.append(q)
            pos_a = np.asarray(pos, dtype=np.int64)
            page = np.asarray(block_table)[np.asarray(seq_idx, dtype=np.int64), pos_a // PAGE_TOKENS]
            slot = pos_a % PAGE_TOKENS
            cache.store(name, page, h, slot, q["codes"])
            getattr(cache, name + "_norms")[page, h, slot] = q["norm16"]
        info[name] = per_head
    return info


def dequantize_rotated4(codes, norm16) -> np.ndarray:
    n = O.fp16_bits_to_float(norm16)
    return centroids4()[np.asarray(codes)] * (n / math.sqrt(HEAD_DIM))[..., None]


def decode_attention4(cache: PagedCache4, blocks_all, q, block_table, seq_lens, scale=None):
    """As isoquant_oracle.decode_attention over 4-bit records."""
    q = np.asarray(q, dtype=np.float64)
    bsz, hq, _ = q.shape
    hkv = cache.n_kv_heads
    grp = hq // hkv
    sc = O.default_scale(scale)
    out = np.zeros_like(q)
    for b in range(bsz):
        length = int(seq_lens[b])
        for g in range(hkv):
            kc, kn = cache.gather(block_table, b, length, g, "k")
            vc, vn = cache.gather(block_table, b, length, g, "v")
            qr = O.forward_rotate(q[b, g * grp:(g + 1) * grp], blocks_all[g])
            o_rot = O._softmax_weighted(sc * qr @ dequantize_rotated4(kc, kn).T, dequantize_rotated4(vc, vn))
            out[b, g * grp:(g + 1) * grp] = O.inverse_rotate(o_rot, blocks_all[g])
    return out


def prefill_attention4(cache: PagedCache4, blocks_all, q, q_start, block_table_row, scale=None,
                       rows=None):
    """As isoquant_oracle.prefill_attention over 4-bit records: query i sits at
    position q_start + i and attends keys 0 .. q_start + i."""
    q = np.asarray(q, dtype=np.float64)
    n_q, hq, _ = q.shape
    hkv = cache.n_kv_heads
    grp = hq // hkv
    sc = O.default_scale(scale)
    rows = np.arange(n_q) if rows is None else np.asarray(rows)
    kv_len = int(q_start + rows.max() + 1)
    bt = np.asarray(block_table_row).reshape(1, -1)
    out = np.zeros((len(rows), hq, HEAD_DIM))
    for g in range(hkv):
        kc, kn = cache.gather(bt, 0, kv_len, g, "k")
        vc, vn = cache.gather(bt, 0, kv_len, g, "v")
        k_rot = dequantize_rotated4(kc, kn)
        v_rot = dequantize_rotated4(vc, vn)
        for ri, i in enumerate(rows):
            visible = int(q_start + i + 1)
            qr = O.forward_rotate(q[i, g * grp:(g + 1) * grp], blocks_all[g])
            o_rot = O._softmax_weighted(sc * qr @ k_rot[:visible].T, v_rot[:visible])
            out[ri, g * grp:(g + 1) * grp] = O.inverse_rotate(o_rot, blocks_all[g])
    return out
