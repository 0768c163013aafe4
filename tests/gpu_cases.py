"""Shared builders for the GPU parity tests: seeded scenarios fed identically to
the HIP path (through the C-ABI binding) and to the CPU oracle."""

from __future__ import annotations

import math

import numpy as np
import torch

from compressed_space_attention_amd import synth
from oracle import isoquant4_oracle as O4
from oracle import isoquant_oracle as O

TORCH_DTYPE = {"f32": torch.float32, "bf16": torch.bfloat16, "f16": torch.float16}


class Scenario:
    """Sequences of given lengths, quantised into one paged cache by the GPU."""

    def __init__(self, seed, lens, hkv, dtype="bf16", outliers=False, shuffle=True,
                 identity=False, extra_pages=2, kv_override=None, hold_last=False, bits=3):
        """hold_last: append all but the last token of each sequence; that token's
        rows are kept in k_last / v_last ([B][Hkv][128], zeros for an empty
        sequence) for a decode step to append.  bits: record width (3 or 4)."""
        from compressed_space_attention_amd import isoquant as iq
        self.iq = iq
        self.bits = bits
        self.seed, self.lens, self.hkv, self.dtype = seed, [int(n) for n in lens], hkv, dtype
        self.quats = synth.identity_quaternions(hkv) if identity else synth.quaternions(seed, hkv)
        self.blocks = O.rotation_matrices(self.quats)
        pages = [max(1, -(-n // 64)) for n in self.lens]
        self.block_table, self.num_pages = synth.block_table(seed + 1, pages, shuffle, extra_pages)
        n_tok = sum(self.lens)
        out_ch = synth.outlier_channels(seed + 2, hkv) if outliers else None
        if kv_override is not None:
            self.k, self.v = kv_override
        else:
            self.k = synth.kv_vectors(seed + 3, n_tok, hkv, dtype, out_ch)
            self.v = synth.kv_vectors(seed + 4, n_tok, hkv, dtype, None)
        self.seq_idx = np.concatenate([np.full(n, b, np.int32) for b, n in enumerate(self.lens)]) \
            if n_tok else np.zeros(0, np.int32)
        self.pos = np.concatenate([np.arange(n, dtype=np.int32) for n in self.lens]) \
            if n_tok else np.zeros(0, np.int32)
        dev = "cuda"
        self.rot = iq.rotation_init(self.quats, device=dev)
        self.cache = iq.PagedCache(self.num_pages, hkv, device=dev, zero=True, bits=bits)
        self.bt_dev = torch.from_numpy(self.block_table).to(dev)
        self.lens_dev = torch.tensor(self.lens, dtype=torch.int32, device=dev)
        keep = np.ones(n_tok, bool)
        if hold_last:
            ends = np.cumsum(self.lens) - 1
            self.k_last = torch.zeros((len(self.lens), hkv, 128), dtype=self.k.dtype)
            self.v_last = torch.zeros_like(self.k_last)
            for b, n in enumerate(self.lens):
                if n:
                    keep[ends[b]] = False
                    self.k_last[b] = self.k[ends[b]]
                    self.v_last[b] = self.v[ends[b]]
            self.k_last, self.v_last = self.k_last.to(dev), self.v_last.to(dev)
        if keep.any():
            sel = torch.from_numpy(np.nonzero(keep)[0])
            iq.quantize_append(self.cache, self.rot, self.k[sel].contiguous().to(dev),
                               self.v[sel].contiguous().to(dev),
                               torch.from_numpy(self.seq_idx[keep]).to(dev),
                               torch.from_numpy(self.pos[keep]).to(dev), self.bt_dev)
        torch.cuda.synchronize()

    def host_cache(self):
        if self.bits == 4:
            return O4.PagedCache4.from_arrays(*self.cache.to_host())
        return O.PagedCache.from_arrays(*self.cache.to_host())

    def oracle_cache(self):
        k, v = self.k.double().numpy(), self.v.double().numpy()
        if self.bits == 4:
            c = O4.PagedCache4(self.num_pages, self.hkv)
            info = O4.quantize_append4(c, self.blocks, k, v, self.seq_idx, self.pos, self.block_table)
        else:
            c = O.PagedCache(self.num_pages, self.hkv)
            info = O.quantize_append(c, self.blocks, k, v, self.seq_idx, self.pos, self.block_table)
        return c, info

    def oracle_decode(self, cache, q, lens=None):
        """The oracle's decode attention over `cache` (a host copy)."""
        fn = O4.decode_attention4 if self.bits == 4 else O.decode_attention
        return fn(cache, self.blocks, q, self.block_table, self.lens if lens is None else lens)

    def queries(self, seed, batch, hq, dtype=None):
        x = synth.normal(seed, (batch, hq, 128))
        return synth.to_dtype(x, dtype or self.dtype)


def code_parity(gpu: O.PagedCache, ref: O.PagedCache, info, scen: Scenario):
    """Compare every written record.  Returns a dict of counts; raises on a
    mismatch that is not explained by the near-boundary exemption."""
    page, slot = scen.block_table[scen.seq_idx, scen.pos // 64], scen.pos % 64
    stats = {"codes": 0, "mismatch": 0, "near": 0, "norm_mismatch": 0}
    for name in ("k", "v"):
        for h in range(scen.hkv):
            g_rec = gpu.records(name, page, h, slot)
            r_rec = ref.records(name, page, h, slot)
            g_codes, r_codes = O.unpack_codes(g_rec), O.unpack_codes(r_rec)
            near = info[name][h]["near"]
            bad = g_codes != r_codes
            stats["codes"] += g_codes.size
            stats["mismatch"] += int(bad.sum())
            stats["near"] += int(near.sum())
            if np.any(bad & ~near):
                i, j = np.argwhere(bad & ~near)[0]
                raise AssertionError(f"{name} head {h} vector {i} coord {j}: gpu {g_codes[i, j]} "
                                     f"oracle {r_codes[i, j]} u={info[name][h]['u'][i, j]!r}")
            # records whose codes agree must agree byte for byte (in place, too)
            same = ~bad.any(axis=1)
            assert np.array_equal(g_rec[same], r_rec[same]), f"{name} packing differs"
            if name == "v" and np.all(same):
                pg = np.unique(page)
                assert np.array_equal(gpu.v_codes[pg, h], ref.v_codes[pg, h]) or len(pg) == 0
            gn = getattr(gpu, name + "_norms")[page, h, slot]
            rn = getattr(ref, name + "_norms")[page, h, slot]
            nb = gn != rn
            stats["norm_mismatch"] += int(nb.sum())
            if np.any(nb & ~info[name][h]["norm_near"]):
                i = int(np.argwhere(nb & ~info[name][h]["norm_near"])[0][0])
                raise AssertionError(f"{name} head {h} vector {i}: norm bits {gn[i]:#x} vs {rn[i]:#x}")
    return stats


def code_parity4(gpu: O4.PagedCache4, ref: O4.PagedCache4, info, scen: Scenario):
    """code_parity for 4-bit caches: codes bit for bit outside the boundary
    exemption; K records of agreeing vectors byte for byte; the V blocks of
    the touched pages byte for byte where every code agrees; norms as there."""
    page, slot = scen.block_table[scen.seq_idx, scen.pos // 64], scen.pos % 64
    stats = {"codes": 0, "mismatch": 0, "near": 0, "norm_mismatch": 0}
    for name in ("k", "v"):
        all_same = True
        for h in range(scen.hkv):
            g_codes, r_codes = gpu.codes(name, page, h, slot), ref.codes(name, page, h, slot)
            near = info[name][h]["near"]
            bad = g_codes != r_codes
            stats["codes"] += g_codes.size
            stats["mismatch"] += int(bad.sum())
            stats["near"] += int(near.sum())
            if np.any(bad & ~near):
                i, j = np.argwhere(bad & ~near)[0]
                raise AssertionError(f"{name} head {h} vector {i} coord {j}: gpu {g_codes[i, j]} "
                                     f"oracle {r_codes[i, j]} u={info[name][h]['u'][i, j]!r}")
            same = ~bad.any(axis=1)
            all_same &= bool(np.all(same))
            if name == "k":
                assert np.array_equal(gpu.k_codes[page, h, slot][same], ref.k_codes[page, h, slot][same])
            gn = getattr(gpu, name + "_norms")[page, h, slot]
            rn = getattr(ref, name + "_norms")[page, h, slot]
            nb = gn != rn
            stats["norm_mismatch"] += int(nb.sum())
            if np.any(nb & ~info[name][h]["norm_near"]):
                i = int(np.argwhere(nb & ~info[name][h]["norm_near"])[0][0])
                raise AssertionError(f"{name} head {h} vector {i}: norm bits {gn[i]:#x} vs {rn[i]:#x}")
        if name == "v" and all_same and len(page):
            pg = np.unique(page)
            assert np.array_equal(gpu.v_codes[pg], ref.v_codes[pg]), "V block bytes differ"
    return stats


def max_row_error(got, ref):
    return float(np.max(O.row_relative_error(got, ref))) if np.size(ref) else 0.0


def tol():
    """Attention tolerance of the path: max over rows of max|err| / max|ref|."""
    return 1e-3


def sqrt_d():
    return math.sqrt(128)
