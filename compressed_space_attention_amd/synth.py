"""Seeded synthetic inputs shared by the HIP path's tests, the oracle's tests
and the benchmark.

This module generates inputs only; it contains none of the method's
arithmetic (no rotation, quantisation or attention).  Every tensor is drawn
from numpy's PCG64 ``default_rng(seed)`` in float32 and, for bf16 workloads,
rounded to bfloat16 by torch (round-to-nearest-even), so both sides receive
bit-identical values.  Large benchmark inputs can instead be drawn on the GPU
with a seeded ``torch.Generator`` (``draw_normal_device``).
"""

from __future__ import annotations

import numpy as np
import torch

PAGE_TOKENS = 64
HEAD_DIM = 128
N_BLOCKS = 32


def rng(seed: int) -> np.random.Generator:
    return np.random.default_rng(seed)


def quaternions(seed: int, n_kv_heads: int) -> np.ndarray:
    """[Hkv][32][2][4] float32, each component N(0,1) (not normalised: the
    library normalises, as its contract says)."""
    return rng(seed).standard_normal((n_kv_heads, N_BLOCKS, 2, 4)).astype(np.float32)


def identity_quaternions(n_kv_heads: int) -> np.ndarray:
    q = np.zeros((n_kv_heads, N_BLOCKS, 2, 4), dtype=np.float32)
    q[..., 0] = 1.0
    return q


def outlier_channels(seed: int, n_kv_heads: int, count: int = 4) -> np.ndarray:
    """Per kv head, `count` distinct channel indices in [0, 128)."""
    g = rng(seed)
    return np.stack([g.choice(HEAD_DIM, size=count, replace=False) for _ in range(n_kv_heads)])


def normal(seed: int, shape, chunk: int = 1 << 24) -> np.ndarray:
    """float32 N(0,1) of the given shape, drawn in chunks to bound memory."""
    g = rng(seed)
    out = np.empty(int(np.prod(shape)), dtype=np.float32)
    for s in range(0, out.size, chunk):
        e = min(out.size, s + chunk)
        out[s:e] = g.standard_normal(e - s, dtype=np.float32)
    return out.reshape(shape)


def to_dtype(x: np.ndarray, dtype: str) -> torch.Tensor:
    t = torch.from_numpy(np.ascontiguousarray(x))
    if dtype == "bf16":
        return t.to(torch.bfloat16)
    if dtype == "f16":
        return t.to(torch.float16)
    if dtype == "f32":
        return t.to(torch.float32)
    raise ValueError(dtype)


def kv_vectors(seed: int, n_tokens: int, n_kv_heads: int, dtype: str,
               outliers: np.ndarray | None = None, scale: float = 10.0) -> torch.Tensor:
    """[n_tokens][Hkv][128]: N(0,1), optionally with the given channels of each
    head multiplied by `scale` before rounding to `dtype` (RoPE-like outliers)."""
    x = normal(seed, (n_tokens, n_kv_heads, HEAD_DIM))
    if outliers is not None:
        for h in range(n_kv_heads):
            x[:, h, outliers[h]] *= scale
    return to_dtype(x, dtype)


def block_table(seed: int, seq_pages, shuffle: bool, extra_pages: int = 0):
    """Hand out pages of one pool to sequences in order.  With `shuffle`, the
    pool is a seeded permutation, so a sequence's pages are scattered.
    Returns (table int32[B][max pages], total pages); unused entries are 0."""
    seq_pages = [int(p) for p in seq_pages]
    total = sum(seq_pages) + extra_pages
    pool = rng(seed).permutation(total) if shuffle else np.arange(total)
    width = max(1, max(seq_pages) if seq_pages else 1)
    table = np.zeros((len(seq_pages), width), dtype=np.int32)
    at = 0
    for b, n in enumerate(seq_pages):
        table[b, :n] = pool[at:at + n]
        at += n
    return table, total


def ragged_lengths(seed: int, count: int, lo: int, hi: int) -> np.ndarray:
    return rng(seed).integers(lo, hi, endpoint=True, size=count).astype(np.int32)


def draw_normal_device(seed: int, shape, dtype: torch.dtype, device="cuda") -> torch.Tensor:
    """Large N(0,1) inputs drawn directly on the device (benchmark caches)."""
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return torch.randn(shape, generator=g, device=device, dtype=torch.float32).to(dtype)
