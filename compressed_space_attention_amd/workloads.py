"""The synthetic workloads of the long-context KV path, with their seeds.

Shapes follow the workloads the pages describe: 32K-128K contexts of MoE
models, GQA groups of 1-8, d = 128, 64-token pages ("RotaryQuant ...",
abstract: 32K retrieval context; FreeToken v0.2.0 release notes, Kernels:
batch-1 decode at 128K).  Inputs are N(0,1); keys of the decode workloads
carry 4 seeded outlier channels per kv head scaled by 10 (RoPE-like).
"""

from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

from . import synth


@dataclass
class DecodeWorkload:
    name: str
    batch: int
    n_q_heads: int
    n_kv_heads: int
    dtype: str            # "f32" or "bf16"
    k_outliers: bool
    shuffle_pages: bool
    seed: int
    context: int = 0      # fixed context (0 -> ragged)
    ragged: tuple = ()    # (lo, hi) inclusive, for ragged batches

    def seq_lens(self) -> np.ndarray:
        if self.ragged:
            return synth.ragged_lengths(self.seed + 1, self.batch, *self.ragged)
        return np.full(self.batch, self.context, dtype=np.int32)

    @property
    def group(self) -> int:
        return self.n_q_heads // self.n_kv_heads


@dataclass
class PrefillWorkload:
    name: str
    n_kv_heads: int
    n_q_heads: int
    cached: int           # tokens already in the cache (quantised untimed)
    appended: int         # tokens quantise-appended in the timed step
    n_queries: int        # causal query chunk = the last n_queries positions
    dtype: str
    seed: int

    @property
    def total(self) -> int:
        return self.cached + self.appended

    @property
    def q_start(self) -> int:
        return self.total - self.n_queries


TINY_DECODE = DecodeWorkload("tiny_decode_2k_1q1kv", batch=1, n_q_heads=1, n_kv_heads=1,
                             dtype="f32", k_outliers=False, shuffle_pages=False,
                             seed=1001, context=2048)
GQA_DECODE_32K = DecodeWorkload("gqa_decode_32k_32q4kv", batch=1, n_q_heads=32, n_kv_heads=4,
                                dtype="bf16", k_outliers=True, shuffle_pages=True,
                                seed=2002, context=32768)
RAGGED_DECODE = DecodeWorkload("ragged_decode_16seq_8k_64k_32q4kv", batch=16, n_q_heads=32,
                               n_kv_heads=4, dtype="bf16", k_outliers=False,
                               shuffle_pages=True, seed=3003, ragged=(8192, 65536))
LONG_DECODE_128K = DecodeWorkload("long_decode_128k_b4_16q8kv", batch=4, n_q_heads=16,
                                  n_kv_heads=8, dtype="bf16", k_outliers=True,
                                  shuffle_pages=True, seed=4004, context=131072)
CHUNKED_PREFILL = PrefillWorkload("chunked_prefill_32k_512q_64q8kv", n_kv_heads=8,
                                  n_q_heads=64, cached=24576, appended=8192,
                                  n_queries=512, dtype="bf16", seed=5005)

DECODE_WORKLOADS = {w.name: w for w in (TINY_DECODE, GQA_DECODE_32K, RAGGED_DECODE,
                                        LONG_DECODE_128K)}
