"""C-ABI checks that need no GPU: the library loads, exports every function
include/isoquant.h declares, and rejects bad arguments on the host before
anything is enqueued (no compute call is made here)."""

import ctypes
import os
import re

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "isoquant.h")

iq = pytest.importorskip("compressed_space_attention_amd.isoquant",
                         reason="libisoquant.so not built")
L = iq.lib
FAKE = 0x1000  # never dereferenced: every call below fails validation first


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(iq_[a-z_]+)\s*\(", text)))


def test_header_declarations_are_exported_and_bound():
    names = declared_functions()
    assert len(names) >= 9
    for n in names:
        assert hasattr(L, n), n                    # dlsym succeeds
    assert sorted(iq.EXPORTED) == names


def test_status_strings_and_sizes():
    for code, text in [(0, "ok"), (-1, "invalid argument"), (-2, "unsupported configuration"),
                       (-3, "workspace too small"), (-4, "HIP copy or kernel launch failed"),
                       (-5, "no usable HIP device"),
                       (-6, "call needs more scratch than the library's static array holds")]:
        assert iq.status_string(code) == text
    assert iq.status_string(7) == "unknown status"
    assert L.iq_version() == 10000
    assert iq.rotation_bytes(8) == 8 * (32 * 16 + 32 * 8) * 4
    assert iq.rotation_bytes(0) == 0
    assert iq.decode_workspace_bytes(0, 32, 4, 1024) == 0


def _cache(hkv=4, pages=8, bits=0):
    return ctypes.byref(iq.IqCacheStruct(FAKE, FAKE, FAKE, FAKE, pages, hkv, bits))


def test_rotation_init_validation():
    q = np.ones((2, 32, 2, 4), np.float32)
    assert L.iq_rotation_init(None, 2, FAKE, 10 ** 6, None) == -1
    assert L.iq_rotation_init(q.ctypes.data, 0, FAKE, 10 ** 6, None) == -1
    assert L.iq_rotation_init(q.ctypes.data, 2, FAKE, 100, None) == -1       # buffer too small
    bad = q.copy()
    bad[1, 5, 1] = 0.0                                                        # zero quaternion
    assert L.iq_rotation_init(bad.ctypes.data, 2, FAKE, 10 ** 6, None) == -1
    bad = q.copy()
    bad[0, 0, 0, 2] = np.nan
    assert L.iq_rotation_init(bad.ctypes.data, 2, FAKE, 10 ** 6, None) == -1


def test_quantize_append_validation():
    c = _cache()
    assert L.iq_quantize_append(None, FAKE, FAKE, FAKE, 1, 4, FAKE, FAKE, FAKE, 8, None) == -1
    assert L.iq_quantize_append(c, FAKE, FAKE, FAKE, 7, 4, FAKE, FAKE, FAKE, 8, None) == -1  # dtype
    assert L.iq_quantize_append(c, FAKE, FAKE, FAKE, 1, -1, FAKE, FAKE, FAKE, 8, None) == -1
    assert L.iq_quantize_append(c, FAKE, None, FAKE, 1, 4, FAKE, FAKE, FAKE, 8, None) == -1
    assert L.iq_quantize_append(c, FAKE, FAKE, FAKE, 1, 0, FAKE, FAKE, FAKE, 8, None) == 0   # no-op
    empty = ctypes.byref(iq.IqCacheStruct(FAKE, FAKE, FAKE, FAKE, 0, 4))
    assert L.iq_quantize_append(empty, FAKE, FAKE, FAKE, 1, 4, FAKE, FAKE, FAKE, 8, None) == -1
    for bad_bits in (1, 2, 5, 8, -3):                      # record width neither 3 nor 4
        bad = _cache(bits=bad_bits)
        assert L.iq_quantize_append(bad, FAKE, FAKE, FAKE, 1, 0, FAKE, FAKE, FAKE, 8, None) == -1
        assert _decode(bad) == -1


def _decode(c, hq=32, ws=10 ** 9, dtype=1, max_len=1024, max_pages=16, batch=1):
    return L.iq_decode_attention(c, FAKE, FAKE, dtype, batch, hq, FAKE, max_pages, FAKE, max_len,
                                 0.0, FAKE, FAKE, ws, None)


def test_decode_validation():
    c = _cache(hkv=4)
    assert _decode(c, hq=30) == -1                  # Hq not a multiple of Hkv
    assert _decode(c, dtype=5) == -1
    assert _decode(c, max_len=2000, max_pages=16) == -1   # lengths exceed the block table
    assert _decode(c, hq=4 * 17) == -2              # group above IQ_MAX_GROUP
    assert _decode(c, ws=16) == -3                  # workspace too small
    assert _decode(c, batch=0) == -1
    assert L.iq_decode_attention(c, FAKE, FAKE, 1, 1, 32, None, 16, FAKE, 1024, 0.0, FAKE, FAKE,
                                 10 ** 9, None) == -1


def _step(c, hq=32, ws=10 ** 9, dtype=1, kv_dtype=1, max_len=1024, max_pages=16, batch=1,
          k_new=FAKE, v_new=FAKE):
    return L.iq_decode_step(c, FAKE, FAKE, dtype, batch, hq, k_new, v_new, kv_dtype, FAKE, max_pages,
                            FAKE, max_len, 0.0, FAKE, FAKE, ws, None)


def test_decode_step_validation():
    c = _cache(hkv=4)
    assert _step(c, hq=30) == -1
    assert _step(c, kv_dtype=3) == -1               # bad dtype of the appended rows
    assert _step(c, k_new=None) == -1
    assert _step(c, v_new=None) == -1
    assert _step(c, max_len=2000, max_pages=16) == -1
    assert _step(c, hq=4 * 17) == -2
    assert _step(c, ws=16) == -3
    assert _step(None) == -1


def test_codebook_validation():
    lv = np.zeros(16)
    th = np.zeros(15, np.float32)
    for bits in (0, 2, 5):
        assert L.iq_codebook(bits, lv.ctypes.data, th.ctypes.data, None) == -1
    assert L.iq_codebook(4, None, th.ctypes.data, None) == -1
    assert L.iq_codebook(4, lv.ctypes.data, None, None) == -1
    assert L.iq_codebook(4, lv.ctypes.data, th.ctypes.data, None) == 0


def test_decode_workspace_is_monotone_in_context():
    a = iq.decode_workspace_bytes(1, 32, 4, 4096)
    b = iq.decode_workspace_bytes(1, 32, 4, 32768)
    assert 0 < a <= b


def test_prefill_validation():
    c = _cache(hkv=8)
    args = dict()
    assert L.iq_prefill_attention(c, FAKE, FAKE, 1, 16, 60, 0, FAKE, 8, 0.0, FAKE, FAKE, 0, None) == -1
    assert L.iq_prefill_attention(c, FAKE, FAKE, 1, 16, 24, 0, FAKE, 8, 0.0, FAKE, FAKE, 0, None) == -2
    assert L.iq_prefill_attention(c, FAKE, FAKE, 1, 16, 64, 500, FAKE, 8, 0.0, FAKE, FAKE, 0, None) == -1
    assert L.iq_prefill_attention(c, FAKE, FAKE, 1, 0, 64, 0, FAKE, 8, 0.0, FAKE, FAKE, 0, None) == 0
    assert L.iq_prefill_attention(c, FAKE, FAKE, 9, 16, 64, 0, FAKE, 8, 0.0, FAKE, FAKE, 0, None) == -1
    c4 = _cache(hkv=8, bits=4)                  # the same checks on a 4-bit cache
    assert L.iq_prefill_attention(c4, FAKE, FAKE, 1, 16, 24, 0, FAKE, 8, 0.0, FAKE, FAKE, 0, None) == -2
    assert L.iq_prefill_attention(c4, FAKE, FAKE, 1, 0, 64, 0, FAKE, 8, 0.0, FAKE, FAKE, 0, None) == 0
    c5 = _cache(hkv=8, bits=5)
    assert L.iq_prefill_attention(c5, FAKE, FAKE, 1, 16, 64, 0, FAKE, 8, 0.0, FAKE, FAKE, 0, None) == -1
    # the page-table staging limit: a causal range of 4,096 pages (262,144 tokens)
    # at most; one token more is refused as unsupported, on either record width
    for cc in (c, c4):
        assert L.iq_prefill_attention(cc, FAKE, FAKE, 1, 32, 64, 262144 - 31, FAKE, 4097, 0.0, FAKE, FAKE, 0,
                                      None) == -2


def test_dense_and_probe_validation():
    dc = ctypes.byref(iq.IqDenseCacheStruct(FAKE, FAKE, 8, 4, 0, 0.0, 0.0))
    for fmt, ks, vs in [(2, 1.0, 1.0), (-1, 1.0, 1.0), (1, -1.0, 1.0), (1, 1.0, float("nan")),
                        (1, float("inf"), 1.0)]:            # unknown format, bad FP8 scales
        bad = ctypes.byref(iq.IqDenseCacheStruct(FAKE, FAKE, 8, 4, fmt, ks, vs))
        assert L.iq_dense_append(bad, FAKE, FAKE, 1, 0, FAKE, FAKE, FAKE, 8, None) == -1
    f8 = ctypes.byref(iq.IqDenseCacheStruct(FAKE, FAKE, 8, 4, 1, 0.0, 2.5))   # 0 selects 1
    assert L.iq_dense_append(f8, FAKE, FAKE, 1, 0, FAKE, FAKE, FAKE, 8, None) == 0

    def pre(c=dc, dtype=1, n_q=16, hq=32, q_start=0, max_pages=8):
        return L.iq_dense_prefill_attention(c, FAKE, dtype, n_q, hq, q_start, FAKE, max_pages, 0.0, FAKE, None)
    assert pre(hq=30) == -1                   # Hq not a multiple of Hkv
    assert pre(q_start=500) == -1             # beyond the block table
    assert pre(dtype=0) == -2                 # q must be bf16
    assert pre(hq=4 * 3) == -2                # group 3 not a power of two
    assert pre(n_q=0) == 0                    # no-op
    assert pre(c=f8, n_q=0) == 0
    assert pre(n_q=64, q_start=300000, max_pages=5000) == -2   # beyond the staging limit
    assert L.iq_dense_append(None, FAKE, FAKE, 1, 4, FAKE, FAKE, FAKE, 8, None) == -1
    assert L.iq_dense_append(dc, FAKE, FAKE, 7, 4, FAKE, FAKE, FAKE, 8, None) == -1
    assert L.iq_dense_append(dc, FAKE, FAKE, 1, 0, FAKE, FAKE, FAKE, 8, None) == 0

    def dec(hq=32, dtype=1, ws=10 ** 9, max_len=1024):
        return L.iq_dense_decode_attention(dc, FAKE, dtype, 1, hq, FAKE, 16, FAKE, max_len, 0.0, FAKE,
                                           FAKE, ws, None)
    assert dec(hq=30) == -1
    assert dec(max_len=2000) == -1
    assert dec(dtype=0) == -2          # q must be bf16
    assert dec(hq=4 * 17) == -2
    assert dec(ws=16) == -3
    assert iq.probe_sink_bytes() > 0
    assert L.iq_probe_read(FAKE, 24, FAKE, 10 ** 9, None) == -1        # not a multiple of 16
    assert L.iq_probe_read(FAKE, 0, FAKE, 10 ** 9, None) == -1
    assert L.iq_probe_read(FAKE, 64, FAKE, 16, None) == -1             # sink too small


def test_prefill_varlen_validation():
    c = _cache(hkv=8)

    def call(batch=2, hq=64, total_q=100, max_q=60, max_kv=500, max_pages=8, dtype=1, cu=FAKE):
        return L.iq_prefill_attention_varlen(c, FAKE, FAKE, dtype, batch, hq, total_q, cu, FAKE, max_q,
                                             max_kv, FAKE, max_pages, 0.0, FAKE, None, 0, None)
    assert call(hq=60) == -1                 # Hq not a multiple of Hkv
    assert call(hq=24) == -2                 # group 3 not a power of two
    assert call(max_kv=600) == -1            # beyond the block table
    assert call(max_q=120) == -1             # more queries per sequence than in total
    assert call(max_q=600, max_kv=500) == -1  # more queries than keys
    assert call(cu=None) == -1
    assert call(batch=0) == -1
    assert call(total_q=0, max_q=0) == 0     # no-op
    assert call(max_kv=300000, max_pages=5000) == -2   # beyond the staging limit


def test_binding_refuses_host_tensors():
    """The binding hands kernels device pointers only: a tensor in host memory
    (here every tensor: this check runs without a GPU) is refused before any
    call reaches the library."""
    import torch
    cache = iq.PagedCache(4, 2, device="cpu")
    rot = torch.zeros(iq.rotation_bytes(2), dtype=torch.uint8)
    q = torch.zeros((1, 4, 128), dtype=torch.bfloat16)
    bt = torch.zeros((1, 4), dtype=torch.int32)
    lens = torch.ones(1, dtype=torch.int32)
    kv = torch.zeros((1, 2, 128), dtype=torch.bfloat16)
    calls = [
        lambda: iq.decode_attention(cache, rot, q, bt, lens, 64),
        lambda: iq.decode_step(cache, rot, q, kv, kv, bt, lens, 64),
        lambda: iq.quantize_append(cache, rot, kv, kv, torch.zeros(1, dtype=torch.int32),
                                   torch.zeros(1, dtype=torch.int32), bt),
        lambda: iq.prefill_attention(cache, rot, q, 0, bt[0]),
        lambda: iq.probe_read(torch.zeros(16, dtype=torch.uint8), torch.zeros(16, dtype=torch.uint8)),
    ]
    for fn in calls:
        with pytest.raises(ValueError, match="GPU memory"):
            fn()


def test_decode_options_validation():
    """iq_decode_options: every field outside its values is refused on the host
    (and the workspace query returns 0 for it); valid options plan a workspace
    that starts with the counter region."""
    c = _cache(hkv=4)
    bad = [dict(waves=6), dict(waves=-4), dict(pages_per_split=-1), dict(rounds=-2), dict(rounds=65),
           dict(plan=3), dict(plan=-1), dict(merge=3), dict(merge=-1)]
    for kw in bad:
        o = iq.DecodeOptions(**kw)
        assert L.iq_decode_attention_ex(c, FAKE, FAKE, 1, 1, 32, FAKE, 16, FAKE, 1024, 0.0, FAKE, FAKE,
                                        10 ** 9, ctypes.byref(o), None) == -1, kw
        assert L.iq_decode_step_ex(c, FAKE, FAKE, 1, 1, 32, FAKE, FAKE, 1, FAKE, 16, FAKE, 1024, 0.0, FAKE,
                                   FAKE, 10 ** 9, ctypes.byref(o), None) == -1, kw
        assert iq.decode_workspace_bytes(1, 32, 4, 1024, o) == 0, kw
    good = [iq.DecodeOptions(), iq.DecodeOptions(waves=8, pages_per_split=3, rounds=2, plan=1, merge=2,
                                                 deterministic=1)]
    for o in good:
        n = iq.decode_workspace_bytes(2, 32, 4, 4096, o)
        # counters + at least one partial row (m, l, 128 accumulators) per query head
        assert n >= iq.DECODE_COUNTER_BYTES + 2 * 32 * 130 * 4
        # a too-small workspace is the only failure left
        assert L.iq_decode_attention_ex(c, FAKE, FAKE, 1, 2, 32, FAKE, 64, FAKE, 4096, 0.0, FAKE, FAKE,
                                        n - 1, ctypes.byref(o), None) == -3
    # a host plan of one-page splits needs one partial row per page and query head
    o = iq.DecodeOptions(plan=1, pages_per_split=1)
    assert iq.decode_workspace_bytes(2, 32, 4, 4096, o) == iq.DECODE_COUNTER_BYTES + 2 * 32 * 64 * 130 * 4


def test_prefill_options_validation():
    c = _cache(hkv=8)
    for w in (1, 2, 16, -4):
        o = iq.PrefillOptions(w)
        assert L.iq_prefill_attention_ex(c, FAKE, FAKE, 1, 16, 64, 0, FAKE, 8, 0.0, FAKE, FAKE, 0,
                                         ctypes.byref(o), None) == -1
    o = iq.PrefillOptions(4)
    assert L.iq_prefill_attention_ex(c, FAKE, FAKE, 1, 0, 64, 0, FAKE, 8, 0.0, FAKE, FAKE, 0,
                                     ctypes.byref(o), None) == 0


def _pa(c, k=FAKE, n_new=64, new_start=0, q=FAKE, n_q=16, hq=64, q_start=0, max_pages=8, ws=FAKE,
        ws_bytes=1 << 30, out=FAKE):
    return L.iq_prefill_append(c, FAKE, k, FAKE, 1, n_new, new_start, q, 1, n_q, hq, q_start, FAKE, max_pages,
                               0.0, out, ws, ws_bytes, None)


def test_prefill_append_validation():
    """The fused quantise-append + prefill refuses bad arguments on the host."""
    c = _cache(hkv=8)
    assert L.iq_prefill_append_workspace_bytes(16, 64, 8, 0) >= iq.DECODE_COUNTER_BYTES
    assert L.iq_prefill_append_workspace_bytes(0, 64, 8, 0) == iq.DECODE_COUNTER_BYTES
    assert L.iq_prefill_append_workspace_bytes(-1, 64, 8, 0) == 0
    assert _pa(c, k=None) == -1                       # rows missing for a non-empty chunk
    assert _pa(c, new_start=-1) == -1
    assert _pa(c, new_start=8 * 64 - 63) == -1        # the chunk runs past the block table
    assert _pa(c, q_start=8 * 64 - 15) == -1          # the queries run past it
    assert _pa(c, hq=60) == -1                        # not a multiple of the kv heads
    assert _pa(c, out=None) == -1
    assert _pa(c, ws=None) == -1
    assert _pa(c, ws_bytes=100) == -3                 # no room for the counters
    assert _pa(c, hq=8 * 3) == -2                     # a group of 3
    assert _pa(c, n_new=0, n_q=0, k=None, q=None, out=None) == 0   # nothing to do
    assert L.iq_prefill_append_launches(16, 64, 8, 5) == -1
    assert L.iq_prefill_append_launches(0, 64, 8, 3) == -1


def _noalloc(c, batch=1, hq=32, max_len=1024, max_pages=16, out=FAKE, k_new=FAKE):
    return L.iq_decode_step_noalloc(c, FAKE, FAKE, 1, batch, hq, k_new, FAKE, 1, FAKE, max_pages, FAKE,
                                    max_len, 0.0, out, None)


def test_decode_step_noalloc_validation():
    """The no-allocation decode step refuses bad arguments, and calls whose plan
    needs more than the static scratch, on the host before touching a device."""
    c = _cache(hkv=4)
    assert _noalloc(c, out=None) == -1
    assert _noalloc(c, k_new=None) == -1
    assert _noalloc(c, hq=30) == -1
    assert _noalloc(c, max_len=2000, max_pages=16) == -1
    assert _noalloc(c, hq=4 * 17) == -2
    big = _cache(hkv=16)
    need = iq.decode_workspace_bytes(64, 256, 16, 65536, iq.DecodeOptions(merge=iq.IQ_MERGE_KERNEL))
    assert need > iq.NOALLOC_SCRATCH_BYTES
    assert _noalloc(big, batch=64, hq=256, max_len=65536, max_pages=1024) == -6
