"""Thin Python binding of libisoquant (ctypes).

Argument marshalling only: every step of the path runs in the HIP kernels of
``libisoquant.so``.  PyTorch provides device memory and streams.  Importing
this module loads the library and raises if it has not been built (there is
no fallback path).
"""

from __future__ import annotations

import ctypes
import os

import numpy as np
import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
# ISOQUANT_LIB may name another build of the same library (e.g. a profiling build).
LIB_PATH = os.environ.get("ISOQUANT_LIB") or os.path.join(_HERE, "libisoquant.so")

HEAD_DIM = 128
PAGE_TOKENS = 64
CODE_BYTES = 48
CODE_BYTES4 = 64
MAX_GROUP = 16

IQ_F32, IQ_BF16, IQ_F16 = 0, 1, 2
_DTYPES = {torch.float32: IQ_F32, torch.bfloat16: IQ_BF16, torch.float16: IQ_F16}


class IsoQuantError(RuntimeError):
    def __init__(self, fn: str, status: int, text: str):
        super().__init__(f"{fn}: {text} (status {status})")
        self.status = status


class IqCacheStruct(ctypes.Structure):
    _fields_ = [
        ("k_codes_dev", ctypes.c_void_p),
        ("k_norms_dev", ctypes.c_void_p),
        ("v_codes_dev", ctypes.c_void_p),
        ("v_norms_dev", ctypes.c_void_p),
        ("num_pages", ctypes.c_int32),
        ("n_kv_heads", ctypes.c_int32),
        ("bits", ctypes.c_int32),
    ]


IQ_KV_BF16, IQ_KV_FP8_E4M3 = 0, 1


class IqDenseCacheStruct(ctypes.Structure):
    _fields_ = [
        ("k_dev", ctypes.c_void_p),
        ("v_dev", ctypes.c_void_p),
        ("num_pages", ctypes.c_int32),
        ("n_kv_heads", ctypes.c_int32),
        ("format", ctypes.c_int32),
        ("k_scale", ctypes.c_float),
        ("v_scale", ctypes.c_float),
    ]


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it with "
                          "`python -m compressed_space_attention_amd.build`")
    lib = ctypes.CDLL(LIB_PATH)
    vp, i32, f32, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_float, ctypes.c_size_t
    cp = ctypes.POINTER(IqCacheStruct)
    dp = ctypes.POINTER(IqDenseCacheStruct)
    sigs = {
        "iq_status_string": (ctypes.c_char_p, [i32]),
        "iq_version": (i32, []),
        "iq_codebook": (i32, [i32, vp, vp, vp]),
        "iq_rotation_bytes": (sz, [i32]),
        "iq_rotation_init": (i32, [vp, i32, vp, sz, vp]),
        "iq_quantize_append": (i32, [cp, vp, vp, vp, i32, i32, vp, vp, vp, i32, vp]),
        "iq_decode_workspace_bytes": (sz, [i32, i32, i32, i32]),
        "iq_decode_attention": (i32, [cp, vp, vp, i32, i32, i32, vp, i32, vp, i32, f32, vp, vp, sz, vp]),
        "iq_decode_step": (i32, [cp, vp, vp, i32, i32, i32, vp, vp, i32, vp, i32, vp, i32, f32, vp, vp,
                                 sz, vp]),
        "iq_dense_append": (i32, [dp, vp, vp, i32, i32, vp, vp, vp, i32, vp]),
        "iq_dense_decode_workspace_bytes": (sz, [i32, i32, i32, i32]),
        "iq_dense_decode_attention": (i32, [dp, vp, i32, i32, i32, vp, i32, vp, i32, f32, vp, vp, sz, vp]),
        "iq_dense_prefill_attention": (i32, [dp, vp, i32, i32, i32, i32, vp, i32, f32, vp, vp]),
        "iq_probe_sink_bytes": (sz, []),
        "iq_probe_read": (i32, [vp, sz, vp, sz, vp]),
        "iq_prefill_workspace_bytes": (sz, [i32, i32, i32, i32]),
        "iq_prefill_attention_varlen": (i32, [cp, vp, vp, i32, i32, i32, i32, vp, vp, i32, i32, vp, i32, f32,
                                              vp, vp, sz, vp]),
        "iq_prefill_attention": (i32, [cp, vp, vp, i32, i32, i32, i32, vp, i32, f32, vp, vp, sz, vp]),
    }
    for name, (res, args) in sigs.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    return lib


lib = _load()
EXPORTED = ("iq_status_string", "iq_version", "iq_codebook", "iq_rotation_bytes", "iq_rotation_init",
            "iq_quantize_append", "iq_decode_workspace_bytes", "iq_decode_attention",
            "iq_decode_step", "iq_prefill_workspace_bytes", "iq_prefill_attention",
            "iq_prefill_attention_varlen",
            "iq_dense_append", "iq_dense_decode_workspace_bytes", "iq_dense_decode_attention",
            "iq_dense_prefill_attention",
            "iq_probe_sink_bytes", "iq_probe_read")


def status_string(status: int) -> str:
    return lib.iq_status_string(status).decode()


def _check(fn: str, status: int):
    if status != 0:
        raise IsoQuantError(fn, status, status_string(status))


def _ptr(t) -> int | None:
    return None if t is None else t.data_ptr()


def _stream(stream) -> int | None:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream if torch.cuda.is_available() else None
    return stream if isinstance(stream, int) else stream.cuda_stream


def _dtype(t: torch.Tensor) -> int:
    if t.dtype not in _DTYPES:
        raise TypeError(f"unsupported dtype {t.dtype}")
    return _DTYPES[t.dtype]


def _contig(t: torch.Tensor, name: str) -> torch.Tensor:
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t


def codebook(bits: int):
    """(levels float64[2^bits], thresholds float32[2^bits - 1], alpha) of the
    library's quantiser for 3- or 4-bit records (host only)."""
    levels = np.zeros(1 << bits, dtype=np.float64)
    thr = np.zeros((1 << bits) - 1, dtype=np.float32)
    alpha = ctypes.c_float(0.0)
    _check("iq_codebook", lib.iq_codebook(bits, levels.ctypes.data, thr.ctypes.data,
                                          ctypes.addressof(alpha)))
    return levels, thr, float(alpha.value)


class PagedCache:
    """One layer's packed cache in caller-owned torch device memory.

    k_codes/v_codes: uint8[num_pages][Hkv][64][48] (bits=3) or [..][64] (bits=4);
    k_norms/v_norms: int16 holding fp16 bit patterns [num_pages][Hkv][64]."""

    def __init__(self, num_pages: int, n_kv_heads: int, device="cuda", zero: bool = False,
                 bits: int = 3):
        if bits not in (3, 4):
            raise ValueError("bits must be 3 or 4")
        alloc = torch.zeros if zero else torch.empty
        self.num_pages, self.n_kv_heads, self.bits = int(num_pages), int(n_kv_heads), int(bits)
        rec = CODE_BYTES if bits == 3 else CODE_BYTES4
        shp = (self.num_pages, self.n_kv_heads, PAGE_TOKENS)
        self.k_codes = alloc(shp + (rec,), dtype=torch.uint8, device=device)
        self.v_codes = alloc(shp + (rec,), dtype=torch.uint8, device=device)
        self.k_norms = alloc(shp, dtype=torch.int16, device=device)
        self.v_norms = alloc(shp, dtype=torch.int16, device=device)
        self._struct = IqCacheStruct(self.k_codes.data_ptr(), self.k_norms.data_ptr(),
                                     self.v_codes.data_ptr(), self.v_norms.data_ptr(),
                                     self.num_pages, self.n_kv_heads, self.bits)

    @property
    def struct(self):
        return ctypes.byref(self._struct)

    def nbytes(self) -> int:
        return sum(t.numel() * t.element_size() for t in
                   (self.k_codes, self.v_codes, self.k_norms, self.v_norms))

    def to_host(self):
        """(k_codes, k_norms uint16, v_codes, v_norms uint16) as numpy arrays."""
        return (self.k_codes.cpu().numpy(), self.k_norms.cpu().numpy().view(np.uint16),
                self.v_codes.cpu().numpy(), self.v_norms.cpu().numpy().view(np.uint16))


def rotation_bytes(n_kv_heads: int) -> int:
    return int(lib.iq_rotation_bytes(n_kv_heads))


def rotation_init(quats, device="cuda", stream=None) -> torch.Tensor:
    """quats: host float32 [Hkv][32][2][4] -> device rotation buffer (uint8 tensor)."""
    q = np.ascontiguousarray(np.asarray(quats, dtype=np.float32))
    hkv = q.shape[0]
    if q.shape != (hkv, 32, 2, 4):
        raise ValueError("quaternions must be [Hkv][32][2][4]")
    rot = torch.empty(rotation_bytes(hkv), dtype=torch.uint8, device=device)
    _check("iq_rotation_init", lib.iq_rotation_init(q.ctypes.data, hkv, rot.data_ptr(), rot.numel(),
                                                    _stream(stream)))
    return rot


def quantize_append(cache: PagedCache, rot: torch.Tensor, k: torch.Tensor, v: torch.Tensor,
                    seq_idx: torch.Tensor, pos: torch.Tensor, block_table: torch.Tensor, stream=None):
    """k, v: [n_tokens][Hkv][128] (f32/bf16/f16); seq_idx, pos: int32[n_tokens];
    block_table: int32[n_seqs][max_pages]."""
    if k.shape != v.shape or k.dtype != v.dtype or k.dim() != 3 or k.shape[2] != HEAD_DIM:
        raise ValueError("k and v must both be [n_tokens][Hkv][128] of one dtype")
    if k.shape[1] != cache.n_kv_heads:
        raise ValueError("kv head count differs from the cache")
    n = k.shape[0]
    _check("iq_quantize_append", lib.iq_quantize_append(
        cache.struct, rot.data_ptr(), _contig(k, "k").data_ptr(), _contig(v, "v").data_ptr(),
        _dtype(k), n, _ptr(_contig(seq_idx, "seq_idx")), _ptr(_contig(pos, "pos")),
        _ptr(_contig(block_table, "block_table")), block_table.shape[-1], _stream(stream)))


def decode_workspace_bytes(batch: int, n_q_heads: int, n_kv_heads: int, max_seq_len: int) -> int:
    return int(lib.iq_decode_workspace_bytes(batch, n_q_heads, n_kv_heads, max_seq_len))


def decode_attention(cache: PagedCache, rot: torch.Tensor, q: torch.Tensor, block_table: torch.Tensor,
                     seq_lens: torch.Tensor, max_seq_len: int, softmax_scale: float = 0.0,
                     out: torch.Tensor | None = None, workspace: torch.Tensor | None = None,
                     stream=None) -> torch.Tensor:
    """q: [B][Hq][128]; block_table int32[B][max_pages]; seq_lens int32[B] -> fp32 [B][Hq][128]."""
    bsz, hq, d = q.shape
    if d != HEAD_DIM:
        raise ValueError("head dim must be 128")
    if out is None:
        out = torch.empty((bsz, hq, HEAD_DIM), dtype=torch.float32, device=q.device)
    if workspace is None:
        nbytes = decode_workspace_bytes(bsz, hq, cache.n_kv_heads, max_seq_len)
        workspace = torch.empty(max(nbytes, 16), dtype=torch.uint8, device=q.device)
    _check("iq_decode_attention", lib.iq_decode_attention(
        cache.struct, rot.data_ptr(), _contig(q, "q").data_ptr(), _dtype(q), bsz, hq,
        _contig(block_table, "block_table").data_ptr(), block_table.shape[-1],
        _contig(seq_lens, "seq_lens").data_ptr(), int(max_seq_len), float(softmax_scale),
        out.data_ptr(), workspace.data_ptr(), workspace.numel() * workspace.element_size(),
        _stream(stream)))
    return out


def decode_step(cache: PagedCache, rot: torch.Tensor, q: torch.Tensor, k_new: torch.Tensor,
                v_new: torch.Tensor, block_table: torch.Tensor, seq_lens: torch.Tensor, max_seq_len: int,
                softmax_scale: float = 0.0, out: torch.Tensor | None = None,
                workspace: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """Append each sequence's current token (k_new, v_new: [B][Hkv][128], at position
    seq_lens[b] - 1) and run decode attention over all seq_lens[b] tokens, in one call."""
    bsz, hq, d = q.shape
    if d != HEAD_DIM:
        raise ValueError("head dim must be 128")
    if (k_new.shape != v_new.shape or k_new.dtype != v_new.dtype
            or tuple(k_new.shape) != (bsz, cache.n_kv_heads, HEAD_DIM)):
        raise ValueError("k_new and v_new must both be [B][Hkv][128] of one dtype")
    if out is None:
        out = torch.empty((bsz, hq, HEAD_DIM), dtype=torch.float32, device=q.device)
    if workspace is None:
        nbytes = decode_workspace_bytes(bsz, hq, cache.n_kv_heads, max_seq_len)
        workspace = torch.empty(max(nbytes, 16), dtype=torch.uint8, device=q.device)
    _check("iq_decode_step", lib.iq_decode_step(
        cache.struct, rot.data_ptr(), _contig(q, "q").data_ptr(), _dtype(q), bsz, hq,
        _contig(k_new, "k_new").data_ptr(), _contig(v_new, "v_new").data_ptr(), _dtype(k_new),
        _contig(block_table, "block_table").data_ptr(), block_table.shape[-1],
        _contig(seq_lens, "seq_lens").data_ptr(), int(max_seq_len), float(softmax_scale),
        out.data_ptr(), workspace.data_ptr(), workspace.numel() * workspace.element_size(),
        _stream(stream)))
    return out


def prefill_workspace_bytes(n_q: int, n_q_heads: int, n_kv_heads: int, q_start: int) -> int:
    return int(lib.iq_prefill_workspace_bytes(n_q, n_q_heads, n_kv_heads, q_start))


def prefill_attention(cache: PagedCache, rot: torch.Tensor, q: torch.Tensor, q_start: int,
                      block_table: torch.Tensor, softmax_scale: float = 0.0,
                      out: torch.Tensor | None = None, workspace: torch.Tensor | None = None,
                      stream=None) -> torch.Tensor:
    """q: [n_q][Hq][128] at positions q_start..; block_table int32[max_pages] -> fp32 [n_q][Hq][128]."""
    n_q, hq, d = q.shape
    if d != HEAD_DIM:
        raise ValueError("head dim must be 128")
    if out is None:
        out = torch.empty((n_q, hq, HEAD_DIM), dtype=torch.float32, device=q.device)
    need = prefill_workspace_bytes(max(n_q, 1), hq, cache.n_kv_heads, q_start)
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    ws_ptr = _ptr(workspace)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check("iq_prefill_attention", lib.iq_prefill_attention(
        cache.struct, rot.data_ptr(), _contig(q, "q").data_ptr(), _dtype(q), n_q, hq, int(q_start),
        _contig(block_table, "block_table").data_ptr(), block_table.shape[-1], float(softmax_scale),
        out.data_ptr(), ws_ptr, ws_bytes, _stream(stream)))
    return out


def prefill_attention_varlen(cache: PagedCache, rot: torch.Tensor, q: torch.Tensor, cu_q: torch.Tensor,
                             q_start: torch.Tensor, block_table: torch.Tensor, max_q_per_seq: int,
                             max_kv_len: int, softmax_scale: float = 0.0,
                             out: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """q: [total_q][Hq][128]; cu_q int32[B+1], q_start int32[B] (device);
    block_table int32[B][max_pages] -> fp32 [total_q][Hq][128]."""
    total_q, hq, d = q.shape
    if d != HEAD_DIM:
        raise ValueError("head dim must be 128")
    bsz = cu_q.numel() - 1
    if out is None:
        out = torch.zeros((total_q, hq, HEAD_DIM), dtype=torch.float32, device=q.device)
    _check("iq_prefill_attention_varlen", lib.iq_prefill_attention_varlen(
        cache.struct, rot.data_ptr(), _contig(q, "q").data_ptr(), _dtype(q), bsz, hq, total_q,
        _contig(cu_q, "cu_q").data_ptr(), _contig(q_start, "q_start").data_ptr(), int(max_q_per_seq),
        int(max_kv_len), _contig(block_table, "block_table").data_ptr(), block_table.shape[-1],
        float(softmax_scale), out.data_ptr(), None, 0, _stream(stream)))
    return out


# ---------------------------------------------------------------------------
# Uncompressed bf16 baseline and the HBM read probe.
# ---------------------------------------------------------------------------
class DenseCache:
    """One layer's uncompressed paged cache: k[num_pages][Hkv][64][128]
    (token-major), v[num_pages][Hkv][128][64] (coordinate-major); format "bf16"
    (bf16 bits as int16) or "fp8" (OCP E4M3 bytes as uint8, holding x / scale)."""

    def __init__(self, num_pages: int, n_kv_heads: int, device="cuda", zero: bool = False,
                 format: str = "bf16", k_scale: float = 1.0, v_scale: float = 1.0):
        if format not in ("bf16", "fp8"):
            raise ValueError("format must be 'bf16' or 'fp8'")
        alloc = torch.zeros if zero else torch.empty
        self.num_pages, self.n_kv_heads, self.format = int(num_pages), int(n_kv_heads), format
        dt = torch.int16 if format == "bf16" else torch.uint8
        self.k = alloc((self.num_pages, self.n_kv_heads, PAGE_TOKENS, HEAD_DIM), dtype=dt, device=device)
        self.v = alloc((self.num_pages, self.n_kv_heads, HEAD_DIM, PAGE_TOKENS), dtype=dt, device=device)
        self._struct = IqDenseCacheStruct(self.k.data_ptr(), self.v.data_ptr(), self.num_pages,
                                          self.n_kv_heads,
                                          IQ_KV_BF16 if format == "bf16" else IQ_KV_FP8_E4M3,
                                          float(k_scale), float(v_scale))

    @property
    def struct(self):
        return ctypes.byref(self._struct)

    def nbytes(self) -> int:
        return self.k.element_size() * (self.k.numel() + self.v.numel())


def dense_append(cache: DenseCache, k: torch.Tensor, v: torch.Tensor, seq_idx: torch.Tensor,
                 pos: torch.Tensor, block_table: torch.Tensor, stream=None):
    if k.shape != v.shape or k.dtype != v.dtype or k.dim() != 3 or k.shape[2] != HEAD_DIM:
        raise ValueError("k and v must both be [n_tokens][Hkv][128] of one dtype")
    if k.shape[1] != cache.n_kv_heads:
        raise ValueError("kv head count differs from the cache")
    _check("iq_dense_append", lib.iq_dense_append(
        cache.struct, _contig(k, "k").data_ptr(), _contig(v, "v").data_ptr(), _dtype(k), k.shape[0],
        _ptr(_contig(seq_idx, "seq_idx")), _ptr(_contig(pos, "pos")),
        _ptr(_contig(block_table, "block_table")), block_table.shape[-1], _stream(stream)))


def dense_decode_workspace_bytes(batch: int, n_q_heads: int, n_kv_heads: int, max_seq_len: int) -> int:
    return int(lib.iq_dense_decode_workspace_bytes(batch, n_q_heads, n_kv_heads, max_seq_len))


def dense_decode_attention(cache: DenseCache, q: torch.Tensor, block_table: torch.Tensor,
                           seq_lens: torch.Tensor, max_seq_len: int, softmax_scale: float = 0.0,
                           out: torch.Tensor | None = None, workspace: torch.Tensor | None = None,
                           stream=None) -> torch.Tensor:
    """q: bf16 [B][Hq][128] -> fp32 [B][Hq][128] over the bf16 cache."""
    bsz, hq, d = q.shape
    if d != HEAD_DIM:
        raise ValueError("head dim must be 128")
    if out is None:
        out = torch.empty((bsz, hq, HEAD_DIM), dtype=torch.float32, device=q.device)
    if workspace is None:
        nbytes = dense_decode_workspace_bytes(bsz, hq, cache.n_kv_heads, max_seq_len)
        workspace = torch.empty(max(nbytes, 16), dtype=torch.uint8, device=q.device)
    _check("iq_dense_decode_attention", lib.iq_dense_decode_attention(
        cache.struct, _contig(q, "q").data_ptr(), _dtype(q), bsz, hq,
        _contig(block_table, "block_table").data_ptr(), block_table.shape[-1],
        _contig(seq_lens, "seq_lens").data_ptr(), int(max_seq_len), float(softmax_scale),
        out.data_ptr(), workspace.data_ptr(), workspace.numel() * workspace.element_size(),
        _stream(stream)))
    return out


def dense_prefill_attention(cache: DenseCache, q: torch.Tensor, q_start: int, block_table: torch.Tensor,
                            softmax_scale: float = 0.0, out: torch.Tensor | None = None,
                            stream=None) -> torch.Tensor:
    """q: bf16 [n_q][Hq][128] at positions q_start..; block_table int32[max_pages]
    -> fp32 [n_q][Hq][128] over the bf16 / FP8 cache."""
    n_q, hq, d = q.shape
    if d != HEAD_DIM:
        raise ValueError("head dim must be 128")
    if out is None:
        out = torch.empty((n_q, hq, HEAD_DIM), dtype=torch.float32, device=q.device)
    _check("iq_dense_prefill_attention", lib.iq_dense_prefill_attention(
        cache.struct, _contig(q, "q").data_ptr(), _dtype(q), n_q, hq, int(q_start),
        _contig(block_table, "block_table").data_ptr(), block_table.shape[-1], float(softmax_scale),
        out.data_ptr(), _stream(stream)))
    return out


def probe_sink_bytes() -> int:
    return int(lib.iq_probe_sink_bytes())


def probe_read(buf: torch.Tensor, sink: torch.Tensor, stream=None):
    """Stream `buf` (contiguous, size a multiple of 16 bytes) once on the GPU."""
    nbytes = buf.numel() * buf.element_size()
    _check("iq_probe_read", lib.iq_probe_read(_contig(buf, "buf").data_ptr(), nbytes, sink.data_ptr(),
                                              sink.numel() * sink.element_size(), _stream(stream)))
