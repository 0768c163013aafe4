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
IQ_PLAN_AUTO, IQ_PLAN_HOST, IQ_PLAN_BALANCED = 0, 1, 2
IQ_MERGE_AUTO, IQ_MERGE_FUSED, IQ_MERGE_KERNEL = 0, 1, 2
DECODE_COUNTER_BYTES = 16384


class DecodeOptions(ctypes.Structure):
    """iq_decode_options: zero fields leave the choice to the planner."""
    _fields_ = [
        ("waves", ctypes.c_int32),
        ("pages_per_split", ctypes.c_int32),
        ("rounds", ctypes.c_int32),
        ("plan", ctypes.c_int32),
        ("merge", ctypes.c_int32),
        ("deterministic", ctypes.c_int32),
    ]


class DecodePlanInfo(ctypes.Structure):
    _fields_ = [
        ("waves", ctypes.c_int32),
        ("splits", ctypes.c_int32),
        ("pages_per_split", ctypes.c_int32),
        ("balanced", ctypes.c_int32),
        ("fused_merge", ctypes.c_int32),
        ("workgroups", ctypes.c_int32),
    ]


class PrefillOptions(ctypes.Structure):
    _fields_ = [("waves", ctypes.c_int32)]


def _opts(options):
    return None if options is None else ctypes.byref(options)


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
    op = ctypes.POINTER(DecodeOptions)
    pp = ctypes.POINTER(PrefillOptions)
    sigs = {
        "iq_status_string": (ctypes.c_char_p, [i32]),
        "iq_version": (i32, []),
        "iq_codebook": (i32, [i32, vp, vp, vp]),
        "iq_rotation_bytes": (sz, [i32]),
        "iq_rotation_init": (i32, [vp, i32, vp, sz, vp]),
        "iq_quantize_append": (i32, [cp, vp, vp, vp, i32, i32, vp, vp, vp, i32, vp]),
        "iq_decode_workspace_bytes": (sz, [i32, i32, i32, i32]),
        "iq_decode_workspace_bytes_ex": (sz, [i32, i32, i32, i32, op]),
        "iq_decode_describe": (i32, [i32, i32, i32, i32, i32, i32, op, ctypes.POINTER(DecodePlanInfo)]),
        "iq_decode_attention": (i32, [cp, vp, vp, i32, i32, i32, vp, i32, vp, i32, f32, vp, vp, sz, vp]),
        "iq_decode_attention_ex": (i32, [cp, vp, vp, i32, i32, i32, vp, i32, vp, i32, f32, vp, vp, sz, op,
                                         vp]),
        "iq_decode_step": (i32, [cp, vp, vp, i32, i32, i32, vp, vp, i32, vp, i32, vp, i32, f32, vp, vp,
                                 sz, vp]),
        "iq_decode_step_ex": (i32, [cp, vp, vp, i32, i32, i32, vp, vp, i32, vp, i32, vp, i32, f32, vp, vp,
                                    sz, op, vp]),
        "iq_decode_step_noalloc": (i32, [cp, vp, vp, i32, i32, i32, vp, vp, i32, vp, i32, vp, i32, f32, vp,
                                         vp]),
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
        "iq_prefill_attention_ex": (i32, [cp, vp, vp, i32, i32, i32, i32, vp, i32, f32, vp, vp, sz, pp, vp]),
        "iq_prefill_append_workspace_bytes": (sz, [i32, i32, i32, i32]),
        "iq_prefill_append_launches": (i32, [i32, i32, i32, i32]),
        "iq_prefill_append": (i32, [cp, vp, vp, vp, i32, i32, i32, vp, i32, i32, i32, i32, vp, i32, f32, vp, vp,
                                    sz, vp]),
    }
    for name, (res, args) in sigs.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    return lib


lib = _load()
EXPORTED = ("iq_status_string", "iq_version", "iq_codebook", "iq_rotation_bytes", "iq_rotation_init",
            "iq_quantize_append", "iq_decode_workspace_bytes", "iq_decode_attention",
            "iq_decode_step", "iq_decode_workspace_bytes_ex", "iq_decode_attention_ex", "iq_decode_step_ex",
            "iq_decode_describe", "iq_decode_step_noalloc",
            "iq_prefill_workspace_bytes", "iq_prefill_attention", "iq_prefill_attention_ex",
            "iq_prefill_append_workspace_bytes", "iq_prefill_append_launches", "iq_prefill_append",
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


def _device_of(t: torch.Tensor, name: str) -> torch.device:
    """The GPU `t` lives on (the device every other operand must share)."""
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise ValueError(f"{name} must be a tensor in GPU memory")
    return t.device


def _dev(t: torch.Tensor, name: str, device: torch.device, dtype: torch.dtype | None = None) -> int:
    """Device pointer of a contiguous tensor on `device` (of `dtype` if given):
    a host tensor would hand a host address to a kernel, and an index tensor
    of another width would be misread."""
    if not isinstance(t, torch.Tensor) or not t.is_cuda or t.device != device:
        raise ValueError(f"{name} must be a tensor on {device}")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    return _contig(t, name).data_ptr()


def _idx(t: torch.Tensor, name: str, device: torch.device) -> int:
    return _dev(t, name, device, torch.int32)


def _check_cache(cache, device: torch.device):
    for name, t in cache.tensors():
        _dev(t, f"cache.{name}", device)


def _torch_stream(stream, device: torch.device):
    if stream is None:
        return None
    if isinstance(stream, int):
        return torch.cuda.ExternalStream(stream, device=device)
    return stream


def _alloc(shape, dtype, device: torch.device, stream, zero: bool = False) -> torch.Tensor:
    """A buffer owned by the caching allocator on the stream the kernels run
    on, so it is not handed out again while they may still use it."""
    fn = torch.zeros if zero else torch.empty
    s = _torch_stream(stream, device)
    if s is None:
        return fn(shape, dtype=dtype, device=device)
    with torch.cuda.stream(s):
        return fn(shape, dtype=dtype, device=device)


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

    def tensors(self):
        return (("k_codes", self.k_codes), ("k_norms", self.k_norms), ("v_codes", self.v_codes),
                ("v_norms", self.v_norms))

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
    dev = torch.device(device)
    if dev.type == "cuda" and dev.index is None:
        dev = torch.device("cuda", torch.cuda.current_device())
    rot = _alloc((rotation_bytes(hkv),), torch.uint8, dev, stream)
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
    dev = _device_of(k, "k")
    if seq_idx.numel() != n or pos.numel() != n:
        raise ValueError("seq_idx and pos must hold one entry per token")
    _check_cache(cache, dev)
    _check("iq_quantize_append", lib.iq_quantize_append(
        cache.struct, _dev(rot, "rot", dev), _dev(k, "k", dev), _dev(v, "v", dev), _dtype(k), n,
        _idx(seq_idx, "seq_idx", dev), _idx(pos, "pos", dev), _idx(block_table, "block_table", dev),
        block_table.shape[-1], _stream(stream)))


def decode_workspace_bytes(batch: int, n_q_heads: int, n_kv_heads: int, max_seq_len: int,
                           options: DecodeOptions | None = None) -> int:
    return int(lib.iq_decode_workspace_bytes_ex(batch, n_q_heads, n_kv_heads, max_seq_len, _opts(options)))


def decode_describe(batch: int, n_q_heads: int, n_kv_heads: int, max_seq_len: int, bits: int = 3,
                    step: bool = False, options: DecodeOptions | None = None) -> dict:
    """The launch plan of a decode call with these arguments (iq_decode_describe)."""
    info = DecodePlanInfo()
    _check("iq_decode_describe", lib.iq_decode_describe(batch, n_q_heads, n_kv_heads, max_seq_len, bits,
                                                        int(step), _opts(options), ctypes.byref(info)))
    return {name: int(getattr(info, name)) for name, _ in DecodePlanInfo._fields_}


def decode_workspace(batch: int, n_q_heads: int, n_kv_heads: int, max_seq_len: int,
                     options: DecodeOptions | None = None, device="cuda", stream=None) -> torch.Tensor:
    """A decode workspace ready for its first call: zero-filled (its leading
    counters must start at zero; every call leaves them zero)."""
    dev = torch.device(device)
    if dev.type == "cuda" and dev.index is None:
        dev = torch.device("cuda", torch.cuda.current_device())
    nbytes = decode_workspace_bytes(batch, n_q_heads, n_kv_heads, max_seq_len, options)
    return _alloc((max(nbytes, 16),), torch.uint8, dev, stream, zero=True)


def _decode_operands(cache, rot, q, block_table, seq_lens, max_seq_len, out, workspace, stream, options):
    bsz, hq, d = q.shape
    if d != HEAD_DIM:
        raise ValueError("head dim must be 128")
    dev = _device_of(q, "q")
    _check_cache(cache, dev)
    if block_table.dim() != 2 or block_table.shape[0] < bsz or seq_lens.numel() != bsz:
        raise ValueError("block_table must be int32[B][max_pages] and seq_lens int32[B]")
    if out is None:
        out = _alloc((bsz, hq, HEAD_DIM), torch.float32, dev, stream)
    elif out.dtype != torch.float32 or tuple(out.shape) != (bsz, hq, HEAD_DIM):
        raise ValueError("out must be float32 [B][Hq][128]")
    if workspace is None:
        workspace = decode_workspace(bsz, hq, cache.n_kv_heads, max_seq_len, options, dev, stream)
    ptrs = (_dev(rot, "rot", dev), _dev(q, "q", dev), _idx(block_table, "block_table", dev),
            _idx(seq_lens, "seq_lens", dev), _dev(out, "out", dev), _dev(workspace, "workspace", dev))
    return dev, out, workspace, ptrs


def decode_attention(cache: PagedCache, rot: torch.Tensor, q: torch.Tensor, block_table: torch.Tensor,
                     seq_lens: torch.Tensor, max_seq_len: int, softmax_scale: float = 0.0,
                     out: torch.Tensor | None = None, workspace: torch.Tensor | None = None,
                     stream=None, options: DecodeOptions | None = None) -> torch.Tensor:
    """q: [B][Hq][128]; block_table int32[B][max_pages]; seq_lens int32[B] -> fp32 [B][Hq][128].
    A workspace passed in must come from decode_workspace (or have zero counters)."""
    bsz, hq, _ = q.shape
    dev, out, workspace, (p_rot, p_q, p_bt, p_len, p_out, p_ws) = _decode_operands(
        cache, rot, q, block_table, seq_lens, max_seq_len, out, workspace, stream, options)
    _check("iq_decode_attention", lib.iq_decode_attention_ex(
        cache.struct, p_rot, p_q, _dtype(q), bsz, hq, p_bt, block_table.shape[-1], p_len, int(max_seq_len),
        float(softmax_scale), p_out, p_ws, workspace.numel() * workspace.element_size(), _opts(options),
        _stream(stream)))
    return out


def decode_step(cache: PagedCache, rot: torch.Tensor, q: torch.Tensor, k_new: torch.Tensor,
                v_new: torch.Tensor, block_table: torch.Tensor, seq_lens: torch.Tensor, max_seq_len: int,
                softmax_scale: float = 0.0, out: torch.Tensor | None = None,
                workspace: torch.Tensor | None = None, stream=None,
                options: DecodeOptions | None = None) -> torch.Tensor:
    """Append each sequence's current token (k_new, v_new: [B][Hkv][128], at position
    seq_lens[b] - 1) and run decode attention over all seq_lens[b] tokens, in one call."""
    bsz, hq, _ = q.shape
    if (k_new.shape != v_new.shape or k_new.dtype != v_new.dtype
            or tuple(k_new.shape) != (bsz, cache.n_kv_heads, HEAD_DIM)):
        raise ValueError("k_new and v_new must both be [B][Hkv][128] of one dtype")
    dev, out, workspace, (p_rot, p_q, p_bt, p_len, p_out, p_ws) = _decode_operands(
        cache, rot, q, block_table, seq_lens, max_seq_len, out, workspace, stream, options)
    _check("iq_decode_step", lib.iq_decode_step_ex(
        cache.struct, p_rot, p_q, _dtype(q), bsz, hq, _dev(k_new, "k_new", dev), _dev(v_new, "v_new", dev),
        _dtype(k_new), p_bt, block_table.shape[-1], p_len, int(max_seq_len), float(softmax_scale),
        p_out, p_ws, workspace.numel() * workspace.element_size(), _opts(options), _stream(stream)))
    return out


NOALLOC_SCRATCH_BYTES = 32 << 20


def decode_step_noalloc(cache: PagedCache, rot: torch.Tensor, q: torch.Tensor, k_new: torch.Tensor,
                        v_new: torch.Tensor, block_table: torch.Tensor, seq_lens: torch.Tensor,
                        max_seq_len: int, out: torch.Tensor, softmax_scale: float = 0.0,
                        stream=None) -> torch.Tensor:
    """decode_step without a workspace: the library's static per-GPU scratch
    holds the split partials, and `out` must be given, so the call allocates
    nothing.  Calls that overlap on one GPU race (they share the scratch)."""
    bsz, hq, d = q.shape
    if d != HEAD_DIM:
        raise ValueError("head dim must be 128")
    if (k_new.shape != v_new.shape or k_new.dtype != v_new.dtype
            or tuple(k_new.shape) != (bsz, cache.n_kv_heads, HEAD_DIM)):
        raise ValueError("k_new and v_new must both be [B][Hkv][128] of one dtype")
    dev = _device_of(q, "q")
    _check_cache(cache, dev)
    if block_table.dim() != 2 or block_table.shape[0] < bsz or seq_lens.numel() != bsz:
        raise ValueError("block_table must be int32[B][max_pages] and seq_lens int32[B]")
    if out.dtype != torch.float32 or tuple(out.shape) != (bsz, hq, HEAD_DIM):
        raise ValueError("out must be float32 [B][Hq][128]")
    _check("iq_decode_step_noalloc", lib.iq_decode_step_noalloc(
        cache.struct, _dev(rot, "rot", dev), _dev(q, "q", dev), _dtype(q), bsz, hq,
        _dev(k_new, "k_new", dev), _dev(v_new, "v_new", dev), _dtype(k_new),
        _idx(block_table, "block_table", dev), block_table.shape[-1], _idx(seq_lens, "seq_lens", dev),
        int(max_seq_len), float(softmax_scale), _dev(out, "out", dev), _stream(stream)))
    return out


def prefill_workspace_bytes(n_q: int, n_q_heads: int, n_kv_heads: int, q_start: int) -> int:
    return int(lib.iq_prefill_workspace_bytes(n_q, n_q_heads, n_kv_heads, q_start))


def prefill_attention(cache: PagedCache, rot: torch.Tensor, q: torch.Tensor, q_start: int,
                      block_table: torch.Tensor, softmax_scale: float = 0.0,
                      out: torch.Tensor | None = None, workspace: torch.Tensor | None = None,
                      stream=None, waves: int = 0) -> torch.Tensor:
    """q: [n_q][Hq][128] at positions q_start..; block_table int32[max_pages] -> fp32 [n_q][Hq][128].
    waves: 0 or 8 (eight waves of 16 rows) or 4 (four waves of 32 rows)."""
    n_q, hq, d = q.shape
    if d != HEAD_DIM:
        raise ValueError("head dim must be 128")
    dev = _device_of(q, "q")
    _check_cache(cache, dev)
    if out is None:
        out = _alloc((n_q, hq, HEAD_DIM), torch.float32, dev, stream)
    elif out.dtype != torch.float32 or tuple(out.shape) != (n_q, hq, HEAD_DIM):
        raise ValueError("out must be float32 [n_q][Hq][128]")
    need = prefill_workspace_bytes(max(n_q, 1), hq, cache.n_kv_heads, q_start)
    if workspace is None and need > 0:
        workspace = _alloc((need,), torch.uint8, dev, stream)
    ws_ptr = None if workspace is None else _dev(workspace, "workspace", dev)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    opts = PrefillOptions(int(waves))
    _check("iq_prefill_attention", lib.iq_prefill_attention_ex(
        cache.struct, _dev(rot, "rot", dev), _dev(q, "q", dev), _dtype(q), n_q, hq, int(q_start),
        _idx(block_table, "block_table", dev), block_table.shape[-1], float(softmax_scale),
        _dev(out, "out", dev), ws_ptr, ws_bytes, ctypes.byref(opts), _stream(stream)))
    return out


def prefill_append_workspace(n_q: int, n_q_heads: int, n_kv_heads: int, q_start: int, device="cuda",
                             stream=None) -> torch.Tensor:
    """A workspace for prefill_append, zero-filled (its counters start at zero)."""
    dev = torch.device(device)
    if dev.type == "cuda" and dev.index is None:
        dev = torch.device("cuda", torch.cuda.current_device())
    n = int(lib.iq_prefill_append_workspace_bytes(n_q, n_q_heads, n_kv_heads, q_start))
    return _alloc((max(n, 16),), torch.uint8, dev, stream, zero=True)


def prefill_append_launches(n_q: int, n_q_heads: int, n_kv_heads: int, bits: int = 3) -> int:
    """Kernels a prefill_append call with a non-empty chunk and queries launches
    on the current GPU: 1 (quantise-append fused into the prefill) or 2."""
    n = int(lib.iq_prefill_append_launches(n_q, n_q_heads, n_kv_heads, bits))
    if n < 0:
        _check("iq_prefill_append_launches", n)
    return n


def prefill_append(cache: PagedCache, rot: torch.Tensor, k_new: torch.Tensor, v_new: torch.Tensor,
                   new_start: int, q: torch.Tensor, q_start: int, block_table: torch.Tensor,
                   softmax_scale: float = 0.0, out: torch.Tensor | None = None,
                   workspace: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """Quantise-append k_new / v_new ([n_new][Hkv][128], positions new_start..) of one
    sequence and run the causal prefill of q ([n_q][Hq][128] at positions q_start..)
    over the cache, in one call; block_table int32[max_pages] -> fp32 [n_q][Hq][128]."""
    n_q, hq, d = q.shape
    if d != HEAD_DIM:
        raise ValueError("head dim must be 128")
    if (k_new.shape != v_new.shape or k_new.dtype != v_new.dtype or k_new.dim() != 3
            or k_new.shape[1] != cache.n_kv_heads or k_new.shape[2] != HEAD_DIM):
        raise ValueError("k_new and v_new must both be [n_new][Hkv][128] of one dtype")
    dev = _device_of(q, "q")
    _check_cache(cache, dev)
    if out is None:
        out = _alloc((n_q, hq, HEAD_DIM), torch.float32, dev, stream)
    elif out.dtype != torch.float32 or tuple(out.shape) != (n_q, hq, HEAD_DIM):
        raise ValueError("out must be float32 [n_q][Hq][128]")
    if workspace is None:
        workspace = prefill_append_workspace(n_q, hq, cache.n_kv_heads, q_start, dev, stream)
    _check("iq_prefill_append", lib.iq_prefill_append(
        cache.struct, _dev(rot, "rot", dev), _dev(k_new, "k_new", dev), _dev(v_new, "v_new", dev),
        _dtype(k_new), k_new.shape[0], int(new_start), _dev(q, "q", dev), _dtype(q), n_q, hq, int(q_start),
        _idx(block_table, "block_table", dev), block_table.shape[-1], float(softmax_scale),
        _dev(out, "out", dev), _dev(workspace, "workspace", dev),
        workspace.numel() * workspace.element_size(), _stream(stream)))
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
    dev = _device_of(q, "q")
    _check_cache(cache, dev)
    bsz = cu_q.numel() - 1
    if bsz < 1 or q_start.numel() != bsz or block_table.dim() != 2 or block_table.shape[0] < bsz:
        raise ValueError("cu_q must be int32[B+1], q_start int32[B], block_table int32[B][max_pages]")
    if out is None:
        out = _alloc((total_q, hq, HEAD_DIM), torch.float32, dev, stream, zero=True)
    elif out.dtype != torch.float32 or tuple(out.shape) != (total_q, hq, HEAD_DIM):
        raise ValueError("out must be float32 [total_q][Hq][128]")
    _check("iq_prefill_attention_varlen", lib.iq_prefill_attention_varlen(
        cache.struct, _dev(rot, "rot", dev), _dev(q, "q", dev), _dtype(q), bsz, hq, total_q,
        _idx(cu_q, "cu_q", dev), _idx(q_start, "q_start", dev), int(max_q_per_seq),
        int(max_kv_len), _idx(block_table, "block_table", dev), block_table.shape[-1],
        float(softmax_scale), _dev(out, "out", dev), None, 0, _stream(stream)))
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

    def tensors(self):
        return (("k", self.k), ("v", self.v))

    def nbytes(self) -> int:
        return self.k.element_size() * (self.k.numel() + self.v.numel())


def dense_append(cache: DenseCache, k: torch.Tensor, v: torch.Tensor, seq_idx: torch.Tensor,
                 pos: torch.Tensor, block_table: torch.Tensor, stream=None):
    if k.shape != v.shape or k.dtype != v.dtype or k.dim() != 3 or k.shape[2] != HEAD_DIM:
        raise ValueError("k and v must both be [n_tokens][Hkv][128] of one dtype")
    if k.shape[1] != cache.n_kv_heads:
        raise ValueError("kv head count differs from the cache")
    dev = _device_of(k, "k")
    if seq_idx.numel() != k.shape[0] or pos.numel() != k.shape[0]:
        raise ValueError("seq_idx and pos must hold one entry per token")
    _check_cache(cache, dev)
    _check("iq_dense_append", lib.iq_dense_append(
        cache.struct, _dev(k, "k", dev), _dev(v, "v", dev), _dtype(k), k.shape[0],
        _idx(seq_idx, "seq_idx", dev), _idx(pos, "pos", dev), _idx(block_table, "block_table", dev),
        block_table.shape[-1], _stream(stream)))


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
    dev = _device_of(q, "q")
    _check_cache(cache, dev)
    if block_table.dim() != 2 or block_table.shape[0] < bsz or seq_lens.numel() != bsz:
        raise ValueError("block_table must be int32[B][max_pages] and seq_lens int32[B]")
    if out is None:
        out = _alloc((bsz, hq, HEAD_DIM), torch.float32, dev, stream)
    elif out.dtype != torch.float32 or tuple(out.shape) != (bsz, hq, HEAD_DIM):
        raise ValueError("out must be float32 [B][Hq][128]")
    if workspace is None:
        nbytes = dense_decode_workspace_bytes(bsz, hq, cache.n_kv_heads, max_seq_len)
        workspace = _alloc((max(nbytes, 16),), torch.uint8, dev, stream)
    _check("iq_dense_decode_attention", lib.iq_dense_decode_attention(
        cache.struct, _dev(q, "q", dev), _dtype(q), bsz, hq, _idx(block_table, "block_table", dev),
        block_table.shape[-1], _idx(seq_lens, "seq_lens", dev), int(max_seq_len), float(softmax_scale),
        _dev(out, "out", dev), _dev(workspace, "workspace", dev),
        workspace.numel() * workspace.element_size(), _stream(stream)))
    return out


def dense_prefill_attention(cache: DenseCache, q: torch.Tensor, q_start: int, block_table: torch.Tensor,
                            softmax_scale: float = 0.0, out: torch.Tensor | None = None,
                            stream=None) -> torch.Tensor:
    """q: bf16 [n_q][Hq][128] at positions q_start..; block_table int32[max_pages]
    -> fp32 [n_q][Hq][128] over the bf16 / FP8 cache."""
    n_q, hq, d = q.shape
    if d != HEAD_DIM:
        raise ValueError("head dim must be 128")
    dev = _device_of(q, "q")
    _check_cache(cache, dev)
    if out is None:
        out = _alloc((n_q, hq, HEAD_DIM), torch.float32, dev, stream)
    elif out.dtype != torch.float32 or tuple(out.shape) != (n_q, hq, HEAD_DIM):
        raise ValueError("out must be float32 [n_q][Hq][128]")
    _check("iq_dense_prefill_attention", lib.iq_dense_prefill_attention(
        cache.struct, _dev(q, "q", dev), _dtype(q), n_q, hq, int(q_start),
        _idx(block_table, "block_table", dev), block_table.shape[-1], float(softmax_scale),
        _dev(out, "out", dev), _stream(stream)))
    return out


def probe_sink_bytes() -> int:
    return int(lib.iq_probe_sink_bytes())


def probe_read(buf: torch.Tensor, sink: torch.Tensor, stream=None):
    """Stream `buf` (contiguous, size a multiple of 16 bytes) once on the GPU."""
    dev = _device_of(buf, "buf")
    nbytes = buf.numel() * buf.element_size()
    _check("iq_probe_read", lib.iq_probe_read(_dev(buf, "buf", dev), nbytes, _dev(sink, "sink", dev),
                                              sink.numel() * sink.element_size(), _stream(stream)))
