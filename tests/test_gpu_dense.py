"""Uncompressed bf16 baseline and FP8 (E4M3) fallback (iq_dense_append,
iq_dense_decode_attention) and the HBM read probe (iq_probe_read), through
the C-ABI.

The baseline's decode must match plain fp64 softmax attention on the same
bf16-rounded q, K and V (or the FP8 oracle's dequantised K and V) within the
path's attention tolerance, max_rows max|gpu - ref| / max|ref| <= 1e-3.  Its
append must place every row exactly (bf16 bits, or the oracle's FP8 bytes) at
the documented offsets.
"""

import numpy as np
import pytest
import torch

from compressed_space_attention_amd import synth
from oracle import fp8_oracle as F
from oracle import isoquant_oracle as O
from tests.gpu_cases import max_row_error, tol

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():
    pytest.skip("needs a GPU", allow_module_level=True)


def _say(*a):
    print(*a, flush=True)


class DenseScenario:
    def __init__(self, seed, lens, hkv, dtype="bf16", outliers=False, shuffle=True, fmt="bf16",
                 k_scale=1.0, v_scale=1.0, fill=None):
        from compressed_space_attention_amd import isoquant as iq
        self.iq, self.lens, self.hkv = iq, [int(n) for n in lens], hkv
        pages = [max(1, -(-n // 64)) for n in self.lens]
        self.block_table, self.num_pages = synth.block_table(seed + 1, pages, shuffle, 2)
        n_tok = sum(self.lens)
        out_ch = synth.outlier_channels(seed + 2, hkv) if outliers else None
        self.k = synth.kv_vectors(seed + 3, n_tok, hkv, dtype, out_ch)
        self.v = synth.kv_vectors(seed + 4, n_tok, hkv, dtype, None)
        self.seq_idx = np.concatenate([np.full(n, b, np.int32) for b, n in enumerate(self.lens)])
        self.pos = np.concatenate([np.arange(n, dtype=np.int32) for n in self.lens])
        self.fmt, self.k_scale, self.v_scale = fmt, k_scale, v_scale
        self.cache = iq.DenseCache(self.num_pages, hkv, zero=True, format=fmt, k_scale=k_scale,
                                   v_scale=v_scale)
        if fill is not None:  # bit pattern of never-written slots
            self.cache.k.fill_(fill)
            self.cache.v.fill_(fill)
        self.bt_dev = torch.from_numpy(self.block_table).cuda()
        self.lens_dev = torch.tensor(self.lens, dtype=torch.int32).cuda()
        if n_tok:
            iq.dense_append(self.cache, self.k.cuda(), self.v.cuda(), torch.from_numpy(self.seq_idx).cuda(),
                            torch.from_numpy(self.pos).cuda(), self.bt_dev)
        torch.cuda.synchronize()
        self.starts = np.concatenate([[0], np.cumsum(self.lens)])

    def reference(self, q):
        """fp64 attention over the bf16 rows (or the FP8 oracle's values) of
        each sequence."""
        if self.fmt == "fp8":
            return F.decode_attention_fp8(self.k.double().numpy(), self.v.double().numpy(),
                                          q.double().numpy(), self.starts, self.hkv,
                                          self.k_scale, self.v_scale)
        q = q.to(torch.float64).numpy()
        bsz, hq, _ = q.shape
        grp = hq // self.hkv
        kk = self.k.to(torch.float64).numpy()
        vv = self.v.to(torch.float64).numpy()
        out = np.zeros((bsz, hq, 128))
        for b in range(bsz):
            s, e = self.starts[b], self.starts[b + 1]
            for g in range(self.hkv):
                if e > s:
                    out[b, g * grp:(g + 1) * grp] = O.reference_attention(
                        q[b, g * grp:(g + 1) * grp], kk[s:e, g], vv[s:e, g])
        return out


def test_dense_append_layout():
    s = DenseScenario(900, [1, 70, 128], hkv=3, dtype="f32")
    k_host = s.cache.k.cpu().numpy().view(np.uint16)
    v_host = s.cache.v.cpu().numpy().view(np.uint16)
    kb = s.k.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)  # RNE bf16 of the f32 rows
    vb = s.v.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    page = s.block_table[s.seq_idx, s.pos // 64]
    slot = s.pos % 64
    for h in range(3):
        assert np.array_equal(k_host[page, h, slot], kb[:, h])
        assert np.array_equal(v_host[page, h, :, slot], vb[:, h])


DENSE_CASES = [
    # (lens, hkv, hq, outliers)
    ([2048], 1, 1, False),
    ([1, 31, 32, 33, 63, 64, 65, 700], 2, 4, True),
    ([130, 1000, 2100], 4, 32, True),
    ([640, 0, 33], 2, 32, False),
]


@pytest.mark.parametrize("case", range(len(DENSE_CASES)))
def test_dense_decode_matches_reference(case):
    lens, hkv, hq, outl = DENSE_CASES[case]
    _say(f"dense decode lens={lens} hkv={hkv} hq={hq}")
    s = DenseScenario(910 + case, lens, hkv=hkv, outliers=outl)
    q = synth.to_dtype(synth.normal(920 + case, (len(lens), hq, 128)), "bf16")
    out = s.iq.dense_decode_attention(s.cache, q.cuda(), s.bt_dev, s.lens_dev, max(lens)).cpu().numpy()
    ref = s.reference(q)
    err = max_row_error(out, ref)
    _say(f"  max row error {err:.3e}")
    assert np.all(np.isfinite(out))
    assert err <= tol()
    for b, n in enumerate(lens):
        if n == 0:
            assert np.all(out[b] == 0)


def test_dense_decode_ignores_unwritten_slots():
    """Slots past the length hold NaN bit patterns: the result must not see them."""
    s = DenseScenario(930, [40, 100], hkv=2)
    s.cache.k.fill_(-1)  # 0xFFFF: bf16 NaN everywhere ...
    s.cache.v.fill_(-1)
    s.iq.dense_append(s.cache, s.k.cuda(), s.v.cuda(), torch.from_numpy(s.seq_idx).cuda(),
                      torch.from_numpy(s.pos).cuda(), s.bt_dev)  # ... except the written slots
    q = synth.to_dtype(synth.normal(931, (2, 8, 128)), "bf16")
    out = s.iq.dense_decode_attention(s.cache, q.cuda(), s.bt_dev, s.lens_dev, 100).cpu().numpy()
    assert np.all(np.isfinite(out))
    assert max_row_error(out, s.reference(q)) <= tol()


def test_probe_reads_every_word_once():
    from compressed_space_attention_amd import isoquant as iq
    # above eight grid strides (8 x 2048 x 256 x 16 B) and not a multiple of
    # one: both the unrolled loop and the tail loop run
    n = (80 << 20) + 48
    host = np.random.default_rng(5).integers(0, 2 ** 32, size=n // 4, dtype=np.uint32)
    buf = torch.from_numpy(host.view(np.int32)).cuda()
    sink = torch.zeros(iq.probe_sink_bytes() // 4, dtype=torch.int32, device="cuda")
    iq.probe_read(buf, sink)
    torch.cuda.synchronize()
    got = np.bitwise_xor.reduce(sink.cpu().numpy().view(np.uint32))
    assert got == np.bitwise_xor.reduce(host)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_fp8_append_bytes(dtype):
    """Every stored byte is the oracle's E4M3 encoding of x / scale, at the
    documented offsets (K token-major, V coordinate-major)."""
    s = DenseScenario(940, [1, 70, 128], hkv=3, dtype=dtype, outliers=True, fmt="fp8",
                      k_scale=0.05, v_scale=3.0)
    k_host, v_host = s.cache.k.cpu().numpy(), s.cache.v.cpu().numpy()
    kb = F.quantize_rows(s.k.float().numpy(), 0.05)
    vb = F.quantize_rows(s.v.float().numpy(), 3.0)
    page = s.block_table[s.seq_idx, s.pos // 64]
    slot = s.pos % 64
    for h in range(3):
        assert np.array_equal(k_host[page, h, slot], kb[:, h])
        assert np.array_equal(v_host[page, h, :, slot], vb[:, h])
    assert np.any(kb == 0x7E) and np.any(kb == 0xFE)   # outliers x 20 saturate at +-448


FP8_CASES = [
    # (lens, hkv, hq, outliers, k_scale, v_scale)
    ([2048], 1, 1, False, 1.0, 1.0),
    ([1, 31, 32, 33, 63, 64, 65, 700], 2, 4, True, 0.125, 1.0),
    ([130, 1000, 2100], 4, 32, True, 0.0, 2.0),     # k_scale 0 selects 1
    ([640, 0, 33], 2, 32, False, 1.0, 0.01),
]


@pytest.mark.parametrize("case", range(len(FP8_CASES)))
def test_fp8_decode_matches_reference(case):
    lens, hkv, hq, outl, ks, vs = FP8_CASES[case]
    _say(f"fp8 decode lens={lens} hkv={hkv} hq={hq} scales={ks},{vs}")
    s = DenseScenario(950 + case, lens, hkv=hkv, outliers=outl, fmt="fp8", k_scale=ks, v_scale=vs)
    s.k_scale = ks or 1.0
    q = synth.to_dtype(synth.normal(960 + case, (len(lens), hq, 128)), "bf16")
    out = s.iq.dense_decode_attention(s.cache, q.cuda(), s.bt_dev, s.lens_dev, max(lens)).cpu().numpy()
    ref = s.reference(q)
    err = max_row_error(out, ref)
    _say(f"  max row error {err:.3e}")
    assert np.all(np.isfinite(out))
    assert err <= tol()
    for b, n in enumerate(lens):
        if n == 0:
            assert np.all(out[b] == 0)


def test_fp8_decode_ignores_unwritten_slots():
    """Never-written slots hold 0xFF (E4M3 NaN): the result must not see them."""
    s = DenseScenario(970, [40, 100], hkv=2, fmt="fp8", fill=255)
    q = synth.to_dtype(synth.normal(971, (2, 8, 128)), "bf16")
    out = s.iq.dense_decode_attention(s.cache, q.cuda(), s.bt_dev, s.lens_dev, 100).cpu().numpy()
    assert np.all(np.isfinite(out))
    assert max_row_error(out, s.reference(q)) <= tol()


DENSE_PREFILL_CASES = [
    # (cache length, n_q, hkv, hq, format): groups 1..128, ragged tiles, one query
    (1000, 200, 2, 16, "bf16"),
    (300, 300, 1, 1, "bf16"),
    (700, 77, 2, 8, "fp8"),
    (640, 1, 2, 4, "fp8"),
    (200, 70, 1, 128, "bf16"),
]


@pytest.mark.parametrize("case", range(len(DENSE_PREFILL_CASES)))
def test_dense_prefill_matches_reference(case):
    total, n_q, hkv, hq, fmt = DENSE_PREFILL_CASES[case]
    _say(f"dense prefill total={total} n_q={n_q} hkv={hkv} hq={hq} format={fmt}")
    ks, vs = (1.0, 1.0) if fmt == "bf16" else (0.5, 2.0)
    s = DenseScenario(980 + case, [total], hkv=hkv, outliers=True, fmt=fmt, k_scale=ks, v_scale=vs,
                      fill=-1 if fmt == "bf16" else 255)       # unwritten slots: NaN patterns
    q = synth.to_dtype(synth.normal(990 + case, (n_q, hq, 128)), "bf16")
    q_start = total - n_q
    out = s.iq.dense_prefill_attention(s.cache, q.cuda(), q_start, s.bt_dev[0]).cpu().numpy()
    assert np.all(np.isfinite(out))
    if fmt == "fp8":
        kq = F.dequantize_rows(F.quantize_rows(s.k.float().numpy(), ks), ks)
        vq = F.dequantize_rows(F.quantize_rows(s.v.float().numpy(), vs), vs)
    else:
        kq, vq = s.k.double().numpy(), s.v.double().numpy()
    qd = q.double().numpy()
    grp = hq // hkv
    rows = np.unique(np.linspace(0, n_q - 1, min(n_q, 24)).astype(int))
    ref = np.zeros((len(rows), hq, 128))
    for ri, i in enumerate(rows):
        vis = q_start + i + 1
        for g in range(hkv):
            ref[ri, g * grp:(g + 1) * grp] = O.reference_attention(qd[i, g * grp:(g + 1) * grp],
                                                                   kq[:vis, g], vq[:vis, g])
    err = max_row_error(out[rows], ref)
    _say(f"  max row error {err:.3e}")
    assert err <= tol()
