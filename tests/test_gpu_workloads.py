"""Parity at the full sizes of the named workloads, in the launch configuration
the benchmark uses (same entry points, same split planning).

Large inputs are drawn on the GPU by a seeded torch generator; the oracle gets
the sampled inputs copied to the host.  Attention parity uses the GPU-written
cache; code parity re-quantises sampled vectors with the oracle.  The cosine
similarity of compressed vs uncompressed fp64 attention is reported."""

import math

import numpy as np
import pytest
import torch

from compressed_space_attention_amd import synth, workloads
from oracle import isoquant4_oracle as O4
from oracle import isoquant_oracle as O
from tests.gpu_cases import max_row_error, tol

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():
    pytest.skip("needs a GPU", allow_module_level=True)

from compressed_space_attention_amd import isoquant as iq  # noqa: E402


def _say(*a):
    print(*a, flush=True)


class Built:
    """A workload's cache quantised by the GPU, inputs kept on the device."""

    def __init__(self, w, lens, device="cuda", bits=3):
        self.w, self.bits = w, bits
        self.lens = np.asarray(lens, dtype=np.int64)
        self.quats = synth.quaternions(w.seed, w.n_kv_heads)
        self.blocks = O.rotation_matrices(self.quats)
        pages = [-(-int(n) // 64) for n in self.lens]
        self.bt, self.num_pages = synth.block_table(w.seed + 5, pages, shuffle=w.shuffle_pages)
        self.bt_dev = torch.from_numpy(self.bt).to(device)
        self.lens_dev = torch.from_numpy(self.lens.astype(np.int32)).to(device)
        self.rot = iq.rotation_init(self.quats, device=device)
        self.cache = iq.PagedCache(self.num_pages, w.n_kv_heads, device=device, zero=True, bits=bits)
        dt = {"bf16": torch.bfloat16, "f32": torch.float32}[w.dtype]
        total = int(self.lens.sum())
        scale = torch.ones(w.n_kv_heads, 128, device=device)
        if w.k_outliers:
            ch = synth.outlier_channels(w.seed + 1, w.n_kv_heads)
            for h in range(w.n_kv_heads):
                scale[h, torch.from_numpy(ch[h]).to(device)] = 10.0
        self.k_scale, self.dt = scale, dt
        self.k = (synth.draw_normal_device(w.seed + 2, (total, w.n_kv_heads, 128), torch.float32, device)
                  * scale).to(dt)
        self.v = synth.draw_normal_device(w.seed + 3, (total, w.n_kv_heads, 128), dt, device)
        self.seq_idx = np.concatenate([np.full(n, b, np.int32) for b, n in enumerate(self.lens)])
        self.pos = np.concatenate([np.arange(n, dtype=np.int32) for n in self.lens])
        iq.quantize_append(self.cache, self.rot, self.k, self.v, torch.from_numpy(self.seq_idx).to(device),
                           torch.from_numpy(self.pos).to(device), self.bt_dev)
        self.q = synth.draw_normal_device(w.seed + 4, (len(self.lens), w.n_q_heads, 128), dt, device)
        torch.cuda.synchronize()

    def host(self):
        arrays = self.cache.to_host()
        return O4.PagedCache4.from_arrays(*arrays) if self.bits == 4 else O.PagedCache.from_arrays(*arrays)

    def sampled_code_parity(self, n_sample, seed):
        rng = np.random.default_rng(seed)
        idx = np.unique(rng.integers(0, len(self.pos), size=n_sample))
        idx = np.unique(np.concatenate([idx, [0, len(self.pos) - 1]]))
        page = self.bt[self.seq_idx[idx], self.pos[idx] // 64]
        slot = self.pos[idx] % 64
        codes = mism = near = 0
        host = self.host()
        for name, x in (("k", self.k), ("v", self.v)):
            xs = x[torch.from_numpy(idx).cuda()].double().cpu().numpy()
            for h in range(self.w.n_kv_heads):
                if self.bits == 4:
                    q = O4.quantize4(xs[:, h], self.blocks[h])
                    gc = host.codes(name, page, h, slot)
                else:
                    q = O.quantize(xs[:, h], self.blocks[h])
                    gc = O.unpack_codes(host.records(name, page, h, slot))
                gn = getattr(host, name + "_norms")[page, h, slot]
                bad = gc != q["codes"]
                assert not np.any(bad & ~q["near"]), f"{name} head {h}: code mismatch off-boundary"
                nb = gn != q["norm16"]
                assert not np.any(nb & ~q["norm_near"]), f"{name} head {h}: norm mismatch"
                codes += gc.size
                mism += int(bad.sum())
                near += int(q["near"].sum())
        _say(f"  sampled codes {codes}: mismatches {mism}, near-boundary {near}")
        assert mism < 1e-5 * codes + 1
        return mism, near, codes

    def decode(self):
        return iq.decode_attention(self.cache, self.rot, self.q, self.bt_dev, self.lens_dev,
                                   int(self.lens.max()))

    def oracle_decode(self, seqs):
        q = self.q.double().cpu().numpy()
        bt = self.bt[seqs]
        fn = O4.decode_attention4 if self.bits == 4 else O.decode_attention
        return fn(self.host(), self.blocks, q[seqs], bt, self.lens[seqs])

    def cosine_vs_uncompressed(self, seq, heads, out):
        grp = self.w.group
        n = int(self.lens[seq])
        start = int(self.lens[:seq].sum())
        cos = []
        for h in heads:
            g = h // grp
            k = self.k[start:start + n, g].double().cpu().numpy()
            v = self.v[start:start + n, g].double().cpu().numpy()
            q = self.q[seq, h:h + 1].double().cpu().numpy()
            ref = O.reference_attention(q, k, v)
            cos.append(float(O.row_cosine(out[seq, h:h + 1], ref)[0]))
        return cos


def test_tiny_decode_full():
    w = workloads.TINY_DECODE
    b = Built(w, w.seq_lens())
    b.sampled_code_parity(4096, 1)
    out = b.decode().cpu().numpy()
    ref = b.oracle_decode(np.arange(w.batch))
    err = max_row_error(out, ref)
    cos = b.cosine_vs_uncompressed(0, range(w.n_q_heads), out)
    _say(f"  {w.name}: max row error {err:.3e}, cosine vs uncompressed {np.round(cos, 4)}")
    assert err <= tol()


@pytest.mark.parametrize("bits", [3, 4])
def test_gqa_decode_32k_full(bits):
    w = workloads.GQA_DECODE_32K
    b = Built(w, w.seq_lens(), bits=bits)
    b.sampled_code_parity(8192, 2)
    out = b.decode().cpu().numpy()
    ref = b.oracle_decode(np.arange(w.batch))
    err = max_row_error(out, ref)
    cos = b.cosine_vs_uncompressed(0, range(0, w.n_q_heads, 4), out)
    _say(f"  {w.name}: max row error {err:.3e}, cosine min {min(cos):.4f} mean {np.mean(cos):.4f}")
    assert err <= tol()


@pytest.mark.parametrize("bits", [3, 4])
def test_gqa_decode_32k_step_full(bits):
    """The benchmarked call itself: iq_decode_step at the 32K GQA shape (batch 1,
    32 query / 4 kv heads, 32,767 cached tokens plus the current one), planned
    as the benchmark plans it.  The step's cache equals quantise-append of the
    token into a copy of the cache, byte for byte; the appended records match
    the oracle's quantiser (codes bit for bit outside the 1e-6 boundary
    exemption, norms outside fp16 midpoints); every query head's row is within
    the tolerance of the oracle attending over the GPU-written cache, and
    within half of it of decode attention on the pair's cache."""
    w = workloads.GQA_DECODE_32K
    L = w.context
    b = Built(w, [L - 1], bits=bits)
    hkv = w.n_kv_heads
    k_new = (synth.draw_normal_device(w.seed + 12, (1, hkv, 128), torch.float32) * b.k_scale).to(b.dt)
    v_new = synth.draw_normal_device(w.seed + 13, (1, hkv, 128), b.dt)
    pair = iq.PagedCache(b.num_pages, hkv, zero=True, bits=bits)
    for dst, src in zip((pair.k_codes, pair.k_norms, pair.v_codes, pair.v_norms),
                        (b.cache.k_codes, b.cache.k_norms, b.cache.v_codes, b.cache.v_norms)):
        dst.copy_(src)
    lens_dev = torch.tensor([L], dtype=torch.int32, device="cuda")
    _say(f"  {w.name} decode step, {bits}-bit records, {L} tokens")
    out = iq.decode_step(b.cache, b.rot, b.q, k_new, v_new, b.bt_dev, lens_dev, L)
    iq.quantize_append(pair, b.rot, k_new, v_new, torch.zeros(1, dtype=torch.int32, device="cuda"),
                       torch.tensor([L - 1], dtype=torch.int32, device="cuda"), b.bt_dev)
    out_pair = iq.decode_attention(pair, b.rot, b.q, b.bt_dev, lens_dev, L)
    torch.cuda.synchronize()
    for x, y in zip((b.cache.k_codes, b.cache.k_norms, b.cache.v_codes, b.cache.v_norms),
                    (pair.k_codes, pair.k_norms, pair.v_codes, pair.v_norms)):
        assert torch.equal(x, y), "the step's cache differs from quantise-append + the same cache"
    host = b.host()
    page, slot = int(b.bt[0, (L - 1) // 64]), (L - 1) % 64
    near = mism = 0
    for name, x in (("k", k_new), ("v", v_new)):
        xs = x[0].double().cpu().numpy()
        for h in range(hkv):
            if bits == 4:
                q = O4.quantize4(xs[h:h + 1], b.blocks[h])
                gc = host.codes(name, np.array([page]), h, np.array([slot]))
            else:
                q = O.quantize(xs[h:h + 1], b.blocks[h])
                gc = O.unpack_codes(host.records(name, np.array([page]), h, np.array([slot])))
            bad = gc != q["codes"]
            assert not np.any(bad & ~q["near"]), f"appended {name} head {h}: code mismatch off-boundary"
            gn = getattr(host, name + "_norms")[page, h, slot]
            assert gn == q["norm16"][0] or q["norm_near"][0], f"appended {name} head {h}: norm"
            mism += int(bad.sum())
            near += int(q["near"].sum())
    _say(f"  appended token: {2 * hkv * 128} codes, mismatches {mism}, near-boundary {near}")
    ref = (O4.decode_attention4 if bits == 4 else O.decode_attention)(
        host, b.blocks, b.q.double().cpu().numpy(), b.bt, np.array([L]))
    o = out.cpu().numpy()
    err = max_row_error(o, ref)
    err_pair = max_row_error(o, out_pair.cpu().numpy())
    b.k, b.v, b.lens = torch.cat([b.k, k_new]), torch.cat([b.v, v_new]), np.array([L])
    cos = b.cosine_vs_uncompressed(0, range(w.n_q_heads), o)
    _say(f"  max row error {err:.3e} (all {w.n_q_heads} heads), vs append + decode {err_pair:.3e}, "
         f"cosine vs uncompressed min {min(cos):.4f} mean {np.mean(cos):.4f}")
    assert np.all(np.isfinite(o))
    assert err <= tol()
    assert err_pair <= 0.5 * tol()


@pytest.mark.parametrize("bits", [3, 4])
def test_ragged_decode_sampled_sequences(bits):
    w = workloads.RAGGED_DECODE
    lens = w.seq_lens()
    b = Built(w, lens, bits=bits)
    b.sampled_code_parity(8192, 3)
    out = b.decode().cpu().numpy()
    pick = np.unique([int(np.argmin(lens)), int(np.argmax(lens)), 5])
    ref = b.oracle_decode(pick)
    err = max_row_error(out[pick], ref)
    _say(f"  {w.name}: lens {lens.tolist()}, checked {pick.tolist()}, max row error {err:.3e}")
    assert err <= tol()


def test_long_decode_128k_sampled_sequence():
    w = workloads.LONG_DECODE_128K
    b = Built(w, w.seq_lens())
    b.sampled_code_parity(4096, 4)
    out = b.decode().cpu().numpy()
    ref = b.oracle_decode(np.array([w.batch - 1]))
    err = max_row_error(out[w.batch - 1:], ref)
    _say(f"  {w.name}: max row error {err:.3e} (last sequence, all heads)")
    assert err <= tol()
    assert np.all(np.isfinite(out))


@pytest.mark.parametrize("bits", [3, 4])
def test_chunked_prefill_full_shape_sampled_rows(bits):
    p = workloads.CHUNKED_PREFILL
    w = workloads.DecodeWorkload(p.name, 1, p.n_q_heads, p.n_kv_heads, p.dtype, False, True,
                                 p.seed, context=p.total)
    # cache: the first `cached` tokens, then the appended chunk in a second call
    b = Built(w, [p.cached], bits=bits)
    k2 = synth.draw_normal_device(p.seed + 7, (p.appended, p.n_kv_heads, 128), torch.bfloat16)
    v2 = synth.draw_normal_device(p.seed + 8, (p.appended, p.n_kv_heads, 128), torch.bfloat16)
    pages = -(-p.total // 64)
    bt, num_pages = synth.block_table(p.seed + 9, [pages], shuffle=True)
    b.bt, b.bt_dev = bt, torch.from_numpy(bt).cuda()
    b.cache = iq.PagedCache(num_pages, p.n_kv_heads, zero=True, bits=bits)
    pos1 = torch.arange(p.cached, dtype=torch.int32, device="cuda")
    pos2 = torch.arange(p.cached, p.total, dtype=torch.int32, device="cuda")
    iq.quantize_append(b.cache, b.rot, b.k, b.v, torch.zeros_like(pos1), pos1, b.bt_dev)
    iq.quantize_append(b.cache, b.rot, k2, v2, torch.zeros_like(pos2), pos2, b.bt_dev)
    b.k = torch.cat([b.k, k2])
    b.v = torch.cat([b.v, v2])
    b.seq_idx = np.zeros(p.total, np.int32)
    b.pos = np.arange(p.total, dtype=np.int32)
    b.lens = np.array([p.total])
    b.sampled_code_parity(4096, 5)
    q = synth.draw_normal_device(p.seed + 10, (p.n_queries, p.n_q_heads, 128), torch.bfloat16)
    out = iq.prefill_attention(b.cache, b.rot, q, p.q_start, b.bt_dev[0]).cpu().numpy()
    rows = np.array([0, 1, 100, 255, 256, 400, p.n_queries - 2, p.n_queries - 1])
    fn = O4.prefill_attention4 if bits == 4 else O.prefill_attention
    ref = fn(b.host(), b.blocks, q.double().cpu().numpy(), p.q_start, bt[0], rows=rows)
    err = max_row_error(out[rows], ref)
    _say(f"  {p.name}: max row error {err:.3e} over rows {rows.tolist()}")
    assert err <= tol()


def test_prefill4_at_the_staging_limit():
    """4-bit records over a causal range of exactly the prefill's page-table
    staging limit (4,096 pages, 262,144 tokens; the 3-bit case is one of the
    prefill cases in tests/test_gpu_parity.py): the last 32 positions attend
    over the whole cache; sampled rows against the oracle.  One token more is
    refused on the host (tests/test_abi_cpu.py)."""
    bits = 4
    total, n_q = 4096 * 64, 32
    w = workloads.DecodeWorkload("prefill_staging_limit", 1, 2, 1, "bf16", False, True, 977, context=total)
    b = Built(w, [total], bits=bits)
    q_start = total - n_q
    q = synth.draw_normal_device(978, (n_q, 2, 128), torch.bfloat16)
    out = iq.prefill_attention(b.cache, b.rot, q, q_start, b.bt_dev[0]).cpu().numpy()
    rows = np.array([0, 1, 15, 30, 31])            # queries; the last one sees every token
    ref = O4.prefill_attention4(b.host(), b.blocks, q.double().cpu().numpy(), q_start, b.bt[0], rows=rows)
    err = max_row_error(out[rows], ref)
    _say(f"  staging limit (4-bit): max row error {err:.3e}")
    assert np.all(np.isfinite(out))
    assert err <= tol()

