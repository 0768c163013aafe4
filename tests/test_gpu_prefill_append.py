"""The fused quantise-append + chunked prefill (iq_prefill_append) on the GPU.

Each schedule runs a sequence of chunks through two caches of one layout: on
cache A one iq_prefill_append call per chunk (one workspace for every call, so
the counters left by a call are the next call's starting state), on cache B
iq_quantize_append of the chunk followed by iq_prefill_attention.  After each
chunk the two caches must hold the same bytes and the two outputs the same
bits (the same tiles, the same arithmetic, the same records).  At the end the
records of A are checked against the oracle's quantiser (codes bit for bit
outside the 1e-6 boundary exemption) and sampled rows of every chunk's output
against the oracle's causal attention over A's records (max_rows max|err| /
max|ref| <= 1e-3).
"""

from types import SimpleNamespace

import numpy as np
import pytest
import torch

from compressed_space_attention_amd import synth
from oracle import isoquant4_oracle as O4
from oracle import isoquant_oracle as O
from tests.gpu_cases import code_parity, code_parity4, max_row_error, tol

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():
    pytest.skip("needs a GPU", allow_module_level=True)


def _say(*a):
    print(*a, flush=True)


# (kv heads, query heads, record bits, chunks (new_start, n_new, q_start, n_q)[, input dtype])
SCHEDULES = {
    # extend attention over a first chunk, a ragged second chunk whose queries
    # are its last 50 positions, then a prefill-only and an append-only call
    "ragged_3bit": (2, 8, 3, [(0, 300, 0, 300), (300, 400, 650, 50), (700, 0, 600, 100), (700, 64, 0, 0)]),
    # one query head per kv head, then a one-token chunk
    "mha_3bit": (1, 1, 3, [(0, 1024, 896, 128), (1024, 1, 1024, 1)]),
    # 4-bit records; the second chunk's queries all sit before the chunk
    "gqa_4bit": (2, 16, 4, [(0, 1500, 1300, 200), (1500, 500, 1000, 100)]),
    # 8 kv heads x 64 row tiles: more workgroups than the GPU holds at once,
    # so the call runs the append and the prefill as two kernels
    "two_kernels": (8, 64, 3, [(0, 276, 0, 0), (276, 1024, 276, 1024)]),
    # fp32 and fp16 K/V rows (the fused coding converts each input type)
    "f32_rows": (2, 8, 3, [(0, 200, 0, 200), (200, 333, 500, 33)], "f32"),
    "f16_rows_4bit": (2, 16, 4, [(0, 130, 0, 130), (130, 200, 300, 30)], "f16"),
}


def _run_schedule(seed, hkv, hq, bits, chunks, total, shared_prefix=0, oracle_codes=True, rows_per_chunk=8,
                  dtype="bf16"):
    from compressed_space_attention_amd import isoquant as iq
    dev = "cuda"
    pages = -(-total // 64)
    bt_np, num_pages = synth.block_table(seed, [pages], True, 2)
    bt = torch.from_numpy(bt_np).to(dev)
    quats = synth.quaternions(seed + 1, hkv)
    blocks = O.rotation_matrices(quats)
    rot = iq.rotation_init(quats, device=dev)
    out_ch = synth.outlier_channels(seed + 2, hkv)
    k = synth.kv_vectors(seed + 3, total, hkv, dtype, out_ch)
    v = synth.kv_vectors(seed + 4, total, hkv, dtype, None)
    kd, vd = k.to(dev), v.to(dev)
    ca = iq.PagedCache(num_pages, hkv, device=dev, zero=True, bits=bits)
    cb = iq.PagedCache(num_pages, hkv, device=dev, zero=True, bits=bits)
    if shared_prefix:
        seq = torch.zeros(shared_prefix, dtype=torch.int32, device=dev)
        pos = torch.arange(shared_prefix, dtype=torch.int32, device=dev)
        for c in (ca, cb):
            iq.quantize_append(c, rot, kd[:shared_prefix], vd[:shared_prefix], seq, pos, bt)
    for _, n_new, _, n_q in chunks:
        if n_new and n_q:
            launches = iq.prefill_append_launches(n_q, hq, hkv, bits)
            _say(f"  {n_q} queries x {hq} heads over {hkv} kv heads: {launches} launch(es)")
            # one kernel unless the grid (kv heads x row tiles) exceeds what the GPU holds
            assert launches == (2 if hkv * n_q * (hq // hkv) > 128 * 256 else 1)
    max_q = max(n_q for _, _, _, n_q in chunks)
    max_start = max(q_start for _, _, q_start, _ in chunks)
    ws = iq.prefill_append_workspace(max(max_q, 1), hq, hkv, max_start, dev)
    outs = []
    for ci, (s0, n_new, q_start, n_q) in enumerate(chunks):
        _say(f"  chunk {ci}: append {s0}..{s0 + n_new - 1}, queries {q_start}..{q_start + n_q - 1}")
        q = synth.to_dtype(synth.normal(seed + 10 + ci, (n_q, hq, 128)), "bf16")
        qd = q.to(dev)
        k_new, v_new = kd[s0:s0 + n_new].contiguous(), vd[s0:s0 + n_new].contiguous()
        out_a = iq.prefill_append(ca, rot, k_new, v_new, s0, qd, q_start, bt[0], workspace=ws)
        if n_new:
            seq = torch.zeros(n_new, dtype=torch.int32, device=dev)
            pos = torch.arange(s0, s0 + n_new, dtype=torch.int32, device=dev)
            iq.quantize_append(cb, rot, k_new, v_new, seq, pos, bt)
        out_b = iq.prefill_attention(cb, rot, qd, q_start, bt[0]) if n_q else out_a
        torch.cuda.synchronize()
        for x, y in zip(ca.to_host(), cb.to_host()):
            assert np.array_equal(x, y), f"chunk {ci}: the caches differ"
        oa, ob = out_a.cpu().numpy(), out_b.cpu().numpy()
        assert np.all(np.isfinite(oa)), f"chunk {ci}: non-finite rows"
        assert np.array_equal(oa, ob), f"chunk {ci}: fused and two-call outputs differ"
        outs.append((q, q_start, oa))
    # the counters are back at zero for the next user of the workspace
    assert int(ws[:iq.DECODE_COUNTER_BYTES].count_nonzero()) == 0

    host = O4.PagedCache4.from_arrays(*ca.to_host()) if bits == 4 else O.PagedCache.from_arrays(*ca.to_host())
    if oracle_codes:
        written = max(s0 + n for s0, n, _, _ in chunks)
        ref = O4.PagedCache4(num_pages, hkv) if bits == 4 else O.PagedCache(num_pages, hkv)
        seq_idx, pos = np.zeros(written, np.int32), np.arange(written, dtype=np.int32)
        quant = O4.quantize_append4 if bits == 4 else O.quantize_append
        info = quant(ref, blocks, k[:written].double().numpy(), v[:written].double().numpy(), seq_idx, pos, bt_np)
        scen = SimpleNamespace(block_table=bt_np, seq_idx=seq_idx, pos=pos, hkv=hkv)
        st = (code_parity4 if bits == 4 else code_parity)(host, ref, info, scen)
        _say("  codes:", st)
        assert st["mismatch"] <= st["near"] and st["mismatch"] < 1e-5 * st["codes"] + 1
    attend = O4.prefill_attention4 if bits == 4 else O.prefill_attention
    worst = 0.0
    for q, q_start, oa in outs:
        n_q = q.shape[0]
        if n_q == 0:
            continue
        rows = np.unique(np.linspace(0, n_q - 1, min(n_q, rows_per_chunk)).astype(int))
        ref = attend(host, blocks, q.double().numpy(), q_start, bt_np[0], rows=rows)
        worst = max(worst, max_row_error(oa[rows], ref))
    _say(f"  max row error {worst:.3e}")
    assert worst <= tol()


@pytest.mark.parametrize("name", list(SCHEDULES))
def test_prefill_append_matches_two_calls_and_oracle(name):
    hkv, hq, bits, chunks, *rest = SCHEDULES[name]
    dtype = rest[0] if rest else "bf16"
    total = max(max(s0 + n, q0 + nq) for s0, n, q0, nq in chunks)
    _say(f"prefill_append schedule {name}: hkv={hkv} hq={hq} bits={bits} total={total} rows {dtype}")
    _run_schedule(7100 + len(name), hkv, hq, bits, chunks, total, dtype=dtype)


@pytest.mark.parametrize("bits", [3, 4])
def test_prefill_append_chunked_prefill_workload(bits):
    """The chunked-prefill workload at its full size: 8,192 tokens appended to a
    24,576-token cache (8 kv heads), then the last 512 positions x 64 query
    heads attend the 32,768 tokens."""
    _say(f"prefill_append 32K workload bits={bits}")
    _run_schedule(7300 + bits, 8, 64, bits, [(24576, 8192, 32256, 512)], 32768, shared_prefix=24576,
                  oracle_codes=False, rows_per_chunk=6)


def test_prefill_append_refuses_bad_ranges():
    from compressed_space_attention_amd import isoquant as iq
    dev = "cuda"
    rot = iq.rotation_init(synth.quaternions(1, 1), device=dev)
    cache = iq.PagedCache(4, 1, device=dev, zero=True)
    bt = torch.arange(2, dtype=torch.int32, device=dev)
    k = torch.zeros((10, 1, 128), dtype=torch.bfloat16, device=dev)
    q = torch.zeros((1, 1, 128), dtype=torch.bfloat16, device=dev)
    with pytest.raises(RuntimeError):  # the chunk runs past the block table (128 positions)
        iq.prefill_append(cache, rot, k, k, 120, q, 0, bt)
    with pytest.raises(RuntimeError):  # the queries run past it
        iq.prefill_append(cache, rot, k, k, 0, q, 128, bt)
    ws = torch.zeros(16, dtype=torch.uint8, device=dev)
    with pytest.raises(RuntimeError):  # a workspace without the counter region
        iq.prefill_append(cache, rot, k, k, 0, q, 0, bt, workspace=ws)
