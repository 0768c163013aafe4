"""HIP path vs CPU oracle, element by element, through the C-ABI.

Codes must match bit for bit except coordinates within 1e-6 of a decision
boundary (their count is reported and must stay below 1e-5 of all codes);
norms bit for bit except values within 1e-6 of an fp16 rounding midpoint.
Attention outputs must satisfy max_rows max|gpu - oracle| / max|oracle| <= 1e-3,
with the oracle attending over the GPU-written cache.
"""


import numpy as np
import pytest
import torch

from compressed_space_attention_amd import synth
from oracle import isoquant_oracle as O
from tests.gpu_cases import Scenario, code_parity, max_row_error, tol

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():
    pytest.skip("needs a GPU", allow_module_level=True)


def _say(*a):
    print(*a, flush=True)


def test_rotation_matrices_match_oracle():
    from compressed_space_attention_amd import isoquant as iq
    quats = synth.quaternions(11, 5) * 3.0
    rot = iq.rotation_init(quats)
    torch.cuda.synchronize()
    mats = rot[: 5 * 32 * 16 * 4].view(torch.float32).cpu().numpy().reshape(5, 32, 4, 4)
    want = O.rotation_matrices(quats)
    assert np.max(np.abs(mats - want)) < 1e-6


# Up to 16384 vectors (K and V together) an append takes the 32-lanes-per-vector
# kernel, above it the 4-lanes-per-vector one: both are covered.
SMALL_LENS = [1, 100, 700, 64]     # 865 tokens x 4 heads x 2 = 6920 vectors
LARGE_LENS = [2100, 77, 64]        # 2241 tokens x 4 heads x 2 = 17928 vectors


@pytest.mark.parametrize("lens", [SMALL_LENS, LARGE_LENS], ids=["lanes32", "quads"])
@pytest.mark.parametrize("dtype,outliers", [("f32", False), ("bf16", True), ("f16", False)])
def test_quantize_append_codes_and_norms(dtype, outliers, lens):
    _say(f"quantize parity dtype={dtype} outliers={outliers} tokens={sum(lens)}")
    s = Scenario(21, lens, hkv=4, dtype=dtype, outliers=outliers)
    ref, info = s.oracle_cache()
    st = code_parity(s.host_cache(), ref, info, s)
    _say(st)
    assert st["mismatch"] <= st["near"]
    assert st["mismatch"] < 1e-5 * st["codes"] + 1


def _special_vectors(k, at):
    """Closed-form cases at tokens at .. at + 5 of k ([n][1][128] fp32)."""
    k[at:at + 6] = 0.0                                     # at: zero vector -> all codes 4, norm 0
    k[at + 1, 0, 0] = 3.0                                  # e_0 -> all codes 5
    k[at + 2, 0] = torch.from_numpy(O.sylvester_hadamard()[:, 37] * 0.25)  # -> code 7 at 37, else 4
    k[at + 3, 0] = 1e5                                     # norm 1.13e6 -> saturates at 65504
    k[at + 4, 0, 5] = -2.0                                 # -e_5 -> u = -1 or +1 by Hadamard sign
    k[at + 5] = torch.from_numpy(synth.normal(3, (1, 128)))


@pytest.mark.parametrize("n", [6, 8300], ids=["lanes32", "quads"])
def test_quantize_special_vectors(n):
    """Zero vectors, a huge norm (fp16 saturation), identity rotation with a
    Hadamard column and a basis vector (closed-form codes), through both append
    kernels: 6 tokens take the 32-lanes-per-vector kernel; 8,300 tokens the
    quad kernel, with the cases on its first (whole, LDS-assembled) page and on
    its last, partial page."""
    k = torch.from_numpy(synth.normal(29, (n, 1, 128))).float()
    bases = [0] if n < 64 else [0, n - 10]
    for at in bases:
        _special_vectors(k, at)
    v = k.clone()
    s = Scenario(31, [n], hkv=1, dtype="f32", identity=True, kv_override=(k, v))
    ref, info = s.oracle_cache()
    code_parity(s.host_cache(), ref, info, s)
    g = s.host_cache()
    want = np.full(128, 4)
    want[37] = 7
    for at in bases:
        page, slot = s.block_table[0, at // 64], at % 64
        assert slot + 6 <= 64
        # K records are slot-ordered (V records, in the matrix-core order, are
        # checked against the oracle by code_parity above)
        codes = O.unpack_codes(g.k_codes[page, 0, slot:slot + 6])
        assert np.all(codes[0] == 4)
        assert np.all(codes[1] == 5)
        assert np.array_equal(codes[2], want)
        for norms in (g.k_norms, g.v_norms):
            assert norms[page, 0, slot] == 0 and norms[page, 0, slot + 3] == 0x7BFF


@pytest.mark.parametrize("n_tok", [3, 5000], ids=["lanes32", "quads"])
def test_quantize_skips_positions_outside_the_table(n_tok):
    """A position past the block table, or a table entry that is no page of the
    cache, writes nothing (and reads nothing out of bounds)."""
    from compressed_space_attention_amd import isoquant as iq
    s = Scenario(41, [64], hkv=2, dtype="f32")
    before = [t.clone() for t in (s.cache.k_codes, s.cache.v_codes, s.cache.k_norms, s.cache.v_norms)]
    k = torch.from_numpy(synth.normal(42, (n_tok, 2, 128))).float().cuda()
    max_pages = s.bt_dev.shape[1]
    pos = torch.full((n_tok,), max_pages * 64 + 5, dtype=torch.int32, device="cuda")
    seq = torch.zeros(n_tok, dtype=torch.int32, device="cuda")
    iq.quantize_append(s.cache, s.rot, k, k, seq, pos, s.bt_dev)
    bad_bt = torch.full_like(s.bt_dev, s.num_pages + 7)
    pos2 = torch.zeros(n_tok, dtype=torch.int32, device="cuda")
    iq.quantize_append(s.cache, s.rot, k, k, seq, pos2, bad_bt)
    torch.cuda.synchronize()
    after = (s.cache.k_codes, s.cache.v_codes, s.cache.k_norms, s.cache.v_norms)
    for a, b in zip(before, after):
        assert torch.equal(a, b)


DECODE_CASES = [
    # (lens, hkv, hq, dtype, outliers)
    ([2048], 1, 1, "f32", False),
    ([1, 63, 64, 65, 700], 2, 4, "bf16", True),
    ([130, 1000, 2100], 4, 32, "bf16", True),
    ([640, 33], 2, 32, "f16", False),
    # one sequence at the prefill staging limit (4,096 pages, 16 per split)
    ([262144], 1, 8, "bf16", True),
]


@pytest.mark.parametrize("case", range(len(DECODE_CASES)))
def test_decode_matches_oracle_on_gpu_cache(case):
    lens, hkv, hq, dtype, outl = DECODE_CASES[case]
    _say(f"decode parity lens={lens} hkv={hkv} hq={hq} dtype={dtype}")
    s = Scenario(100 + case, lens, hkv=hkv, dtype=dtype, outliers=outl)
    q = s.queries(200 + case, len(lens), hq)
    out = s.iq.decode_attention(s.cache, s.rot, q.cuda(), s.bt_dev, s.lens_dev, max(lens))
    torch.cuda.synchronize()
    ref = O.decode_attention(s.host_cache(), s.blocks, q.double().numpy(), s.block_table, lens)
    err = max_row_error(out.cpu().numpy(), ref)
    _say(f"  max row error {err:.3e}")
    assert np.all(np.isfinite(out.cpu().numpy()))
    assert err <= tol()


def test_decode_edge_lengths_and_empty_sequence():
    lens = [0, 1, 64, 129]
    s = Scenario(300, lens, hkv=2, dtype="bf16")
    q = s.queries(301, len(lens), 16)
    out = s.iq.decode_attention(s.cache, s.rot, q.cuda(), s.bt_dev, s.lens_dev, max(lens)).cpu().numpy()
    ref = O.decode_attention(s.host_cache(), s.blocks, q.double().numpy(), s.block_table, lens)
    assert np.all(out[0] == 0)
    assert max_row_error(out, ref) <= tol()
    # context 1: the output is the dequantised value of token 0
    hc = s.host_cache()
    vc, vn = hc.gather(s.block_table, 1, 1, 0, "v")
    v0 = O.dequantize(vc, vn, s.blocks[0])[0]
    assert np.max(np.abs(out[1, :8] - v0)) <= 1e-3 * np.max(np.abs(v0))


def test_decode_split_plans_agree():
    """Pages per split from 1 (one page per workgroup) to 512 (one split per
    sequence, most pages claimed by the waves as they go): every plan is within
    the oracle tolerance and the plans agree with each other.  Plans (and, with
    in-split page claiming, repeated runs of one plan) differ only in where P~
    is rounded to f16 relative to a running maximum, about 2^-11 per weight."""
    lens = [3000, 1500]
    s = Scenario(400, lens, hkv=2, dtype="bf16", outliers=True)
    q = s.queries(401, 2, 16).cuda()
    outs = []
    iq = s.iq
    for pps in (1, 3, 16, 512):            # host plans from the longest length
        opts = iq.DecodeOptions(plan=iq.IQ_PLAN_HOST, pages_per_split=pps)
        outs.append(iq.decode_attention(s.cache, s.rot, q, s.bt_dev, s.lens_dev, 3000, options=opts)
                    .cpu().numpy())
    again = iq.decode_attention(s.cache, s.rot, q, s.bt_dev, s.lens_dev, 3000, options=opts).cpu().numpy()
    # the device-balanced plan
    outs.append(iq.decode_attention(s.cache, s.rot, q, s.bt_dev, s.lens_dev, 3000).cpu().numpy())
    ref = O.decode_attention(s.host_cache(), s.blocks, q.double().cpu().numpy(), s.block_table, lens)
    for o in outs + [again]:
        assert max_row_error(o, ref) <= tol()
        assert max_row_error(o, outs[0]) <= 0.5 * tol()
    assert max_row_error(again, outs[3]) <= 0.5 * tol()


BALANCED_CASES = [
    # (lens, hkv, hq, waves): very unequal lengths, empty and one-token
    # sequences, more sequences than one wave of lanes would hold per kv head
    ([0, 5, 64, 20000, 3000, 1], 2, 16, None),
    ([40000, 64, 65, 128, 100, 7000, 3, 900], 4, 32, 8),
    ([9000] * 3 + [0], 1, 4, 4),
    (list(range(1, 2000, 45)), 2, 4, None),          # 45 sequences
]


@pytest.mark.parametrize("case", range(len(BALANCED_CASES)))
def test_decode_balanced_plan(case):
    """The device-balanced split plan (several sequences) against the oracle
    and against the host plan from the longest length."""
    lens, hkv, hq, waves = BALANCED_CASES[case]
    _say(f"balanced decode lens={lens[:8]}... B={len(lens)} hkv={hkv} hq={hq} waves={waves}")
    s = Scenario(450 + case, lens, hkv=hkv, dtype="bf16", outliers=True)
    q = s.queries(460 + case, len(lens), hq).cuda()
    iq = s.iq
    bal = iq.decode_attention(s.cache, s.rot, q, s.bt_dev, s.lens_dev, max(lens),
                              options=iq.DecodeOptions(waves=waves or 0, plan=iq.IQ_PLAN_BALANCED)).cpu().numpy()
    uni = iq.decode_attention(s.cache, s.rot, q, s.bt_dev, s.lens_dev, max(lens),
                              options=iq.DecodeOptions(waves=waves or 0, plan=iq.IQ_PLAN_HOST)).cpu().numpy()
    ref = O.decode_attention(s.host_cache(), s.blocks, q.double().cpu().numpy(), s.block_table, lens)
    err = max_row_error(bal, ref)
    _say(f"  max row error {err:.3e}")
    assert np.all(np.isfinite(bal))
    assert err <= tol()
    assert max_row_error(bal, uni) <= 0.5 * tol()
    for b, n in enumerate(lens):
        if n == 0:
            assert np.all(bal[b] == 0)


def test_decode_shuffled_equals_contiguous_block_table():
    lens = [777]
    k = synth.kv_vectors(5, 777, 2, "bf16")
    v = synth.kv_vectors(6, 777, 2, "bf16")
    a = Scenario(500, lens, hkv=2, dtype="bf16", shuffle=False, kv_override=(k, v))
    b = Scenario(500, lens, hkv=2, dtype="bf16", shuffle=True, kv_override=(k, v))
    q = a.queries(501, 1, 8).cuda()
    oa = a.iq.decode_attention(a.cache, a.rot, q, a.bt_dev, a.lens_dev, 777).cpu().numpy()
    ob = b.iq.decode_attention(b.cache, b.rot, q, b.bt_dev, b.lens_dev, 777).cpu().numpy()
    assert np.array_equal(oa, ob)


PREFILL_CASES = [
    # (cache length, n_q, hkv, hq): groups 1..128 (1..128 queries per 128-row
    # tile), ragged last tiles, a page-aligned chunk start, a single query
    (1000, 200, 2, 16),
    (300, 300, 1, 1),
    (700, 77, 2, 8),
    (1024, 128, 1, 32),
    (640, 1, 2, 4),
    (200, 70, 1, 128),
    # causal ranges of one to three pages: the page pipeline's start and its
    # steps past the last page
    (64, 64, 1, 1),
    (130, 130, 1, 2),
    (10, 10, 2, 8),
    # the largest causal range one call stages: 4,096 pages
    (262144, 16, 1, 8),
]


@pytest.mark.parametrize("case", range(len(PREFILL_CASES)))
def test_prefill_matches_oracle(case):
    total, n_q, hkv, hq = PREFILL_CASES[case]
    _say(f"prefill parity total={total} n_q={n_q} hkv={hkv} hq={hq}")
    s = Scenario(600 + case, [total], hkv=hkv, dtype="bf16")
    q = synth.to_dtype(synth.normal(601 + case, (n_q, hq, 128)), "bf16")
    q_start = total - n_q
    out = s.iq.prefill_attention(s.cache, s.rot, q.cuda(), q_start, s.bt_dev[0]).cpu().numpy()
    rows = np.unique(np.linspace(0, n_q - 1, min(n_q, 24)).astype(int))
    ref = O.prefill_attention(s.host_cache(), s.blocks, q.double().numpy(), q_start, s.block_table[0],
                              rows=rows)
    err = max_row_error(out[rows], ref)
    _say(f"  max row error {err:.3e}")
    assert err <= tol()


def test_prefill_ignores_unwritten_slots():
    """Slots past the appended chunk hold NaN norm patterns (an uninitialised
    cache): the masked tail of the last page must not reach the output."""
    total, n_q = 700, 60
    s = Scenario(650, [total], hkv=2, dtype="bf16")
    bt = s.block_table[0]
    last_page, first_unwritten = bt[(total - 1) // 64], total % 64
    for norms in (s.cache.k_norms, s.cache.v_norms):
        norms[last_page, :, first_unwritten:] = -1  # 0xFFFF: fp16 NaN
    q = synth.to_dtype(synth.normal(651, (n_q, 16, 128)), "bf16")
    out = s.iq.prefill_attention(s.cache, s.rot, q.cuda(), total - n_q, s.bt_dev[0]).cpu().numpy()
    assert np.all(np.isfinite(out))
    rows = np.array([0, 17, n_q - 1])
    ref = O.prefill_attention(s.host_cache(), s.blocks, q.double().numpy(), total - n_q, bt, rows=rows)
    assert max_row_error(out[rows], ref) <= tol()


VARLEN_CASES = [
    # (cache lengths, queries per sequence (the last ones), hkv, hq)
    ([700, 130, 2048, 64], [77, 0, 128, 64], 2, 16),
    ([300, 1000, 65], [300, 1, 65], 1, 1),
    ([900, 640], [200, 640], 2, 64),
]


@pytest.mark.parametrize("case", range(len(VARLEN_CASES)))
def test_prefill_varlen_matches_oracle_and_single_calls(case):
    lens, nq, hkv, hq = VARLEN_CASES[case]
    _say(f"prefill varlen lens={lens} n_q={nq} hkv={hkv} hq={hq}")
    s = Scenario(680 + case, lens, hkv=hkv, dtype="bf16")
    total_q = sum(nq)
    q = synth.to_dtype(synth.normal(690 + case, (total_q, hq, 128)), "bf16")
    cu = np.concatenate([[0], np.cumsum(nq)]).astype(np.int32)
    starts = np.array([n - k for n, k in zip(lens, nq)], dtype=np.int32)
    out = s.iq.prefill_attention_varlen(
        s.cache, s.rot, q.cuda(), torch.from_numpy(cu).cuda(), torch.from_numpy(starts).cuda(), s.bt_dev,
        max(nq), max(lens)).cpu().numpy()
    host = s.host_cache()
    worst = 0.0
    for b in range(len(lens)):
        if nq[b] == 0:
            continue
        rows = np.unique(np.linspace(0, nq[b] - 1, min(nq[b], 12)).astype(int))
        ref = O.prefill_attention(host, s.blocks, q[cu[b]:cu[b + 1]].double().numpy(), int(starts[b]),
                                  s.block_table[b], rows=rows)
        worst = max(worst, max_row_error(out[cu[b] + rows], ref))
        one = s.iq.prefill_attention(s.cache, s.rot, q[cu[b]:cu[b + 1]].cuda(), int(starts[b]),
                                     s.bt_dev[b]).cpu().numpy()
        assert np.array_equal(one, out[cu[b]:cu[b + 1]])   # the same tiles, the same arithmetic
    _say(f"  max row error {worst:.3e}")
    assert worst <= tol()
