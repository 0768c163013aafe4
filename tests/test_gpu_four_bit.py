"""4-bit records on the GPU against the 4-bit oracle, through the C-ABI.

Same bar as the 3-bit path: codes bit for bit except coordinates within 1e-6
of a decision boundary (count reported, below 1e-5 of all codes), packed bytes
identical wherever the codes agree, norms bit for bit outside the fp16
rounding-midpoint exemption; attention max_rows max|gpu - oracle| / max|oracle|
<= 1e-3 with the oracle attending over the GPU-written cache.  A decode step
must write the records a separate append writes, byte for byte.
"""


import numpy as np
import pytest
import torch

from compressed_space_attention_amd import synth
from oracle import isoquant4_oracle as O4
from oracle import isoquant_oracle as O
from tests.gpu_cases import Scenario, code_parity4, max_row_error, tol

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():
    pytest.skip("needs a GPU", allow_module_level=True)


def _say(*a):
    print(*a, flush=True)


def _with_waves(waves, fn):
    """fn(options) with `waves` waves per decode workgroup (None: the planner's choice)."""
    from compressed_space_attention_amd import isoquant as iq
    return fn(iq.DecodeOptions(waves=waves or 0))


SMALL_LENS = [1, 100, 700, 64]     # 6920 vectors: the 32-lanes-per-vector kernel
LARGE_LENS = [2100, 77, 64]        # 17928 vectors: the 4-lanes-per-vector kernel


@pytest.mark.parametrize("lens", [SMALL_LENS, LARGE_LENS], ids=["lanes32", "quads"])
@pytest.mark.parametrize("dtype,outliers", [("f32", False), ("bf16", True), ("f16", False)])
def test_quantize4_codes_and_norms(dtype, outliers, lens):
    _say(f"4-bit quantize parity dtype={dtype} outliers={outliers} tokens={sum(lens)}")
    s = Scenario(1021, lens, hkv=4, dtype=dtype, outliers=outliers, bits=4)
    ref, info = s.oracle_cache()
    st = code_parity4(s.host_cache(), ref, info, s)
    _say(" ", st)
    assert st["mismatch"] <= st["near"]
    assert st["mismatch"] < 1e-5 * st["codes"] + 1


@pytest.mark.parametrize("n_pad", [0, 20000], ids=["lanes32", "quads"])
def test_quantize4_closed_form_vectors(n_pad):
    """Identity rotation (T = H / sqrt(d)): a zero vector gives code 8 and norm
    0; 3 e_0 gives u = 1 everywhere (code 11); a quarter of Hadamard column 37
    gives u = sqrt(128) at 37 (code 15) and 0 elsewhere (code 8); -2 e_5 gives
    u = -1 or +1 by the column's signs (codes 4 and 11)."""
    n = 5 + n_pad
    k = torch.zeros((n, 1, 128), dtype=torch.float32)
    k[1, 0, 0] = 3.0
    k[2, 0] = torch.from_numpy(O.sylvester_hadamard()[:, 37] * 0.25)
    k[3, 0, 5] = -2.0
    k[4] = torch.from_numpy(synth.normal(3, (1, 128)))
    if n_pad:
        k[5:] = torch.from_numpy(synth.normal(4, (n_pad, 1, 128)))
    s = Scenario(1031, [n], hkv=1, dtype="f32", identity=True, kv_override=(k, k.clone()), bits=4)
    ref, info = s.oracle_cache()
    code_parity4(s.host_cache(), ref, info, s)
    g = s.host_cache()
    pg = s.block_table[0, 0]
    for which in ("k", "v"):
        codes = g.codes(which, np.full(4, pg), 0, np.arange(4))
        assert np.all(codes[0] == 8)
        assert getattr(g, which + "_norms")[pg, 0, 0] == 0
        assert np.all(codes[1] == 11)
        want = np.full(128, 8)
        want[37] = 15
        assert np.array_equal(codes[2], want)
        col = O.sylvester_hadamard()[:, 5]
        assert np.array_equal(codes[3], np.where(col > 0, 4, 11))


DECODE4_CASES = [
    # (lens, hkv, hq, dtype, outliers, waves per workgroup or None)
    ([2048], 1, 1, "f32", False, None),
    ([1, 63, 64, 65, 700], 2, 4, "bf16", True, None),
    ([130, 1000, 2100], 4, 32, "bf16", True, 8),     # group 8, eight waves
    ([640, 33], 2, 32, "f16", False, None),          # group 16
    ([5000], 4, 32, "bf16", True, 4),                # four waves over many pages
]


@pytest.mark.parametrize("case", range(len(DECODE4_CASES)))
def test_decode4_matches_oracle_on_gpu_cache(case):
    lens, hkv, hq, dtype, outl, waves = DECODE4_CASES[case]
    _say(f"4-bit decode parity lens={lens} hkv={hkv} hq={hq} dtype={dtype} waves={waves}")
    s = Scenario(1100 + case, lens, hkv=hkv, dtype=dtype, outliers=outl, bits=4)
    q = s.queries(1200 + case, len(lens), hq)
    out = _with_waves(waves, lambda o: s.iq.decode_attention(s.cache, s.rot, q.cuda(), s.bt_dev,
                                                               s.lens_dev, max(lens), options=o))
    torch.cuda.synchronize()
    ref = s.oracle_decode(s.host_cache(), q.double().numpy())
    o = out.cpu().numpy()
    err = max_row_error(o, ref)
    _say(f"  max row error {err:.3e}")
    assert np.all(np.isfinite(o))
    assert err <= tol()


STEP4_CASES = [
    ([2048], 1, 1, "f32", False, None),                 # the new token fills a page's last slot
    ([1, 63, 64, 65, 700], 2, 4, "bf16", True, None),   # alone in the cache; first slot of a page
    ([130, 1000, 2100], 4, 32, "bf16", True, 8),
    ([640, 33], 2, 32, "f16", False, None),
    ([0, 5, 129], 2, 16, "bf16", False, 8),             # an empty sequence appends nothing
]


@pytest.mark.parametrize("case", range(len(STEP4_CASES)))
def test_decode4_step_matches_append_then_decode(case):
    lens, hkv, hq, dtype, outl, waves = STEP4_CASES[case]
    _say(f"4-bit decode step lens={lens} hkv={hkv} hq={hq} dtype={dtype} waves={waves}")
    full = Scenario(1300 + case, lens, hkv=hkv, dtype=dtype, outliers=outl, bits=4)
    step = Scenario(1300 + case, lens, hkv=hkv, dtype=dtype, outliers=outl, bits=4,
                    kv_override=(full.k, full.v), hold_last=True)
    q = step.queries(1400 + case, len(lens), hq).cuda()
    out = _with_waves(waves, lambda o: step.iq.decode_step(
        step.cache, step.rot, q, step.k_last, step.v_last, step.bt_dev, step.lens_dev, max(lens), options=o))
    pair = _with_waves(waves, lambda o: full.iq.decode_attention(
        full.cache, full.rot, q, full.bt_dev, full.lens_dev, max(lens), options=o))
    torch.cuda.synchronize()
    for a, b in zip(step.cache.to_host(), full.cache.to_host()):
        assert np.array_equal(a, b)
    ref_cache, info = full.oracle_cache()
    _say(" ", code_parity4(step.host_cache(), ref_cache, info, full))
    ref = step.oracle_decode(step.host_cache(), q.double().cpu().numpy())
    o = out.cpu().numpy()
    err = max_row_error(o, ref)
    _say(f"  max row error {err:.3e}")
    assert np.all(np.isfinite(o))
    assert err <= tol()
    assert max_row_error(o, pair.cpu().numpy()) <= 0.5 * tol()
    for b, n in enumerate(lens):
        if n == 0:
            assert np.all(o[b] == 0)


def test_decode4_single_token_is_its_value():
    """Context 1: every head's output is the dequantised new value row."""
    s = Scenario(1460, [1, 1], hkv=2, dtype="bf16", hold_last=True, bits=4)
    q = s.queries(1461, 2, 8).cuda()
    out = s.iq.decode_step(s.cache, s.rot, q, s.k_last, s.v_last, s.bt_dev, s.lens_dev, 1).cpu().numpy()
    hc = s.host_cache()
    for b in range(2):
        for h in range(2):
            vc, vn = hc.gather(s.block_table, b, 1, h, "v")
            v0 = O.inverse_rotate(O4.dequantize_rotated4(vc, vn), s.blocks[h])[0]
            rows = out[b, 4 * h:4 * h + 4]
            assert np.max(np.abs(rows - v0)) <= 1e-3 * np.max(np.abs(v0))


PREFILL4_CASES = [
    # (cache length, n_q, hkv, hq, waves per workgroup or None): groups 1..128,
    # ragged last tiles, a single query, both workgroup shapes
    (1000, 200, 2, 16, None),
    (300, 300, 1, 1, None),
    (700, 77, 2, 8, 4),
    (640, 1, 2, 4, None),
    (200, 70, 1, 128, 4),
    # causal ranges of one to three pages (pipeline start and end)
    (130, 130, 1, 2, None),
    (10, 10, 2, 8, 4),
]


@pytest.mark.parametrize("case", range(len(PREFILL4_CASES)))
def test_prefill4_matches_oracle(case):
    total, n_q, hkv, hq, waves = PREFILL4_CASES[case]
    _say(f"4-bit prefill parity total={total} n_q={n_q} hkv={hkv} hq={hq} waves={waves}")
    s = Scenario(1500 + case, [total], hkv=hkv, dtype="bf16", bits=4)
    q = synth.to_dtype(synth.normal(1501 + case, (n_q, hq, 128)), "bf16")
    q_start = total - n_q
    out = s.iq.prefill_attention(s.cache, s.rot, q.cuda(), q_start, s.bt_dev[0], waves=waves or 0).cpu().numpy()
    rows = np.unique(np.linspace(0, n_q - 1, min(n_q, 24)).astype(int))
    ref = O4.prefill_attention4(s.host_cache(), s.blocks, q.double().numpy(), q_start, s.block_table[0],
                                rows=rows)
    err = max_row_error(out[rows], ref)
    _say(f"  max row error {err:.3e}")
    assert np.all(np.isfinite(out))
    assert err <= tol()


def test_prefill4_varlen_matches_oracle_and_single_calls():
    lens, nq, hkv, hq = [700, 130, 2048, 64], [77, 0, 128, 64], 2, 16
    s = Scenario(1560, lens, hkv=hkv, dtype="bf16", bits=4)
    total_q = sum(nq)
    q = synth.to_dtype(synth.normal(1561, (total_q, hq, 128)), "bf16")
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
        ref = O4.prefill_attention4(host, s.blocks, q[cu[b]:cu[b + 1]].double().numpy(), int(starts[b]),
                                    s.block_table[b], rows=rows)
        worst = max(worst, max_row_error(out[cu[b] + rows], ref))
        one = s.iq.prefill_attention(s.cache, s.rot, q[cu[b]:cu[b + 1]].cuda(), int(starts[b]),
                                     s.bt_dev[b]).cpu().numpy()
        assert np.array_equal(one, out[cu[b]:cu[b + 1]])
    _say(f"  max row error {worst:.3e}")
    assert worst <= tol()


def test_prefill4_agrees_with_decode4_on_the_last_query():
    """The last query of a chunk attends the whole cache: prefill's row and the
    decode call on the same 4-bit cache agree (two different kernels)."""
    total, n_q, hkv, hq = 900, 33, 2, 16
    s = Scenario(1570, [total], hkv=hkv, dtype="bf16", bits=4)
    q = synth.to_dtype(synth.normal(1571, (n_q, hq, 128)), "bf16")
    pre = s.iq.prefill_attention(s.cache, s.rot, q.cuda(), total - n_q, s.bt_dev[0]).cpu().numpy()
    dec = s.iq.decode_attention(s.cache, s.rot, q[-1:].contiguous().cuda(), s.bt_dev, s.lens_dev,
                                total).cpu().numpy()
    assert max_row_error(pre[-1:], dec) <= tol()
