"""Merge of the decode splits and determinism, through the C ABI.

The merge workgroups of the split launch (on request, where the whole grid can
be resident at once) and the separate merge kernel merge the same partial rows
with the same code, so with a fixed page order inside each split (the
deterministic option) both give bit-identical outputs, run after run; both are
within the tolerance of the oracle; and the arrival counters at the head of the
workspace are zero again after every call, so a workspace can be reused by
calls of any shape.  Graph replays of fused-merge steps match the eager runs.
The merge kernel's three chunk sizes (slots each thread loads at once, chosen
from the plan's slot count) each match the oracle.
"""

import numpy as np
import pytest
import torch

from tests.gpu_cases import Scenario, max_row_error, tol

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():
    pytest.skip("needs a GPU", allow_module_level=True)

from compressed_space_attention_amd import isoquant as iq  # noqa: E402


def _say(*a):
    print(*a, flush=True)


CASES = [
    # (lens, hkv, hq, dtype, bits, merge workgroups expected in the split launch)
    ([4096], 4, 32, "bf16", 3, True),          # one sequence, group 8 (the 32K shape at 1/8 length)
    ([3000, 1500], 2, 16, "bf16", 3, True),    # host plan over two sequences
    ([0, 700], 2, 8, "bf16", 3, True),         # an empty sequence: zeros from its merge workgroups
    ([130], 1, 16, "f16", 3, True),            # group 16: one score tile per token block
    ([5000, 64, 1], 4, 24, "bf16", 3, True),   # group 6, a one-page and a one-token sequence
    ([4096], 4, 32, "bf16", 4, False),         # 4-bit pages: the workgroup's LDS leaves no room
]


@pytest.mark.parametrize("case", range(len(CASES)))
def test_merge_modes_agree_bit_for_bit(case):
    lens, hkv, hq, dtype, bits, fused = CASES[case]
    _say(f"merge modes lens={lens} hkv={hkv} hq={hq} bits={bits} fused expected={fused}")
    s = Scenario(2100 + case, lens, hkv=hkv, dtype=dtype, outliers=True, bits=bits)
    q = s.queries(2200 + case, len(lens), hq).cuda()
    det = iq.DecodeOptions(plan=iq.IQ_PLAN_HOST, deterministic=1, merge=iq.IQ_MERGE_FUSED)
    ker = iq.DecodeOptions(plan=iq.IQ_PLAN_HOST, deterministic=1, merge=iq.IQ_MERGE_KERNEL)
    info = iq.decode_describe(len(lens), hq, hkv, max(lens), bits, False, det)
    _say(f"  plan {info}")
    assert info["fused_merge"] == int(fused)
    assert iq.decode_describe(len(lens), hq, hkv, max(lens), bits, False, ker)["fused_merge"] == 0
    nbytes = max(iq.decode_workspace_bytes(len(lens), hq, hkv, max(lens), det),
                 iq.decode_workspace_bytes(len(lens), hq, hkv, max(lens)))    # the default plan too
    ws = torch.zeros(nbytes, dtype=torch.uint8, device="cuda")
    outs = [iq.decode_attention(s.cache, s.rot, q, s.bt_dev, s.lens_dev, max(lens), workspace=ws,
                                options=det) for _ in range(3)]
    out_k = iq.decode_attention(s.cache, s.rot, q, s.bt_dev, s.lens_dev, max(lens), workspace=ws, options=ker)
    out_auto = iq.decode_attention(s.cache, s.rot, q, s.bt_dev, s.lens_dev, max(lens), workspace=ws)
    torch.cuda.synchronize()
    assert int(torch.count_nonzero(ws[:iq.DECODE_COUNTER_BYTES])) == 0, "counters left nonzero"
    for o in outs[1:] + [out_k]:
        assert torch.equal(o, outs[0]), "deterministic runs differ"
    ref = s.oracle_decode(s.host_cache(), q.double().cpu().numpy())
    o = outs[0].cpu().numpy()
    err = max_row_error(o, ref)
    err_auto = max_row_error(out_auto.cpu().numpy(), ref)
    _say(f"  max row error {err:.3e} (deterministic), {err_auto:.3e} (default options)")
    assert np.all(np.isfinite(o))
    assert err <= tol() and err_auto <= tol()
    for b, n in enumerate(lens):
        if n == 0:
            assert np.all(o[b] == 0)


def test_deterministic_balanced_plan_repeats_bit_for_bit():
    """The device-balanced plan (eight waves) with a fixed page order."""
    lens = [9000, 20000, 300, 4100]
    s = Scenario(2300, lens, hkv=4, dtype="bf16", outliers=True)
    q = s.queries(2301, len(lens), 16).cuda()
    det = iq.DecodeOptions(deterministic=1, waves=8)
    a = iq.decode_attention(s.cache, s.rot, q, s.bt_dev, s.lens_dev, max(lens), options=det)
    b = iq.decode_attention(s.cache, s.rot, q, s.bt_dev, s.lens_dev, max(lens), options=det)
    assert torch.equal(a, b)
    ref = s.oracle_decode(s.host_cache(), q.double().cpu().numpy())
    assert max_row_error(a.cpu().numpy(), ref) <= tol()


def test_workspace_reused_across_shapes():
    """One workspace, calls of different shapes and plans in a row (the
    counters each call leaves at zero are where the next one looks)."""
    a = Scenario(2400, [2000], hkv=2, dtype="bf16")
    b = Scenario(2401, [700, 64, 3000], hkv=4, dtype="bf16", outliers=True)
    qa = a.queries(2402, 1, 16).cuda()
    qb = b.queries(2403, 3, 32).cuda()
    host = iq.DecodeOptions(plan=iq.IQ_PLAN_HOST, merge=iq.IQ_MERGE_FUSED)
    n = max(iq.decode_workspace_bytes(1, 16, 2, 2000), iq.decode_workspace_bytes(3, 32, 4, 3000, host),
            iq.decode_workspace_bytes(3, 32, 4, 3000))
    ws = torch.zeros(n, dtype=torch.uint8, device="cuda")
    ra = a.oracle_decode(a.host_cache(), qa.double().cpu().numpy())
    rb = b.oracle_decode(b.host_cache(), qb.double().cpu().numpy())
    for _ in range(2):
        oa = iq.decode_attention(a.cache, a.rot, qa, a.bt_dev, a.lens_dev, 2000, workspace=ws)
        ob = iq.decode_attention(b.cache, b.rot, qb, b.bt_dev, b.lens_dev, 3000, workspace=ws, options=host)
        oc = iq.decode_attention(b.cache, b.rot, qb, b.bt_dev, b.lens_dev, 3000, workspace=ws)
        torch.cuda.synchronize()
        assert max_row_error(oa.cpu().numpy(), ra) <= tol()
        assert max_row_error(ob.cpu().numpy(), rb) <= tol()
        assert max_row_error(oc.cpu().numpy(), rb) <= tol()
    assert int(torch.count_nonzero(ws[:iq.DECODE_COUNTER_BYTES])) == 0


def test_fused_merge_step_graph_replays():
    """A stack of three one-sequence decode steps (merge workgroups in the
    split launch) captured in a graph and replayed, with eager work between
    replays: every replay equals the eager run bit for bit (fixed page order)."""
    layers = [Scenario(2500 + i, [3000], hkv=4, dtype="bf16", outliers=True, hold_last=True) for i in range(3)]
    qs = [s.queries(2510 + i, 1, 32).cuda() for i, s in enumerate(layers)]
    det = iq.DecodeOptions(deterministic=1, merge=iq.IQ_MERGE_FUSED)
    assert iq.decode_describe(1, 32, 4, 3000, 3, True, det)["fused_merge"] == 1
    ws = iq.decode_workspace(1, 32, 4, 3000, det)
    outs = [torch.empty((1, 32, 128), dtype=torch.float32, device="cuda") for _ in layers]

    def stack():
        for s, q, o in zip(layers, qs, outs):
            iq.decode_step(s.cache, s.rot, q, s.k_last, s.v_last, s.bt_dev, s.lens_dev, 3000, out=o,
                           workspace=ws, options=det)

    stack()
    torch.cuda.synchronize()
    eager = [o.clone() for o in outs]
    refs = [s.oracle_decode(s.host_cache(), q.double().cpu().numpy()) for s, q in zip(layers, qs)]
    for e, r in zip(eager, refs):
        assert max_row_error(e.cpu().numpy(), r) <= tol()
    g = torch.cuda.CUDAGraph()
    st = torch.cuda.Stream()
    st.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(st):
        with torch.cuda.graph(g, stream=st):
            stack()
    torch.cuda.current_stream().wait_stream(st)
    for rep in range(4):
        for o in outs:
            o.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        for o, e in zip(outs, eager):
            assert torch.equal(o, e), f"replay {rep} differs"
        assert int(torch.count_nonzero(ws[:iq.DECODE_COUNTER_BYTES])) == 0


CHUNK_CASES = [
    # (lens, hkv, hq, slots range): the merge kernel's chunk is 4 slots per
    # thread up to 32 slots, 8 up to 64 and 16 beyond; every regime and a
    # balanced plan whose sequences use fewer slots than the rows hold
    ([4096], 8, 16, (1, 32)),
    ([4096], 4, 32, (33, 64)),
    ([8192], 1, 8, (65, 256)),
    ([8192, 3000, 64], 1, 8, (65, 256)),
]


@pytest.mark.parametrize("case", range(len(CHUNK_CASES)))
def test_merge_chunk_regimes_match_oracle(case):
    lens, hkv, hq, (lo, hi) = CHUNK_CASES[case]
    _say(f"merge chunk regime lens={lens} hkv={hkv} hq={hq}")
    info = iq.decode_describe(len(lens), hq, hkv, max(lens), 3, False)
    _say(f"  plan {info}")
    assert lo <= info["splits"] <= hi
    s = Scenario(2300 + case, lens, hkv=hkv, dtype="bf16", outliers=True)
    q = s.queries(2400 + case, len(lens), hq).cuda()
    ws = torch.zeros(iq.decode_workspace_bytes(len(lens), hq, hkv, max(lens)), dtype=torch.uint8, device="cuda")
    det = iq.DecodeOptions(deterministic=1)
    a = iq.decode_attention(s.cache, s.rot, q, s.bt_dev, s.lens_dev, max(lens), workspace=ws, options=det)
    b = iq.decode_attention(s.cache, s.rot, q, s.bt_dev, s.lens_dev, max(lens), workspace=ws, options=det)
    torch.cuda.synchronize()
    assert torch.equal(a, b), "deterministic runs differ"
    ref = s.oracle_decode(s.host_cache(), q.double().cpu().numpy())
    err = max_row_error(a.cpu().numpy(), ref)
    _say(f"  max row error {err:.3e}")
    assert err <= tol()
