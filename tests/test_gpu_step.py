"""Decode step (iq_decode_step: the current token's quantise-append fused into
decode attention) against the unfused pair and the CPU oracle, through the
C-ABI.

The step must write exactly the records iq_quantize_append writes (the same
quantiser arithmetic, so byte for byte), those records must match the oracle
(codes bit for bit outside the 1e-6 boundary exemption), and the attention
must include the new token: max_rows max|gpu - oracle| / max|oracle| <= 1e-3,
with the oracle attending over the cache holding every token.
"""

import numpy as np
import pytest
import torch

from oracle import isoquant_oracle as O
from tests.gpu_cases import Scenario, code_parity, max_row_error, tol

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():
    pytest.skip("needs a GPU", allow_module_level=True)


def _say(*a):
    print(*a, flush=True)


STEP_CASES = [
    # (lens incl. the new token, hkv, hq, dtype, outliers, waves per workgroup or None)
    ([2048], 1, 1, "f32", False, None),                 # the new token fills a page's last slot
    ([1, 63, 64, 65, 700], 2, 4, "bf16", True, None),   # alone in the cache; first slot of a page
    ([130, 1000, 2100], 4, 32, "bf16", True, None),     # GQA group 8
    ([130, 1000, 2100], 4, 32, "bf16", True, 8),        # ... with eight waves per workgroup
    ([640, 33], 2, 32, "f16", False, None),             # group 16 (one score tile per token block)
    ([0, 5, 129], 2, 16, "bf16", False, 8),             # an empty sequence appends nothing
]


@pytest.mark.parametrize("case", range(len(STEP_CASES)))
def test_decode_step_matches_append_then_decode(case):
    lens, hkv, hq, dtype, outl, waves = STEP_CASES[case]
    _say(f"decode step lens={lens} hkv={hkv} hq={hq} dtype={dtype} waves={waves}")
    full = Scenario(700 + case, lens, hkv=hkv, dtype=dtype, outliers=outl)
    step = Scenario(700 + case, lens, hkv=hkv, dtype=dtype, outliers=outl,
                    kv_override=(full.k, full.v), hold_last=True)
    q = step.queries(800 + case, len(lens), hq).cuda()
    opts = step.iq.DecodeOptions(waves=waves or 0)
    out = step.iq.decode_step(step.cache, step.rot, q, step.k_last, step.v_last, step.bt_dev, step.lens_dev,
                              max(lens), options=opts)
    pair = full.iq.decode_attention(full.cache, full.rot, q, full.bt_dev, full.lens_dev, max(lens),
                                    options=opts)
    torch.cuda.synchronize()
    # the cache after the step is the cache after appending every token
    for a, b in zip(step.cache.to_host(), full.cache.to_host()):
        assert np.array_equal(a, b)
    ref_cache, info = full.oracle_cache()
    _say(" ", code_parity(step.host_cache(), ref_cache, info, full))
    ref = O.decode_attention(step.host_cache(), step.blocks, q.double().cpu().numpy(),
                             step.block_table, lens)
    o = out.cpu().numpy()
    err = max_row_error(o, ref)
    _say(f"  max row error {err:.3e}")
    assert np.all(np.isfinite(o))
    assert err <= tol()
    assert max_row_error(o, pair.cpu().numpy()) <= 0.5 * tol()
    for b, n in enumerate(lens):
        if n == 0:
            assert np.all(o[b] == 0)


# Host plan, four waves, eight pages per split (three splits at 1,536 tokens):
# the step's last wave loads its pages w + 4 and w in that order.  Lengths
# whose last split has exactly eight pages put the sequence's last page in that
# wave's first slot, processed first (full: 1,536; partial: 1,526); the others
# end in splits of six, four, two and one pages (last page in its own buffer,
# the wave's stream starting from its second slot or absent).
SWAP_LENS = [1536, 1526, 1408, 1275, 577, 64, 1]


@pytest.mark.parametrize("bits,hkv,hq,det", [(3, 4, 32, 0), (3, 2, 32, 1), (4, 4, 32, 0), (4, 4, 16, 1)])
def test_decode_step_four_wave_eight_page_splits(bits, hkv, hq, det):
    lens = SWAP_LENS
    _say(f"decode step, 4 waves x 8-page splits, bits={bits} hkv={hkv} hq={hq} det={det} lens={lens}")
    from compressed_space_attention_amd import isoquant as iq
    opts = iq.DecodeOptions(waves=4, pages_per_split=8, plan=iq.IQ_PLAN_HOST, deterministic=det)
    info = iq.decode_describe(len(lens), hq, hkv, max(lens), bits, True, opts)
    assert (info["waves"], info["pages_per_split"], info["splits"], info["balanced"]) == (4, 8, 3, 0)
    seed = 770 + 10 * bits + hkv + det
    full = Scenario(seed, lens, hkv=hkv, dtype="bf16", outliers=True, bits=bits)
    step = Scenario(seed, lens, hkv=hkv, dtype="bf16", outliers=True, bits=bits,
                    kv_override=(full.k, full.v), hold_last=True)
    q = step.queries(seed + 1, len(lens), hq).cuda()
    outs = [step.iq.decode_step(step.cache, step.rot, q, step.k_last, step.v_last, step.bt_dev,
                                step.lens_dev, max(lens), options=opts)]
    pair = full.iq.decode_attention(full.cache, full.rot, q, full.bt_dev, full.lens_dev, max(lens),
                                    options=opts)
    torch.cuda.synchronize()
    for a, b in zip(step.cache.to_host(), full.cache.to_host()):
        assert np.array_equal(a, b)
    ref = step.oracle_decode(step.host_cache(), q.double().cpu().numpy())
    # a second step over the same cache rewrites the same records
    outs.append(step.iq.decode_step(step.cache, step.rot, q, step.k_last, step.v_last, step.bt_dev,
                                    step.lens_dev, max(lens), options=opts))
    torch.cuda.synchronize()
    for a, b in zip(step.cache.to_host(), full.cache.to_host()):
        assert np.array_equal(a, b)
    for out in outs:
        o = out.cpu().numpy()
        err = max_row_error(o, ref)
        _say(f"  max row error {err:.3e}")
        assert np.all(np.isfinite(o))
        assert err <= tol()
        assert max_row_error(o, pair.cpu().numpy()) <= 0.5 * tol()
    if det:
        assert torch.equal(outs[0], outs[1])


def test_decode_step_single_token_is_its_value():
    """Context 1: the output of every head is the dequantised new value row."""
    s = Scenario(760, [1, 1], hkv=2, dtype="bf16", hold_last=True)
    q = s.queries(761, 2, 8).cuda()
    out = s.iq.decode_step(s.cache, s.rot, q, s.k_last, s.v_last, s.bt_dev, s.lens_dev, 1).cpu().numpy()
    hc = s.host_cache()
    for b in range(2):
        for h in range(2):
            vc, vn = hc.gather(s.block_table, b, 1, h, "v")
            v0 = O.dequantize(vc, vn, s.blocks[h])[0]
            rows = out[b, 4 * h:4 * h + 4]
            assert np.max(np.abs(rows - v0)) <= 1e-3 * np.max(np.abs(v0))
