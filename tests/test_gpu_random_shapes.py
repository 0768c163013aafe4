"""Seeded random shapes through the C ABI against the oracle.

The named cases pin chosen shapes; these draw their combinations from a seed
instead: batch 1-5, sequence lengths 1-3,000, kv heads 1/2/4, query groups
1-16 (decode; powers of two for prefill), fp32/bf16/f16 inputs, outlier key
channels or not, 3- and 4-bit records, four or eight waves per decode
workgroup.  Codes are compared with the oracle's quantiser (bit for bit outside
the near-boundary exemption) and attention rows within the same relative
tolerance as the fixed cases; a decode step (the token's append fused into
attention) must leave the cache byte-identical to appending every token first.
"""


import numpy as np
import pytest
import torch

from compressed_space_attention_amd import synth
from oracle import isoquant4_oracle as O4
from oracle import isoquant_oracle as O
from tests.gpu_cases import Scenario, code_parity, code_parity4, max_row_error, tol

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():
    pytest.skip("needs a GPU", allow_module_level=True)


def _say(*a):
    print(*a, flush=True)


def _draw(seed, prefill):
    rng = np.random.default_rng(seed)
    batch = 1 if prefill else int(rng.integers(1, 6))
    lens = [int(x) for x in rng.integers(1, 3001, size=batch)]
    hkv = int(rng.choice([1, 2, 4]))
    group = int(rng.choice([1, 2, 4, 8, 16] if prefill else [1, 2, 3, 4, 6, 8, 12, 16]))
    dtype = "bf16" if prefill else str(rng.choice(["f32", "bf16", "f16"]))
    outliers = bool(rng.integers(0, 2))
    bits = int(rng.choice([3, 4]))
    return lens, hkv, group, dtype, outliers, bits


def _codes(s):
    ref, info = s.oracle_cache()
    check = code_parity4 if s.bits == 4 else code_parity
    return check(s.host_cache(), ref, info, s)


@pytest.mark.parametrize("seed", range(10))
def test_decode_random_shape(seed):
    lens, hkv, group, dtype, outliers, bits = _draw(7000 + seed, prefill=False)
    _say(f"decode random seed={seed} lens={lens} hkv={hkv} group={group} dtype={dtype} "
         f"outliers={outliers} bits={bits}")
    s = Scenario(7100 + seed, lens, hkv=hkv, dtype=dtype, outliers=outliers, bits=bits)
    _say("  codes", _codes(s))
    q = s.queries(7200 + seed, len(lens), hkv * group)
    out = s.iq.decode_attention(s.cache, s.rot, q.cuda(), s.bt_dev, s.lens_dev, max(lens)).cpu().numpy()
    ref = s.oracle_decode(s.host_cache(), q.double().numpy())
    err = max_row_error(out, ref)
    _say(f"  max row error {err:.3e}")
    assert np.all(np.isfinite(out))
    assert err <= tol()


@pytest.mark.parametrize("seed", range(6))
def test_prefill_random_shape(seed):
    lens, hkv, group, dtype, outliers, bits = _draw(7300 + seed, prefill=True)
    total = lens[0]
    n_q = int(np.random.default_rng(7400 + seed).integers(1, min(total, 300) + 1))
    _say(f"prefill random seed={seed} total={total} n_q={n_q} hkv={hkv} group={group} "
         f"outliers={outliers} bits={bits}")
    s = Scenario(7500 + seed, lens, hkv=hkv, dtype=dtype, outliers=outliers, bits=bits)
    q = synth.to_dtype(synth.normal(7600 + seed, (n_q, hkv * group, 128)), "bf16")
    q_start = total - n_q
    out = s.iq.prefill_attention(s.cache, s.rot, q.cuda(), q_start, s.bt_dev[0]).cpu().numpy()
    rows = np.unique(np.linspace(0, n_q - 1, min(n_q, 16)).astype(int))
    fn = O4.prefill_attention4 if bits == 4 else O.prefill_attention
    ref = fn(s.host_cache(), s.blocks, q.double().numpy(), q_start, s.block_table[0], rows=rows)
    err = max_row_error(out[rows], ref)
    _say(f"  max row error {err:.3e}")
    assert np.all(np.isfinite(out))
    assert err <= tol()


@pytest.mark.parametrize("seed", range(6))
def test_decode_step_random_shape(seed):
    lens, hkv, group, dtype, outliers, bits = _draw(7700 + seed, prefill=False)
    waves = int(np.random.default_rng(7800 + seed).choice([4, 8]))
    _say(f"decode step random seed={seed} lens={lens} hkv={hkv} group={group} dtype={dtype} "
         f"outliers={outliers} bits={bits} waves={waves}")
    full = Scenario(7900 + seed, lens, hkv=hkv, dtype=dtype, outliers=outliers, bits=bits)
    step = Scenario(7900 + seed, lens, hkv=hkv, dtype=dtype, outliers=outliers, bits=bits,
                    kv_override=(full.k, full.v), hold_last=True)
    q = step.queries(8000 + seed, len(lens), hkv * group).cuda()
    opts = step.iq.DecodeOptions(waves=waves)
    out = step.iq.decode_step(step.cache, step.rot, q, step.k_last, step.v_last, step.bt_dev,
                              step.lens_dev, max(lens), options=opts)
    pair = full.iq.decode_attention(full.cache, full.rot, q, full.bt_dev, full.lens_dev, max(lens),
                                    options=opts)
    torch.cuda.synchronize()
    for a, b in zip(step.cache.to_host(), full.cache.to_host()):
        assert np.array_equal(a, b)
    o = out.cpu().numpy()
    ref = step.oracle_decode(step.host_cache(), q.double().cpu().numpy())
    err = max_row_error(o, ref)
    _say(f"  max row error {err:.3e}")
    assert np.all(np.isfinite(o))
    assert err <= tol()
    assert max_row_error(o, pair.cpu().numpy()) <= 0.5 * tol()


@pytest.mark.parametrize("seed", range(4))
def test_prefill_varlen_random_shape(seed):
    rng = np.random.default_rng(8100 + seed)
    batch = int(rng.integers(2, 6))
    lens = [int(x) for x in rng.integers(1, 2501, size=batch)]
    nq = [int(rng.integers(0, min(n, 200) + 1)) for n in lens]
    if sum(nq) == 0:
        nq[0] = 1
    hkv = int(rng.choice([1, 2, 4]))
    group = int(rng.choice([1, 2, 4, 8, 16]))
    bits = int(rng.choice([3, 4]))
    _say(f"prefill varlen random seed={seed} lens={lens} n_q={nq} hkv={hkv} group={group} bits={bits}")
    s = Scenario(8200 + seed, lens, hkv=hkv, dtype="bf16", outliers=bool(rng.integers(0, 2)), bits=bits)
    q = synth.to_dtype(synth.normal(8300 + seed, (sum(nq), hkv * group, 128)), "bf16")
    cu = np.concatenate([[0], np.cumsum(nq)]).astype(np.int32)
    starts = np.array([n - k for n, k in zip(lens, nq)], dtype=np.int32)
    out = s.iq.prefill_attention_varlen(
        s.cache, s.rot, q.cuda(), torch.from_numpy(cu).cuda(), torch.from_numpy(starts).cuda(), s.bt_dev,
        max(nq), max(lens)).cpu().numpy()
    host = s.host_cache()
    fn = O4.prefill_attention4 if bits == 4 else O.prefill_attention
    worst = 0.0
    for b in range(batch):
        if nq[b] == 0:
            continue
        rows = np.unique(np.linspace(0, nq[b] - 1, min(nq[b], 8)).astype(int))
        ref = fn(host, s.blocks, q[cu[b]:cu[b + 1]].double().numpy(), int(starts[b]), s.block_table[b], rows=rows)
        worst = max(worst, max_row_error(out[cu[b] + rows], ref))
        one = s.iq.prefill_attention(s.cache, s.rot, q[cu[b]:cu[b + 1]].cuda(), int(starts[b]),
                                     s.bt_dev[b]).cpu().numpy()
        assert np.array_equal(one, out[cu[b]:cu[b + 1]])
    _say(f"  max row error {worst:.3e}")
    assert np.all(np.isfinite(out))
    assert worst <= tol()
