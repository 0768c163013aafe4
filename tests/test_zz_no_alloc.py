"""The no-allocation decode step (iq_decode_step_noalloc: split partials in the
library's static per-GPU scratch) against iq_decode_step with a workspace,
through the C ABI, on two calls in a row, the second with a smaller input.

Both calls run the same kernels on identical copies of the inputs: the caches
after the step must be byte-identical, the outputs within half the tolerance
of each other, and both within the tolerance of the oracle over the
GPU-written cache."""

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


def _pair(seed, lens, hkv, hq, bits):
    """Two identical scenarios (the new token of each sequence held back)."""
    a = Scenario(seed, lens, hkv=hkv, dtype="bf16", outliers=True, hold_last=True, bits=bits)
    b = Scenario(seed, lens, hkv=hkv, dtype="bf16", outliers=True, hold_last=True, bits=bits,
                 kv_override=(a.k, a.v))
    return a, b


@pytest.mark.parametrize("bits", [3, 4])
def test_noalloc_step_matches_workspace_step(bits):
    # first call: one 32K-like sequence (shortened), then a smaller batch
    calls = [([8192], 4, 32), ([700, 1, 2000], 2, 8)]
    for i, (lens, hkv, hq) in enumerate(calls):
        _say(f"no-alloc decode step call {i}: lens={lens} hkv={hkv} hq={hq} bits={bits}")
        a, b = _pair(3100 + 10 * i + bits, lens, hkv, hq, bits)
        q = a.queries(3200 + 10 * i + bits, len(lens), hq).cuda()
        out_a = torch.full((len(lens), hq, 128), float("nan"), dtype=torch.float32, device="cuda")
        iq.decode_step_noalloc(a.cache, a.rot, q, a.k_last, a.v_last, a.bt_dev, a.lens_dev, max(lens), out_a)
        out_b = iq.decode_step(b.cache, b.rot, q, b.k_last, b.v_last, b.bt_dev, b.lens_dev, max(lens))
        torch.cuda.synchronize()
        for x, y in zip(a.cache.to_host(), b.cache.to_host()):
            assert np.array_equal(x, y), "the caches after the step differ"
        ref = a.oracle_decode(a.host_cache(), q.double().cpu().numpy())
        oa, ob = out_a.cpu().numpy(), out_b.cpu().numpy()
        err_a, err_b, err_ab = max_row_error(oa, ref), max_row_error(ob, ref), max_row_error(oa, ob)
        _say(f"  max row error {err_a:.3e} (no-alloc), {err_b:.3e} (workspace), {err_ab:.3e} between them")
        assert np.all(np.isfinite(oa))
        assert err_a <= tol() and err_b <= tol()
        assert err_ab <= 0.5 * tol()
