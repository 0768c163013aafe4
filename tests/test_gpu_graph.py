"""A multi-layer stack of decode steps captured in a HIP graph (torch.cuda.CUDAGraph)
and replayed: every replay must give what eager calls give (within the
run-to-run spread of in-split page claiming, 0.5 x the attention tolerance)
and stay within the oracle tolerance; the appended records must be those of
the eager step.  Replays are interleaved with eager work and synchronisations,
and no graph node clears memory (the library enqueues kernels only)."""

import numpy as np
import pytest
import torch

from oracle import isoquant_oracle as O
from tests.gpu_cases import Scenario, max_row_error, tol

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():
    pytest.skip("needs a GPU", allow_module_level=True)


def test_decode_step_stack_graph_replays():
    lens = [700, 1301]
    layers = [Scenario(1100 + i, lens, hkv=2, dtype="bf16", outliers=(i == 1), hold_last=True)
              for i in range(3)]
    qs = [s.queries(1200 + i, len(lens), 16).cuda() for i, s in enumerate(layers)]
    iq = layers[0].iq
    ws = iq.decode_workspace(len(lens), 16, 2, max(lens))
    outs = [torch.empty((len(lens), 16, 128), dtype=torch.float32, device="cuda") for _ in layers]

    def stack():
        for s, q, o in zip(layers, qs, outs):
            iq.decode_step(s.cache, s.rot, q, s.k_last, s.v_last, s.bt_dev, s.lens_dev, max(lens),
                           out=o, workspace=ws)

    stack()
    torch.cuda.synchronize()
    eager = [o.cpu().numpy().copy() for o in outs]
    caches = [s.cache.to_host() for s in layers]
    refs = [O.decode_attention(s.host_cache(), s.blocks, q.double().cpu().numpy(), s.block_table, lens)
            for s, q in zip(layers, qs)]
    for e, r in zip(eager, refs):
        assert max_row_error(e, r) <= tol()

    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        with torch.cuda.graph(g, stream=side):
            stack()
    torch.cuda.current_stream().wait_stream(side)
    for rep in range(3):
        for o in outs:
            o.fill_(float("nan"))          # eager work between replays
        g.replay()
        torch.cuda.synchronize()
        for i, (o, e, r) in enumerate(zip(outs, eager, refs)):
            got = o.cpu().numpy()
            assert np.all(np.isfinite(got)), (rep, i)
            assert max_row_error(got, e) <= 0.5 * tol(), (rep, i)
            assert max_row_error(got, r) <= tol(), (rep, i)
        for s, c in zip(layers, caches):
            for a, b in zip(s.cache.to_host(), c):
                assert np.array_equal(a, b)
