#!/usr/bin/env python3
"""Benchmark of the IsoQuant packed-KV attention path on one MI355X.

Default workload: GQA decode at 32K context (batch 1, 32 query / 4 kv heads,
d = 128, bf16 inputs, 64-token pages, shuffled page table).  One step = one
layer's decode step: quantise-append the current token's K/V into the packed
cache, then decode attention of all query heads over the 32,768 cached tokens.
Steps walk a ring of layer caches (>= 1 GB in total, above the 256 MB
Infinity Cache) so every step reads its packed KV from HBM.  The steps are
recorded once into a HIP graph (torch.cuda.CUDAGraph) and replayed, so the
host's launch rate does not pace the GPU.

Prints one JSON line: metric/value (packed-KV GB/s), the roofline of the
dominant kernel (measured live with HIP events on the launch stream) and the
CPU oracle timed on a bounded sample on the host.
"""

from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0            # MI355X HBM3E, published
MFMA_F16_PEAK_TFLOPS = 2500.0    # MI355X dense f16 matrix peak, published
METRIC = "packed-KV decode attention GB/s (% of HBM peak) + tokens/s at 32K ctx"
REC_BYTES = 100                  # K + V records per (token, kv head): 2 x (48 + 2)
REC_BYTES4 = 132                 # the same with 4-bit records: 2 x (64 + 2)


def parse():
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=2000)
    ap.add_argument("--warmup", type=int, default=160)
    ap.add_argument("--workload", default="gqa_decode_32k_32q4kv")
    ap.add_argument("--bits", type=int, default=3, choices=(3, 4),
                    help="record width of the measured packed cache (3: the method's; 4: the 4-bit variant)")
    ap.add_argument("--ring-bytes", type=float, default=1.0e9,
                    help="minimum bytes of distinct layer caches cycled by the steps")
    ap.add_argument("--cpu-seconds", type=float, default=10.0,
                    help="target CPU time of the oracle baseline sample")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-graph", action="store_true", help="launch eagerly (profiling runs)")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only run a plain device copy of MIB MiB (20 times): the known-size "
                         "reference that scales the HBM byte counters")
    ap.add_argument("--write-traffic-record", metavar="DIR", default=None,
                    help="no GPU work: read the FETCH_SIZE / WRITE_SIZE counter CSVs of the decode "
                         "call and of the copy calibration under DIR (pmc_FETCH_SIZE, pmc_WRITE_SIZE, "
                         "cal_FETCH_SIZE, cal_WRITE_SIZE) and write the traffic record under profiles/")
    ap.add_argument("--no-aux", action="store_true",
                    help="skip the chunked-prefill side measurements (append, prefill)")
    return ap.parse_args()


def log(*a):
    print(*a, file=sys.stderr, flush=True)


class DecodeLayer:
    """One layer: rotation, packed cache holding context-1 tokens, and the
    current token's q/k/v."""

    def __init__(self, iq, synth, w, idx, block_table, num_pages, device, bits=3):
        import torch
        self.idx = idx
        seed = w.seed * 1000 + idx
        self.rot = iq.rotation_init(synth.quaternions(seed, w.n_kv_heads), device=device)
        self.cache = iq.PagedCache(num_pages, w.n_kv_heads, device=device, bits=bits)
        lens = w.seq_lens()
        n_prev = [int(n) - 1 for n in lens]
        total = sum(n_prev)
        outl = synth.outlier_channels(seed + 1, w.n_kv_heads) if w.k_outliers else None
        dt = {"bf16": torch.bfloat16, "f32": torch.float32}[w.dtype]
        scale = torch.ones(w.n_kv_heads, 128, device=device)
        if outl is not None:
            for h in range(w.n_kv_heads):
                scale[h, torch.from_numpy(outl[h]).to(device)] = 10.0
        seq_idx = torch.cat([torch.full((n,), b, dtype=torch.int32) for b, n in enumerate(n_prev)]).to(device)
        pos = torch.cat([torch.arange(n, dtype=torch.int32) for n in n_prev]).to(device)
        chunk = 1 << 16
        for s in range(0, total, chunk):
            e = min(total, s + chunk)
            k = (synth.draw_normal_device(seed * 7 + s, (e - s, w.n_kv_heads, 128), torch.float32, device)
                 * scale).to(dt)
            v = synth.draw_normal_device(seed * 11 + s, (e - s, w.n_kv_heads, 128), dt, device)
            iq.quantize_append(self.cache, self.rot, k, v, seq_idx[s:e], pos[s:e], block_table)
        # the current token of every sequence (position len-1) and the queries
        b = w.batch
        self.k_new = (synth.draw_normal_device(seed * 13, (b, w.n_kv_heads, 128), torch.float32, device)
                      * scale).to(dt)
        self.v_new = synth.draw_normal_device(seed * 17, (b, w.n_kv_heads, 128), dt, device)
        self.q = synth.draw_normal_device(seed * 19, (b, w.n_q_heads, 128), dt, device)
        self.seq_new = torch.arange(b, dtype=torch.int32, device=device)
        self.pos_new = torch.tensor(n_prev, dtype=torch.int32, device=device)
        self.out = torch.empty((b, w.n_q_heads, 128), dtype=torch.float32, device=device)


def measured_traffic(workload: str):
    """HBM bytes per decode call from the committed rocprofv3 FETCH_SIZE /
    WRITE_SIZE record (scaled by the copy-kernel calibration), or None when no
    record exists for this workload or the kernel sources changed since."""
    import hashlib
    path = os.path.join(ROOT, "profiles", "decode_gqa_decode_32k_traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("workload") != workload:
        return None
    h = hashlib.sha256()
    for src in rec["sources"]:
        with open(os.path.join(ROOT, src), "rb") as f:
            h.update(f.read())
    if h.hexdigest() != rec["sources_sha256"]:
        return None
    return int(rec["traffic_bytes_per_call"])


def run_decode(args):
    import torch

    from compressed_space_attention_amd import isoquant as iq
    from compressed_space_attention_amd import synth, workloads

    w = workloads.DECODE_WORKLOADS[args.workload]
    device = "cuda"
    torch.cuda.set_device(0)
    lens = w.seq_lens()
    pages = [-(-int(n) // 64) for n in lens]
    bt_np, num_pages = synth.block_table(w.seed + 5, pages, shuffle=w.shuffle_pages)
    block_table = torch.from_numpy(bt_np).to(device)
    seq_lens = torch.from_numpy(lens).to(device)
    max_len = int(lens.max())
    rec_bytes = REC_BYTES if args.bits == 3 else REC_BYTES4
    kv_bytes = rec_bytes * int(lens.sum()) * w.n_kv_heads            # read by one decode call
    layer_bytes = num_pages * w.n_kv_heads * 64 * rec_bytes
    ring = max(1, math.ceil(args.ring_bytes / layer_bytes))
    log(f"[bench] workload {w.name}: {kv_bytes / 1e6:.1f} MB packed KV per call, ring of {ring} layers "
        f"({ring * layer_bytes / 1e9:.2f} GB)")
    t0 = time.time()
    layers = [DecodeLayer(iq, synth, w, i, block_table, num_pages, device, args.bits) for i in range(ring)]
    torch.cuda.synchronize()
    log(f"[bench] caches built in {time.time() - t0:.1f} s")
    ws = torch.empty(max(16, iq.decode_workspace_bytes(w.batch, w.n_q_heads, w.n_kv_heads, max_len)),
                     dtype=torch.uint8, device=device)

    def step(layer, mode="step"):
        """mode "step": the fused decode step (append + attention, one call);
        "pair": the same as two calls (quantise-append, then decode attention);
        "decode": decode attention alone (the cache already holds the token)."""
        if mode == "step":
            iq.decode_step(layer.cache, layer.rot, layer.q, layer.k_new, layer.v_new, block_table,
                           seq_lens, max_len, out=layer.out, workspace=ws)
            return
        if mode == "pair":
            iq.quantize_append(layer.cache, layer.rot, layer.k_new, layer.v_new, layer.seq_new,
                               layer.pos_new, block_table)
        iq.decode_attention(layer.cache, layer.rot, layer.q, block_table, seq_lens, max_len,
                            out=layer.out, workspace=ws)

    def run_steps(n, start, mode="step"):
        for i in range(n):
            step(layers[(start + i) % ring], mode)

    # warmup (eager)
    run_steps(args.warmup, 0)
    run_steps(2, 0, "pair")
    torch.cuda.synchronize()

    def make_graph(n, mode):
        g = torch.cuda.CUDAGraph()
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):
            with torch.cuda.graph(g, stream=s):
                run_steps(n, 0, mode)
        torch.cuda.current_stream().wait_stream(s)
        return g

    def timed(n_steps, mode):
        """Time exactly n_steps steps; returns seconds measured by HIP events."""
        stream = torch.cuda.current_stream()
        if args.no_graph:
            torch.cuda.synchronize()
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(stream)
            run_steps(n_steps, 0, mode)
            b.record(stream)
            torch.cuda.synchronize()
            return a.elapsed_time(b) / 1e3
        full, rem = divmod(n_steps, ring)
        g_full = make_graph(ring, mode) if full else None
        g_rem = make_graph(rem, mode) if rem else None
        if g_full:
            g_full.replay()      # one untimed replay: the graph's first launch uploads it
        if g_rem:
            g_rem.replay()
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        for _ in range(full):
            g_full.replay()
        if g_rem:
            g_rem.replay()
        b.record(stream)
        torch.cuda.synchronize()
        return a.elapsed_time(b) / 1e3

    t_step = timed(args.steps, "step") / args.steps
    t_decode = timed(args.steps, "decode") / args.steps
    t_pair = timed(args.steps, "pair") / args.steps
    gbs = kv_bytes / t_step / 1e9
    dec_gbs = kv_bytes / t_decode / 1e9
    log(f"[bench] step {t_step * 1e6:.2f} us ({gbs:.0f} GB/s), decode call {t_decode * 1e6:.2f} us "
        f"({dec_gbs:.0f} GB/s), unfused append + decode {t_pair * 1e6:.2f} us")

    result = {
        "metric": METRIC,
        "value": round(gbs, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(t_step * 1e3, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16",
        "data": ("synthetic: seeded N(0,1) bf16 K/V/Q"
                 + (", 4 outlier key channels x10 per kv head" if w.k_outliers else "")
                 + ", seeded random quaternion rotations, "
                 + ("shuffled" if w.shuffle_pages else "contiguous") + " 64-token page table"),
        "config": {
            "workload": w.name, "batch": w.batch, "context": max_len, "n_q_heads": w.n_q_heads,
            "n_kv_heads": w.n_kv_heads, "head_dim": 128, "page_tokens": 64, "record_bits": args.bits,
            "packed_kv_bytes_per_step": kv_bytes, "layer_ring": ring,
            "step": "one layer's decode step: quantise-append of the current token fused into "
                    "decode attention (iq_decode_step)",
        },
        "roofline": {
            "bound": "hbm",
            "kernel": "decode attention call (decode_split_kernel + decode_merge_kernel)",
            "achieved": round(dec_gbs, 2),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(dec_gbs / HBM_PEAK_GBS, 4),
            "traffic": measured_traffic(w.name) if args.bits == 3 else None,
            "algorithmic_bytes": kv_bytes,
        },
        "detail": {
            "pct_hbm_peak_step": round(100 * gbs / HBM_PEAK_GBS, 2),
            "decode_call_us": round(t_decode * 1e6, 3),
            "step_us": round(t_step * 1e6, 3),
            "unfused_append_then_decode_us": round(t_pair * 1e6, 3),
            "tokens_per_s_per_layer": round(w.batch / t_step, 1),
        },
    }
    layer0 = layers[0]
    if not args.no_aux:
        del layers
        torch.cuda.empty_cache()
        result["detail"]["dense_bf16_baseline"] = run_dense_aux(w, lens, bt_np, num_pages, t_decode)
        log(f"[bench] dense bf16 baseline: {result['detail']['dense_bf16_baseline']}")
        result["detail"]["fp8_baseline"] = run_dense_aux(w, lens, bt_np, num_pages, t_decode, fmt="fp8")
        log(f"[bench] fp8 baseline: {result['detail']['fp8_baseline']}")
        if args.bits == 3:
            result["detail"]["four_bit"] = run_four_bit_aux(w, lens, bt_np, num_pages, t_decode, t_step)
            log(f"[bench] 4-bit records: {result['detail']['four_bit']}")
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline_decode(args, w, layer0, bt_np, lens)
    return result


def probe_bandwidth(mib: int = 2048, iters: int = 20):
    """Achievable HBM bandwidth on this GPU, on a buffer far above the 256 MB
    Infinity Cache: the library's streaming read probe (iq_probe_read) and a
    device-to-device copy (read + write)."""
    import torch

    from compressed_space_attention_amd import isoquant as iq
    n = mib * (1 << 20)
    src = torch.ones(n // 4, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    sink = torch.empty(iq.probe_sink_bytes() // 4, dtype=torch.int32, device="cuda")

    def timeit(fn):
        for _ in range(3):
            fn()
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(iters):
            fn()
        b.record()
        torch.cuda.synchronize()
        return a.elapsed_time(b) / 1e3 / iters

    t_read = timeit(lambda: iq.probe_read(src, sink))
    t_copy = timeit(lambda: dst.copy_(src))
    del src, dst
    return {"bytes": n, "read_gbs": round(n / t_read / 1e9, 1), "copy_gbs": round(2 * n / t_copy / 1e9, 1),
            "read_kernel": "probe_read_kernel (16-byte loads, 8 in flight per thread)"}


def run_dense_aux(w, lens, bt_np, num_pages, t_packed, ring_bytes=1.0e9, steps=400, fmt="bf16"):
    """The uncompressed baseline on the same workload: a ring of bf16 (or FP8
    E4M3, unit scales) layer caches (same paging), the decode call timed the
    same way as the packed one (graph replay, HIP events on the launch
    stream)."""
    import torch

    from compressed_space_attention_amd import isoquant as iq
    from compressed_space_attention_amd import synth
    dev = "cuda"
    block_table = torch.from_numpy(bt_np).to(dev)
    seq_lens = torch.from_numpy(lens).to(dev)
    max_len = int(lens.max())
    per_tok = 512 if fmt == "bf16" else 256                      # K + V rows per (token, kv head)
    dense_bytes = per_tok * int(lens.sum()) * w.n_kv_heads
    layer_bytes = num_pages * w.n_kv_heads * 64 * per_tok
    ring = max(1, math.ceil(ring_bytes / layer_bytes))
    caches, qs, outs = [], [], []
    seq_idx = torch.cat([torch.full((int(n),), b, dtype=torch.int32) for b, n in enumerate(lens)]).to(dev)
    pos = torch.cat([torch.arange(int(n), dtype=torch.int32) for n in lens]).to(dev)
    total = int(lens.sum())
    for i in range(ring):
        c = iq.DenseCache(num_pages, w.n_kv_heads, device=dev, format=fmt)
        seed = w.seed * 1000 + 500 + i
        chunk = 1 << 16
        for s0 in range(0, total, chunk):
            e = min(total, s0 + chunk)
            k = synth.draw_normal_device(seed * 7 + s0, (e - s0, w.n_kv_heads, 128), torch.bfloat16, dev)
            v = synth.draw_normal_device(seed * 11 + s0, (e - s0, w.n_kv_heads, 128), torch.bfloat16, dev)
            iq.dense_append(c, k, v, seq_idx[s0:e], pos[s0:e], block_table)
        caches.append(c)
        qs.append(synth.draw_normal_device(seed * 19, (w.batch, w.n_q_heads, 128), torch.bfloat16, dev))
        outs.append(torch.empty((w.batch, w.n_q_heads, 128), dtype=torch.float32, device=dev))
    ws = torch.empty(max(16, iq.dense_decode_workspace_bytes(w.batch, w.n_q_heads, w.n_kv_heads, max_len)),
                     dtype=torch.uint8, device=dev)

    def run(n):
        for i in range(n):
            j = i % ring
            iq.dense_decode_attention(caches[j], qs[j], block_table, seq_lens, max_len, out=outs[j],
                                      workspace=ws)

    run(ring)
    torch.cuda.synchronize()
    reps = max(1, steps // ring)
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            run(ring)
    torch.cuda.current_stream().wait_stream(s)
    g.replay()
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(reps):
        g.replay()
    b.record()
    torch.cuda.synchronize()
    t = a.elapsed_time(b) / 1e3 / (reps * ring)
    del caches
    return {"kernel": f"dense_decode_split_kernel + decode_merge_kernel ({fmt} paged cache)",
            "decode_call_us": round(t * 1e6, 3), f"{fmt}_bytes_per_call": dense_bytes,
            "gbs": round(dense_bytes / t / 1e9, 1), "frac_of_hbm_peak": round(dense_bytes / t / 1e9 / HBM_PEAK_GBS, 4),
            "packed_speedup": round(t / t_packed, 3)}


def run_four_bit_aux(w, lens, bt_np, num_pages, t_decode3, t_step3, ring_bytes=1.0e9, steps=400):
    """The 4-bit variant on the same workload: a ring of 4-bit layer caches
    (same paging, same synthetic recipe), its decode step and decode call
    timed like the 3-bit ones (graph replay, HIP events on the launch stream)."""
    import torch

    from compressed_space_attention_amd import isoquant as iq
    from compressed_space_attention_amd import synth
    dev = "cuda"
    block_table = torch.from_numpy(bt_np).to(dev)
    seq_lens = torch.from_numpy(lens).to(dev)
    max_len = int(lens.max())
    kv_bytes = REC_BYTES4 * int(lens.sum()) * w.n_kv_heads
    layer_bytes = num_pages * w.n_kv_heads * 64 * REC_BYTES4
    ring = max(1, math.ceil(ring_bytes / layer_bytes))
    n_prev = [int(n) - 1 for n in lens]
    seq_idx = torch.cat([torch.full((n,), b, dtype=torch.int32) for b, n in enumerate(n_prev)]).to(dev)
    pos = torch.cat([torch.arange(n, dtype=torch.int32) for n in n_prev]).to(dev)
    total = sum(n_prev)
    layers = []
    for i in range(ring):
        seed = w.seed * 1000 + 700 + i
        rot = iq.rotation_init(synth.quaternions(seed, w.n_kv_heads), device=dev)
        c = iq.PagedCache(num_pages, w.n_kv_heads, device=dev, bits=4)
        chunk = 1 << 16
        for s0 in range(0, total, chunk):
            e = min(total, s0 + chunk)
            k = synth.draw_normal_device(seed * 7 + s0, (e - s0, w.n_kv_heads, 128), torch.bfloat16, dev)
            v = synth.draw_normal_device(seed * 11 + s0, (e - s0, w.n_kv_heads, 128), torch.bfloat16, dev)
            iq.quantize_append(c, rot, k, v, seq_idx[s0:e], pos[s0:e], block_table)
        kn = synth.draw_normal_device(seed * 13, (w.batch, w.n_kv_heads, 128), torch.bfloat16, dev)
        vn = synth.draw_normal_device(seed * 17, (w.batch, w.n_kv_heads, 128), torch.bfloat16, dev)
        q = synth.draw_normal_device(seed * 19, (w.batch, w.n_q_heads, 128), torch.bfloat16, dev)
        out = torch.empty((w.batch, w.n_q_heads, 128), dtype=torch.float32, device=dev)
        layers.append((c, rot, kn, vn, q, out))
    ws = torch.empty(max(16, iq.decode_workspace_bytes(w.batch, w.n_q_heads, w.n_kv_heads, max_len)),
                     dtype=torch.uint8, device=dev)

    def run(n, mode):
        for i in range(n):
            c, rot, kn, vn, q, out = layers[i % ring]
            if mode == "step":
                iq.decode_step(c, rot, q, kn, vn, block_table, seq_lens, max_len, out=out, workspace=ws)
            else:
                iq.decode_attention(c, rot, q, block_table, seq_lens, max_len, out=out, workspace=ws)

    def timed(mode):
        run(ring, mode)
        torch.cuda.synchronize()
        reps = max(1, steps // ring)
        g = torch.cuda.CUDAGraph()
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):
            with torch.cuda.graph(g, stream=s):
                run(ring, mode)
        torch.cuda.current_stream().wait_stream(s)
        g.replay()
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(reps):
            g.replay()
        b.record()
        torch.cuda.synchronize()
        return a.elapsed_time(b) / 1e3 / (reps * ring)

    t_step = timed("step")
    t_dec = timed("decode")
    del layers
    torch.cuda.empty_cache()
    return {"kernel": "decode_split_kernel<..., 4-bit> + decode_merge_kernel",
            "packed_kv_bytes_per_call": kv_bytes,
            "step_us": round(t_step * 1e6, 3), "decode_call_us": round(t_dec * 1e6, 3),
            "decode_call_gbs": round(kv_bytes / t_dec / 1e9, 1),
            "decode_call_frac_of_hbm_peak": round(kv_bytes / t_dec / 1e9 / HBM_PEAK_GBS, 4),
            "time_vs_3bit_decode_call": round(t_dec / t_decode3, 3),
            "time_vs_3bit_step": round(t_step / t_step3, 3)}


def median_call_seconds(fn, calls=10, reps=5, warm=20):
    """Seconds per call of fn: `warm` untimed calls (until the GPU's clocks
    have settled under this load), then `reps` event-timed runs of `calls`
    calls each on the current stream; the median run."""
    import torch
    for _ in range(warm):
        fn()
    torch.cuda.synchronize()
    runs = []
    for _ in range(reps):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(calls):
            fn()
        b.record()
        torch.cuda.synchronize()
        runs.append(a.elapsed_time(b) / 1e3 / calls)
    return sorted(runs)[len(runs) // 2]


def run_prefill_aux(bits=3):
    """The chunked-prefill workload (8192-token quantise-append into a 32,768-token
    cache, then causal attention of the last 512 positions x 64 query heads):
    append tokens/s and prefill TFLOP/s against the f16 matrix-core peak, on a
    cache of 3- or 4-bit records."""
    import torch

    from compressed_space_attention_amd import isoquant as iq
    from compressed_space_attention_amd import synth, workloads

    p = workloads.CHUNKED_PREFILL
    dev = "cuda"
    pages = -(-p.total // 64)
    bt_np, num_pages = synth.block_table(p.seed + 9, [pages], shuffle=True)
    bt = torch.from_numpy(bt_np).to(dev)
    rot = iq.rotation_init(synth.quaternions(p.seed, p.n_kv_heads), device=dev)
    cache = iq.PagedCache(num_pages, p.n_kv_heads, device=dev, zero=True, bits=bits)
    k = synth.draw_normal_device(p.seed + 2, (p.total, p.n_kv_heads, 128), torch.bfloat16, dev)
    v = synth.draw_normal_device(p.seed + 3, (p.total, p.n_kv_heads, 128), torch.bfloat16, dev)
    pos = torch.arange(p.total, dtype=torch.int32, device=dev)
    seq = torch.zeros(p.total, dtype=torch.int32, device=dev)
    iq.quantize_append(cache, rot, k[:p.cached], v[:p.cached], seq[:p.cached], pos[:p.cached], bt)
    k2, v2 = k[p.cached:].contiguous(), v[p.cached:].contiguous()
    s2, p2 = seq[p.cached:].contiguous(), pos[p.cached:].contiguous()
    q = synth.draw_normal_device(p.seed + 10, (p.n_queries, p.n_q_heads, 128), torch.bfloat16, dev)
    out = torch.empty((p.n_queries, p.n_q_heads, 128), dtype=torch.float32, device=dev)
    ws_n = iq.prefill_workspace_bytes(p.n_queries, p.n_q_heads, p.n_kv_heads, p.q_start)
    ws = torch.empty(max(16, ws_n), dtype=torch.uint8, device=dev)

    t_app = median_call_seconds(lambda: iq.quantize_append(cache, rot, k2, v2, s2, p2, bt), calls=30)
    t_pre = median_call_seconds(lambda: iq.prefill_attention(cache, rot, q, p.q_start, bt[0], out=out,
                                                             workspace=ws))
    # algorithmic flops: 2 d for q.k and 2 d for p.v per (query head, key) pair
    keys = sum(p.q_start + i + 1 for i in range(p.n_queries))
    flops = 4.0 * 128 * p.n_q_heads * keys
    rec = 50 if bits == 3 else 66
    moved = p.appended * p.n_kv_heads * 2 * (128 * 2 + rec)  # bf16 in, packed record out
    tf = flops / t_pre / 1e12
    return {
        "workload": p.name,
        "record_bits": bits,
        "append_us": round(t_app * 1e6, 2),
        "append_tokens_per_s": round(p.appended / t_app, 1),
        "append_gbs": round(moved / t_app / 1e9, 1),
        "prefill_us": round(t_pre * 1e6, 2),
        "prefill_tflops": round(tf, 2),
        "prefill_frac_of_f16_peak": round(tf / MFMA_F16_PEAK_TFLOPS, 4),
        "prefill_mfma_tflops_issued": round(1.5 * tf, 2),  # q.k runs as two f16 products
    }


def run_dense_prefill_aux(fmt="bf16"):
    """The chunked-prefill workload's attention over an uncompressed (bf16 or
    FP8, unit scales) cache of the same 32,768 tokens: the baseline of the
    packed prefill call."""
    import torch

    from compressed_space_attention_amd import isoquant as iq
    from compressed_space_attention_amd import synth, workloads

    p = workloads.CHUNKED_PREFILL
    dev = "cuda"
    pages = -(-p.total // 64)
    bt_np, num_pages = synth.block_table(p.seed + 9, [pages], shuffle=True)
    bt = torch.from_numpy(bt_np).to(dev)
    cache = iq.DenseCache(num_pages, p.n_kv_heads, device=dev, zero=True, format=fmt)
    k = synth.draw_normal_device(p.seed + 2, (p.total, p.n_kv_heads, 128), torch.bfloat16, dev)
    v = synth.draw_normal_device(p.seed + 3, (p.total, p.n_kv_heads, 128), torch.bfloat16, dev)
    pos = torch.arange(p.total, dtype=torch.int32, device=dev)
    iq.dense_append(cache, k, v, torch.zeros_like(pos), pos, bt)
    q = synth.draw_normal_device(p.seed + 10, (p.n_queries, p.n_q_heads, 128), torch.bfloat16, dev)
    out = torch.empty((p.n_queries, p.n_q_heads, 128), dtype=torch.float32, device=dev)
    t = median_call_seconds(lambda: iq.dense_prefill_attention(cache, q, p.q_start, bt[0], out=out))
    keys = sum(p.q_start + i + 1 for i in range(p.n_queries))
    tf = 4.0 * 128 * p.n_q_heads * keys / t / 1e12
    del cache
    return {"kernel": f"dense_prefill_kernel ({fmt} paged cache)", "prefill_us": round(t * 1e6, 2),
            "prefill_tflops": round(tf, 2), "prefill_frac_of_f16_peak": round(tf / MFMA_F16_PEAK_TFLOPS, 4)}


def cpu_baseline_decode(args, w, layer, bt_np, lens):
    """The CPU oracle, as it stands, on a bounded sample of the same step:
    quantise-append the current token, then decode over the layer's cache."""
    import threadpoolctl

    from oracle import isoquant4_oracle as O4
    from oracle import isoquant_oracle as O

    four = layer.cache.bits == 4
    host = (O4.PagedCache4 if four else O.PagedCache).from_arrays(*layer.cache.to_host())
    append = O4.quantize_append4 if four else O.quantize_append
    decode = O4.decode_attention4 if four else O.decode_attention
    from compressed_space_attention_amd import synth
    quats = synth.quaternions(w.seed * 1000 + layer.idx, w.n_kv_heads)
    blocks = O.rotation_matrices(quats)
    q = layer.q.float().cpu().numpy().astype(np.float64)
    k_new = layer.k_new.float().cpu().numpy().astype(np.float64)
    v_new = layer.v_new.float().cpu().numpy().astype(np.float64)
    pos_new = layer.pos_new.cpu().numpy()
    seq_new = layer.seq_new.cpu().numpy()
    kv_bytes = (REC_BYTES4 if four else REC_BYTES) * int(lens.sum()) * w.n_kv_heads
    info = threadpoolctl.threadpool_info()
    threads = max([i.get("num_threads", 1) for i in info if i.get("user_api") == "blas"] or [1])
    def run(seconds):
        steps, t0 = 0, time.perf_counter()
        while True:
            append(host, blocks, k_new, v_new, seq_new, pos_new, bt_np)
            decode(host, blocks, q, bt_np, lens)
            steps += 1
            el = time.perf_counter() - t0
            if el >= seconds or el * (steps + 1) / steps > 3 * seconds:
                return steps, el

    steps, el = run(args.cpu_seconds)
    with threadpoolctl.threadpool_limits(1):       # the same oracle on one core
        steps1, el1 = run(args.cpu_seconds / 2)
    return {
        "value": round(kv_bytes * steps / el / 1e9, 5),
        "unit": "GB/s",
        "cores": int(threads),
        "kind": "oracle",
        "sample": f"{steps} {'4-bit ' if four else ''}oracle steps of one layer (append 1 token + decode over "
                  f"{int(lens.max())} tokens, {w.n_q_heads}q/{w.n_kv_heads}kv) in {el:.1f} s; "
                  f"host has {os.cpu_count()} logical CPUs",
        "single_thread": {"value": round(kv_bytes * steps1 / el1 / 1e9, 5), "unit": "GB/s", "cores": 1,
                          "sample": f"{steps1} steps in {el1:.1f} s"},
    }


TRAFFIC_SOURCES = ["compressed_space_attention_amd/csrc/decode.hip",
                   "compressed_space_attention_amd/csrc/iq_device.h",
                   "compressed_space_attention_amd/csrc/iq_internal.h"]


def write_traffic_record(root: str, workload: str = "gqa_decode_32k_32q4kv", calib_mib: int = 512):
    """HBM bytes per decode attention call from rocprofv3 counter CSVs: the
    median FETCH_SIZE and WRITE_SIZE (KiB per dispatch) of the decode-only
    split kernel and of the merge kernel, each scaled by what the counter
    reads for a plain copy of known size."""
    import csv
    import glob
    import hashlib

    def medians(sub):
        vals = {}
        for f in glob.glob(os.path.join(root, sub, "**", "*counter_collection.csv"), recursive=True):
            for r in csv.DictReader(open(f)):
                vals.setdefault(r["Kernel_Name"], []).append(float(r["Counter_Value"]))
        return {k: sorted(v)[len(v) // 2] for k, v in vals.items()}

    def pick(table, pred):
        hits = [v for k, v in table.items() if pred(k)]
        if len(hits) != 1:
            raise SystemExit(f"expected one kernel, found {len(hits)}")
        return hits[0]

    def split(k):  # decode_split_kernel<PACK8, waves, APPEND = false, record bits = 3, BALANCED>
        if "decode_split_kernel<" not in k or "dense" in k:
            return False
        targs = [a.strip() for a in k.split("<")[1].split(">")[0].split(",")]
        return len(targs) == 5 and targs[2] == "false" and targs[3] == "3"

    merge = lambda k: "decode_merge_kernel<true>" in k
    copy = lambda k: "copy" in k.lower()
    fetch, write = medians("pmc_FETCH_SIZE"), medians("pmc_WRITE_SIZE")
    cf, cw = medians("cal_FETCH_SIZE"), medians("cal_WRITE_SIZE")
    moved_kib = calib_mib * 1024
    f_fac = moved_kib / pick(cf, copy)
    w_fac = moved_kib / pick(cw, copy)
    counters = {"decode_split_kernel (decode only)": {"FETCH_SIZE": pick(fetch, split), "WRITE_SIZE": pick(write, split)},
                "decode_merge_kernel": {"FETCH_SIZE": pick(fetch, merge), "WRITE_SIZE": pick(write, merge)}}
    total_kib = sum(c["FETCH_SIZE"] * f_fac + c["WRITE_SIZE"] * w_fac for c in counters.values())
    h = hashlib.sha256()
    for src in TRAFFIC_SOURCES:
        with open(os.path.join(ROOT, src), "rb") as f:
            h.update(f.read())
    rec = {
        "kernel": "decode_split_kernel + decode_merge_kernel (one decode attention call)",
        "workload": workload,
        "sources_sha256": h.hexdigest(),
        "sources": TRAFFIC_SOURCES,
        "counters_kib_per_dispatch": counters,
        "copy_calibration": {"bytes_per_launch": calib_mib << 20, "FETCH_SIZE_kib": pick(cf, copy),
                             "WRITE_SIZE_kib": pick(cw, copy), "fetch_factor": round(f_fac, 4),
                             "write_factor": round(w_fac, 4)},
        "traffic_bytes_per_call": int(round(total_kib * 1024)),
        "commands": [
            "rocprofv3 --pmc FETCH_SIZE --kernel-include-regex 'decode_split|decode_merge' -d DIR/pmc_FETCH_SIZE "
            "-o d --output-format csv -- python3 bench.py --steps 40 --warmup 8 --no-cpu-baseline --no-graph --no-aux",
            "rocprofv3 --pmc WRITE_SIZE --kernel-include-regex 'decode_split|decode_merge' -d DIR/pmc_WRITE_SIZE "
            "-o d --output-format csv -- python3 bench.py --steps 40 --warmup 8 --no-cpu-baseline --no-graph --no-aux",
            "rocprofv3 --pmc FETCH_SIZE -d DIR/cal_FETCH_SIZE -o c --output-format csv -- python3 bench.py "
            "--copy-calibration 512",
            "rocprofv3 --pmc WRITE_SIZE -d DIR/cal_WRITE_SIZE -o c --output-format csv -- python3 bench.py "
            "--copy-calibration 512",
            "python3 bench.py --write-traffic-record DIR",
        ],
    }
    out = os.path.join(ROOT, "profiles", "decode_gqa_decode_32k_traffic.json")
    with open(out, "w") as f:
        json.dump(rec, f, indent=1)
    print(json.dumps({"traffic_bytes_per_call": rec["traffic_bytes_per_call"], "record": out}))


def copy_calibration(mib: int, reps: int = 20):
    """A plain device-to-device copy of known size, for scaling FETCH_SIZE and
    WRITE_SIZE: each launch reads and writes exactly mib MiB."""
    import torch
    n = mib * (1 << 20)
    src = torch.ones(n, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(reps):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes_per_launch": n, "launches": reps}), flush=True)


def main():
    args = parse()
    if args.write_traffic_record:
        write_traffic_record(args.write_traffic_record)
        return
    if args.copy_calibration:
        copy_calibration(args.copy_calibration)
        return
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(json.dumps({"error": "this benchmark measures one GPU; the path has no multi-GPU "
                                   "collective (each GPU would own its own sequences/kv heads)",
                          "n_gpus": args.gpus}))
        sys.exit(2)
    res = run_decode(args)
    if not args.no_aux:
        res["detail"]["prefill"] = run_prefill_aux()
        res["detail"]["prefill_4bit"] = run_prefill_aux(bits=4)
        res["detail"]["prefill_bf16_baseline"] = run_dense_prefill_aux("bf16")
        res["detail"]["prefill_fp8_baseline"] = run_dense_prefill_aux("fp8")
        probe = probe_bandwidth()
        res["detail"]["hbm_probe"] = probe
        res["detail"]["decode_call_frac_of_probe_read"] = round(
            res["roofline"]["achieved"] / probe["read_gbs"], 4)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
