#!/usr/bin/env python3
"""Decode-attention throughput over a quantized KV cache on one MI355X.

One step = the whole hot path for one batch, one kvq_decode_step call per
layer: quantize-append the step's new K/V row of every sequence and KV head
into the cache, split-K decode attention over the cache and the merge of the
chunk partials (three launches at 32K; one when a context is one chunk per
sequence and KV head).  Inputs are resident in HBM before timing.
The K timed steps run as one HIP graph of K steps (the way a model's layers
follow each other inside one decode step); the line also reports a graph of
one step replayed K times, eager steps, and the separate calls timed with
events between them.

The headline workload is 32 sequences x 32 query heads / 8 KV heads x
head_dim 128 at a 32K-token context with nibble-packed int4 K and V
(one fp16 scale per head and position).  `value` is whole-step throughput in
GB/s of algorithmic bytes (the bytes the method must move: the cache it
streams, q in, out, and the appended rows); `roofline` prices the split-K
kernel alone against MI355X's 8 TB/s HBM peak.

By default (--modes all) the line also carries every mode of the other
workloads, each with its split kernel's rate, % of peak, step time and
tokens/s (`summary` lists them): K8V4 at 32K, the FP16 / K4V8 / 32-value
group / zero-point modes of the 32K shape, the same 32K workloads paged, the 8K K8V4
workload in K8V4 / FP16 / K8V8 / K4V4 and the 64 + 1536 window (both cold:
they fit in the 256 MB MALL), TinyLoop-like in K8V8 / FP16 / per-layer
widths, Tiny, the mni-ml-like generation loop, and bulk prefill.

    python bench.py [--steps K] [--warmup W] [--modes headline|targets|paged|all]

Prints one JSON line.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import threading
import time
from pathlib import Path

ROOT = Path(__file__).resolve().parent
if str(ROOT) not in sys.path:
    sys.path.insert(0, str(ROOT))

PEAK_HBM_GBS = 8000.0          # MI355X HBM3E, AMD's published peak
METRIC = "decode-attention achieved HBM GB/s (% of MI355X peak) and tokens/s per mode"


def bpt_head(mode, w) -> float:
    """Cache bytes per position per KV head (fp16 scales included; the
    zero-point codec stores a 32-bit word, scale and zero, per group)."""
    import decode_attention_quantized_kvq_amd as kvq
    g = _group(mode, w)
    b = kvq.kvq_bytes_per_token(mode.k_bits, mode.v_bits, w.n_kv_heads, w.head_dim, g) / w.n_kv_heads
    if getattr(mode, "zero_point", False):
        b += 2 * (w.head_dim / g) * ((mode.k_bits < 16) + (mode.v_bits < 16))
    return b


def _group(mode, w) -> int:
    if mode.k_bits >= 16:
        return w.head_dim
    return mode.group_size(w.n_kv_heads, w.head_dim)


def attended(w) -> int:
    return min(w.n_pos, w.capacity)


def split_bytes(w, mode) -> float:
    """Algorithmic bytes of one split-K launch: the attended cache + q."""
    return w.batch * w.n_kv_heads * attended(w) * bpt_head(mode, w) + w.batch * w.n_q_heads * w.head_dim * 4


def step_bytes(w, mode) -> float:
    """Algorithmic bytes of one step (per layer): cache + q in + out + appended rows."""
    append = w.batch * w.n_kv_heads * (w.head_dim * 2 * 4 + bpt_head(mode, w))
    return split_bytes(w, mode) + w.batch * w.n_q_heads * w.head_dim * 4 + append


def run_mode(w, mode, steps: int, warmup: int, chunk: int = 0, flush: bool = False, log=print,
             settle_ms: float = 100.0, page_size: int = 0, layer_modes=None) -> dict:
    """One bench line.  page_size > 0 stores the cache in a pool of pages of
    that many slots, assigned to the sequences in a seeded random order.
    layer_modes: one mode per layer (bit widths chosen per layer; `mode`
    then only names the line and picks the split-alone figure's layer 0)."""
    import torch

    import decode_attention_quantized_kvq_amd as kvq
    from workloads.device import fill, positions, queries

    t_fill = time.perf_counter()
    layers = []
    for layer in range(w.n_layers):
        paging = {}
        if page_size:
            pps = w.capacity // page_size
            n_pages = w.batch * pps
            order = torch.randperm(n_pages, generator=torch.Generator().manual_seed(w.seed + layer))
            paging = dict(page_size=page_size, n_pages=n_pages,
                          block_table=order.to(torch.int32).view(w.batch, pps).to("cuda"))
        lm = layer_modes[layer] if layer_modes else mode
        cache = kvq.alloc_cache(w.batch, w.n_kv_heads, w.head_dim, w.capacity, lm.k_bits, lm.v_bits,
                                _group(lm, w), w.n_anchor, w.window, zero_point=int(lm.zero_point), **paging)
        k_last, v_last = fill([cache], w, layer, w.n_pos)
        q = queries(w, layer)
        layers.append((cache, k_last, v_last, q))
    name = f"{w.name}-paged{page_size}" if page_size else w.name
    log(f"[bench] {name} {mode.name}: {w.n_layers} layer(s) filled in {time.perf_counter() - t_fill:.1f} s")

    max_len = w.n_pos
    ch = kvq.kvq_chunk_tokens(layers[0][0], w.n_q_heads, max_len) if chunk == 0 else chunk
    n_chunks = kvq.kvq_chunk_count(layers[0][0], w.n_q_heads, max_len, chunk)
    ws_bytes = kvq.kvq_workspace_bytes(layers[0][0], w.n_q_heads, max_len, chunk)
    ws = torch.zeros(ws_bytes // 4 + 64, dtype=torch.float32, device="cuda")   # zero-filled: the step's ticket counters
    out = torch.empty((w.batch, w.n_q_heads, w.head_dim), dtype=torch.float32, device="cuda")
    pos = positions([w.n_pos - 1] * w.batch)
    lens = positions([w.n_pos] * w.batch)
    # MALL scrub: a 1 GiB read (> the 256 MB MALL) before each step evicts the
    # cache's lines with clean ones, so the step reads cold data and pays for
    # no write-back of the scrub itself (a 1 GiB write would leave the MALL
    # full of dirty lines to be written back inside the timed step)
    scrub = torch.ones(1 << 28, dtype=torch.float32, device="cuda") if flush else None
    scrub_out = torch.empty((), dtype=torch.float32, device="cuda") if flush else None
    stream = torch.cuda.current_stream()

    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(steps * w.n_layers)]

    def one_step(st):
        # the whole hot path of a decode step: one call per layer
        for cache, k_last, v_last, q in layers:
            if scrub is not None:
                torch.sum(scrub, dim=0, out=scrub_out)
            kvq.kvq_decode_step(cache, k_last, v_last, 1, pos, q, w.n_q_heads, lens, max_len, 0.0, chunk, out, ws,
                                ws_bytes, st)

    def parts_step(record, st):
        # the same work as separate calls, with events between them
        for li, (cache, k_last, v_last, q) in enumerate(layers):
            e = ev[record * w.n_layers + li]
            if scrub is not None:
                torch.sum(scrub, dim=0, out=scrub_out)
            e[0].record(st)
            kvq.kvq_append(cache, k_last, v_last, 1, pos, st)
            e[1].record(st)
            kvq.kvq_decode_partials(cache, q, w.n_q_heads, lens, max_len, 0.0, chunk, ws, ws_bytes, st)
            e[2].record(st)
            kvq.kvq_combine(w.batch, w.n_q_heads, w.head_dim, n_chunks, ws, ws_bytes, out, st)
            e[3].record(st)

    for _ in range(warmup):
        one_step(stream)
    torch.cuda.synchronize()
    # (1) per-kernel breakdown: events around each call, eager launches
    t0 = time.perf_counter()
    for s_ in range(steps):
        parts_step(s_, stream)
    torch.cuda.synchronize()
    wall_eager = time.perf_counter() - t0
    t_app = sum(e[0].elapsed_time(e[1]) for e in ev) / len(ev)
    t_split = sum(e[1].elapsed_time(e[2]) for e in ev) / len(ev)
    t_comb = sum(e[2].elapsed_time(e[3]) for e in ev) / len(ev)
    # (1b) with the MALL scrub: the step itself, cold, events around each
    # kvq_decode_step (the scrub outside them)
    ms_step_cold = None
    if scrub is not None:
        ev_step = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                   for _ in range(steps * w.n_layers)]
        for s_ in range(steps):
            for li, (cache, k_last, v_last, q) in enumerate(layers):
                e = ev_step[s_ * w.n_layers + li]
                torch.sum(scrub, dim=0, out=scrub_out)
                e[0].record(stream)
                kvq.kvq_decode_step(cache, k_last, v_last, 1, pos, q, w.n_q_heads, lens, max_len, 0.0, chunk, out,
                                    ws, ws_bytes, stream)
                e[1].record(stream)
        torch.cuda.synchronize()
        ms_step_cold = sum(e[0].elapsed_time(e[1]) for e in ev_step) / steps
    # (2) the split launch alone, back to back, events only around the loop.
    # After an idle pause the first few dozen launches of a busy GPU run up to
    # 40% slower for some milliseconds (a power-management transient; clocks
    # and temperatures stay flat), so launches run untimed for `settle_ms`
    # first and the timed loop is long enough to average over what remains.
    cache0, _, _, q0 = layers[0]
    ea, eb = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)

    def timed(fn, n, st=stream):
        ea.record(st)
        for _ in range(n):
            fn()
        eb.record(st)
        torch.cuda.synchronize()
        return ea.elapsed_time(eb)

    mode0 = layer_modes[0] if layer_modes else mode
    if mode0.k_bits < 16:
        # the split kernel alone: one query preparation, then split launches on it
        kvq.kvq_prepare_query(cache0, q0, w.n_q_heads, max_len, 0.0, chunk, ws, ws_bytes, stream)
        split = lambda: kvq.kvq_decode_partials_prepared(cache0, w.n_q_heads, lens, max_len, chunk, ws, ws_bytes, stream)
    else:
        split = lambda: kvq.kvq_decode_partials(cache0, q0, w.n_q_heads, lens, max_len, 0.0, chunk, ws, ws_bytes, stream)
    settled = 0.0
    while settled < settle_ms:
        settled += timed(split, 50)
    n_split = max(steps, 200)
    t_split_loop = timed(split, n_split) / n_split
    # (3) eager fused steps, back to back
    ms_step_eager = timed(lambda: one_step(stream), steps) / steps
    # (4) the step as HIP graphs: one step per replay, and `steps` steps in
    # one graph (as the layers of a model's decode step run: no host launch
    # between them); the latter is the timed number
    ms_step_graph1 = ms_step_graph = ms_step_graph_avg = None
    if scrub is None:
        cs = torch.cuda.Stream()
        cs.wait_stream(stream)
        with torch.cuda.stream(cs):
            one_step(cs)                             # warm the capture stream
        torch.cuda.synchronize()
        g1 = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g1, stream=cs):
            one_step(cs)
        gk = torch.cuda.CUDAGraph()
        with torch.cuda.graph(gk, stream=cs):
            for _ in range(steps):
                one_step(cs)
        for _ in range(warmup):
            g1.replay()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(steps):
            g1.replay()
        torch.cuda.synchronize()
        ms_step_graph1 = (time.perf_counter() - t0) / steps * 1e3
        # the K-step graph: untimed replays for >= settle_ms (the clock
        # transient after the graph's first launch), then exactly K steps (one
        # replay) timed, and the average over >= settle_ms of replays as a
        # cross-check
        t0 = time.perf_counter()
        while True:
            gk.replay()
            torch.cuda.synchronize()
            if (time.perf_counter() - t0) * 1e3 >= settle_ms:
                break
        t0 = time.perf_counter()
        gk.replay()
        torch.cuda.synchronize()
        ms_step_graph = (time.perf_counter() - t0) / steps * 1e3
        n_rep = max(1, int(settle_ms / (ms_step_graph * steps)) + 1)
        t0 = time.perf_counter()
        for _ in range(n_rep):
            gk.replay()
        torch.cuda.synchronize()
        ms_step_graph_avg = (time.perf_counter() - t0) / (n_rep * steps) * 1e3
        del g1, gk
    ms_step_wall = wall_eager / steps * 1e3
    ms_step_gpu = (t_app + t_split + t_comb) * w.n_layers
    sbytes = sum(step_bytes(w, m) for m in layer_modes) if layer_modes else step_bytes(w, mode) * w.n_layers
    # with the MALL scrub inside the loop, wall time includes it: the step's
    # own events then
    ms_step = ms_step_cold if flush else ms_step_graph
    res = {
        "workload": name, "mode": mode.name, "page_size": page_size, "batch": w.batch, "n_q_heads": w.n_q_heads,
        "n_kv_heads": w.n_kv_heads, "head_dim": w.head_dim, "context": attended(w), "n_layers": w.n_layers,
        "capacity": w.capacity, "n_anchor": w.n_anchor, "window": w.window, "group_size": _group(mode, w),
        "chunk_tokens": ch, "n_chunks": n_chunks, "mall_scrub": flush,
        "ms_per_step": ms_step, "ms_per_step_graph": ms_step_graph, "ms_per_step_graph_avg": ms_step_graph_avg,
        "ms_per_step_graph_1step": ms_step_graph1,
        "ms_per_step_eager": ms_step_eager, "ms_per_step_eager_parts_with_events": ms_step_wall,
        "ms_per_step_kernels": ms_step_gpu, "ms_per_step_cold": ms_step_cold,
        "us_split_back_to_back": t_split_loop * 1e3,
        "split_launches_timed": n_split, "split_settle_ms": settled,
        "step_GBps": sbytes / (ms_step * 1e-3) / 1e9,
        "tokens_per_s": w.batch / (ms_step * 1e-3),
        "us_append": t_app * 1e3, "us_split": t_split * 1e3, "us_combine": t_comb * 1e3,
        # MALL-resident workloads: the split rate from the cold (scrubbed) split,
        # not from the back-to-back loop, whose cache stays in the MALL
        "split_bytes": split_bytes(w, mode0),
        "split_GBps": split_bytes(w, mode0) / ((t_split if flush else t_split_loop) * 1e-3) / 1e9,
    }
    res["split_pct_of_peak"] = 100.0 * res["split_GBps"] / PEAK_HBM_GBS
    g1s = f"{ms_step_graph1 * 1e3:.1f} us" if ms_step_graph1 is not None else "not timed (MALL scrubbed)"
    log(f"[bench] {name} {mode.name}: step {ms_step * 1e3:.1f} us ({res['step_GBps']:.0f} GB/s, "
        f"{res['tokens_per_s']:.0f} tok/s; 1-step graph {g1s}, eager "
        f"{ms_step_eager * 1e3:.1f} us); split{' (cold)' if flush else ''} "
        f"{(t_split if flush else t_split_loop) * 1e3:.1f} us = {res['split_GBps']:.0f} GB/s "
        f"({res['split_pct_of_peak']:.1f}% of peak); append {t_app * 1e3:.1f} us, combine {t_comb * 1e3:.1f} us")
    del layers, ws, out, scrub, scrub_out
    torch.cuda.empty_cache()
    return res


def prefill(w, mode, rows_per_call: int = 4096, reps: int = 3, log=print) -> dict:
    """Bulk quantization of a whole context (a prompt) into the cache:
    kvq_append in calls of `rows_per_call` rows per sequence over the
    workload's context, timed with HIP events after one untimed pass.
    Algorithmic bytes: the float32 K and V rows read, the codes and scales
    written."""
    import torch

    import decode_attention_quantized_kvq_amd as kvq
    from workloads.device import positions
    cache = kvq.alloc_cache(w.batch, w.n_kv_heads, w.head_dim, w.capacity, mode.k_bits, mode.v_bits,
                            _group(mode, w))
    n = min(rows_per_call, w.capacity)
    g = torch.Generator(device="cuda").manual_seed(w.seed)
    K = torch.randn((w.batch, w.n_kv_heads, n, w.head_dim), device="cuda", generator=g)
    V = torch.randn((w.batch, w.n_kv_heads, n, w.head_dim), device="cuda", generator=g)
    starts = [positions([p0] * w.batch) for p0 in range(0, w.capacity - n + 1, n)]
    stream = torch.cuda.current_stream()

    def run():
        for sp in starts:
            kvq.kvq_append(cache, K, V, n, sp, stream)

    run()
    ea, eb = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ea.record(stream)
    for _ in range(reps):
        run()
    eb.record(stream)
    torch.cuda.synchronize()
    ms = ea.elapsed_time(eb) / reps
    rows = w.batch * w.n_kv_heads * n * len(starts)
    nbytes = rows * w.head_dim * 4 * 2 + rows * bpt_head(mode, w)
    res = {"workload": w.name, "mode": mode.name, "rows_per_call": n, "calls": len(starts), "ms": ms,
           "bytes": nbytes, "GBps": nbytes / (ms * 1e-3) / 1e9}
    res["pct_of_peak"] = 100.0 * res["GBps"] / PEAK_HBM_GBS
    log(f"[bench] prefill {w.name} {mode.name}: {len(starts)} calls of {n} rows, {ms:.3f} ms = "
        f"{res['GBps']:.0f} GB/s ({res['pct_of_peak']:.1f}% of peak)")
    del cache, K, V
    torch.cuda.empty_cache()
    return res


def generation_loop(w, mode, reps: int = 5, log=print) -> dict:
    """A generation loop on one sequence (the mni-ml-like workload): the
    prompt appended in one call, then one kvq_decode_step per generated
    token (append its row, attend with its query), all rows and queries
    already in device memory.  Timed as eager calls and as one HIP graph of
    the whole loop; tokens/s = generated tokens / loop time."""
    import torch

    import decode_attention_quantized_kvq_amd as kvq
    from workloads.device import positions, to_device
    cache = kvq.alloc_cache(w.batch, w.n_kv_heads, w.head_dim, w.capacity, mode.k_bits, mode.v_bits,
                            _group(mode, w))
    k_rows, v_rows = wl_rows(w, 0)
    kd, vd = to_device(k_rows[None]), to_device(v_rows[None])      # [1][Hkv][n_pos][HD]
    kvq.kvq_append(cache, kd[:, :, :w.prompt].contiguous(), vd[:, :, :w.prompt].contiguous(), w.prompt,
                   positions([0]))
    n_gen = w.n_pos - w.prompt
    rows = [(kd[:, :, p:p + 1].contiguous(), vd[:, :, p:p + 1].contiguous()) for p in range(w.prompt, w.n_pos)]
    qs = [to_device(wl_query(w, s)[None]) for s in range(n_gen)]
    pos = [positions([w.prompt + s]) for s in range(n_gen)]
    lens = [positions([w.prompt + s + 1]) for s in range(n_gen)]
    ws_bytes = kvq.kvq_workspace_bytes(cache, w.n_q_heads, w.capacity, 0)
    ws = torch.zeros(ws_bytes // 4 + 64, dtype=torch.float32, device="cuda")   # zero-filled: the step's ticket counters
    out = torch.empty((1, w.n_q_heads, w.head_dim), dtype=torch.float32, device="cuda")

    def loop(st):
        for s_ in range(n_gen):
            kvq.kvq_decode_step(cache, rows[s_][0], rows[s_][1], 1, pos[s_], qs[s_], w.n_q_heads, lens[s_],
                                w.capacity, 0.0, 0, out, ws, ws_bytes, st)

    stream = torch.cuda.current_stream()
    loop(stream)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(reps):
        loop(stream)
    torch.cuda.synchronize()
    eager_s = (time.perf_counter() - t0) / reps
    cs = torch.cuda.Stream()
    cs.wait_stream(stream)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=cs):
        loop(cs)
    g.replay()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(reps):
        g.replay()
    torch.cuda.synchronize()
    graph_s = (time.perf_counter() - t0) / reps
    res = {"workload": w.name, "mode": mode.name, "prompt": w.prompt, "generated": n_gen,
           "cache_bytes_per_token": kvq.kvq_bytes_per_token(mode.k_bits, mode.v_bits, w.n_kv_heads, w.head_dim,
                                                            _group(mode, w)),
           "us_per_token_eager": eager_s / n_gen * 1e6, "us_per_token_graph": graph_s / n_gen * 1e6,
           "tokens_per_s_eager": n_gen / eager_s, "tokens_per_s_graph": n_gen / graph_s}
    log(f"[bench] generation {w.name} {mode.name}: {n_gen} tokens after a {w.prompt}-token prompt, "
        f"{res['tokens_per_s_graph']:.0f} tok/s in one graph ({res['us_per_token_graph']:.1f} us/token), "
        f"{res['tokens_per_s_eager']:.0f} tok/s eager; cache {res['cache_bytes_per_token']} B/token")
    del g, cache, ws, out
    torch.cuda.empty_cache()
    return res


def wl_rows(w, layer: int):
    """K and V rows of sequence 0 of `layer`: ([Hkv][n_pos][HD], [Hkv][n_pos][HD])."""
    import workloads as wl
    return wl.rows(w, wl.K_STREAM, layer, 0, w.n_pos), wl.rows(w, wl.V_STREAM, layer, 0, w.n_pos)


def wl_query(w, step: int):
    import workloads as wl
    return wl.query(w, 0, 0, step)


def read_probe(log=print, gib: int = 2, launches: int = 50) -> dict:
    """The bandwidth a plain read stream reaches on this device
    (kvq_read_probe over `gib` GiB, larger than the 256 MB MALL), after a
    settle period, timed with HIP events over `launches` launches."""
    import torch

    import decode_attention_quantized_kvq_amd as kvq
    nbytes = gib << 30
    buf = torch.ones(nbytes // 4, dtype=torch.float32, device="cuda")
    sink = torch.empty(8192, dtype=torch.int32, device="cuda")
    stream = torch.cuda.current_stream()
    for _ in range(20):
        kvq.kvq_read_probe(buf, nbytes, sink, 8192 * 4, stream)
    ea, eb = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ea.record(stream)
    for _ in range(launches):
        kvq.kvq_read_probe(buf, nbytes, sink, 8192 * 4, stream)
    eb.record(stream)
    torch.cuda.synchronize()
    us = ea.elapsed_time(eb) / launches * 1e3
    gbs = nbytes / us / 1e3
    log(f"[bench] read probe: {gib} GiB in {us:.1f} us = {gbs:.0f} GB/s ({100 * gbs / PEAK_HBM_GBS:.1f}% of peak)")
    del buf, sink
    torch.cuda.empty_cache()
    return {"GBps": round(gbs, 1), "pct_of_peak": round(100 * gbs / PEAK_HBM_GBS, 2), "bytes": nbytes,
            "us_per_launch": round(us, 2), "kernel": "read_probe_kernel (8 x 16-byte nontemporal loads per thread)"}


def _cpu_facts() -> dict:
    """The host CPU as the process sees it."""
    model = None
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    try:
        affinity = len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        affinity = os.cpu_count() or 1
    return {"nproc": os.cpu_count(), "affinity": affinity, "omp_num_threads": os.environ.get("OMP_NUM_THREADS"),
            "model": model}


def cpu_baseline(w, mode, log=print, budget_s: float = 15.0, runs: int = 3) -> dict:
    """The CPU oracle's decode step, untuned, on a bounded sample of the
    workload: whole sequences (every KV and query head, the full context),
    one per thread, on the CPU share this process may use (its affinity mask,
    capped by OMP_NUM_THREADS and at 16, the share one GPU's host has).
    `runs` timed runs of about budget_s / runs seconds each (whole rounds of
    one sequence per thread, after one untimed round); the median run is
    reported.  Then one thread alone, median of 3 runs of one sequence."""
    import numpy as np

    import oracle
    import workloads as wl

    oracle.lib()
    facts = _cpu_facts()
    omp = facts["omp_num_threads"]
    cores = max(1, min(facts["affinity"], int(omp) if omp and omp.isdigit() else 16, 16, w.batch))
    g = _group(mode, w)
    scale = 1.0 / np.sqrt(w.head_dim)
    seqs = list(range(cores))
    data = {s_: (wl.rows(w, wl.K_STREAM, 0, s_, w.n_pos), wl.rows(w, wl.V_STREAM, 0, s_, w.n_pos),
                 wl.query(w, 0, s_)) for s_ in seqs}

    def work(s_):
        K, V, q = data[s_]
        oracle.decode_step(mode.k_bits, mode.v_bits, g, w.n_anchor, w.window, K, V, q, scale)

    def round_():
        threads = [threading.Thread(target=work, args=(s_,)) for s_ in seqs]
        t0 = time.perf_counter()
        for t in threads:
            t.start()
        for t in threads:
            t.join()
        return time.perf_counter() - t0

    round_()                                         # untimed: first touch of the inputs
    rates, total = [], 0
    for _ in range(runs):
        done, t_run = 0, 0.0
        while done == 0 or t_run < budget_s / runs:
            t_run += round_()
            done += len(seqs)
        rates.append(done / t_run)                   # sequence-steps per second
        total += done
    rate = sorted(rates)[len(rates) // 2]
    log(f"[bench] cpu oracle: {total} sequence-steps on {cores} thread(s), runs at "
        f"{', '.join(f'{r:.2f}' for r in rates)} seq-steps/s ({facts['model']}, nproc {facts['nproc']})")
    one = []
    for _ in range(3):
        t0 = time.perf_counter()
        work(0)
        one.append(time.perf_counter() - t0)
    t_one = sorted(one)[1]
    log(f"[bench] cpu oracle, one thread: {t_one:.2f} s per sequence-step (median of 3)")
    per_seq = step_bytes(w, mode) / w.batch
    return {
        "value": per_seq * rate / 1e9, "unit": "GB/s", "cores": cores, "kind": "oracle",
        "sample": f"sequences 0-{cores - 1} of {w.name} ({mode.name}; {w.batch} per step), every head, full "
                  f"{attended(w)}-position context, one sequence per thread; median of {runs} runs of about "
                  f"{budget_s / runs:.0f} s ({total} sequence-steps in all); float64 oracle (encode every row, then "
                  f"softmax attention); input generation excluded",
        "tokens_per_s": rate,
        "runs_tokens_per_s": rates,
        "host": facts,
        "one_core": {"value": per_seq / t_one / 1e9, "unit": "GB/s", "tokens_per_s": 1.0 / t_one,
                     "sample": "sequence 0, median of 3 sequence-steps on one thread"},
    }


def traffic_record(key: str):
    """HBM bytes per launch of the split kernel of workload/mode `key` from
    the committed counter summary, if it was taken on the kernel sources as
    they are now."""
    import hashlib
    path = ROOT / "profiles" / "traffic.json"
    if not path.exists():
        return None
    rec = json.loads(path.read_text())
    h = hashlib.sha256()
    for f in rec.get("sources", []):
        h.update((ROOT / f).read_bytes())
    entry = rec.get("workloads", {}).get(key)
    if entry is None or h.hexdigest() != rec.get("sha256"):
        return None
    return entry


TRAFFIC_SOURCES = ["decode_attention_quantized_kvq_amd/csrc/kvq_decode_quant.hpp",
                   "decode_attention_quantized_kvq_amd/csrc/kvq_device.hpp",
                   "decode_attention_quantized_kvq_amd/csrc/kvq.hip"]


PROBE_WORKLOADS = {"k4v4-32k": ("K4V4_32K", "K4V4", "decode_quant_kernel<4,4,128,4,1,false,false>"),
                   "k8v4-32k": ("K8V4_32K", "K8V4", "decode_quant_kernel<8,4,128,4,1,false,false>"),
                   "k4v4-g32-32k": ("K4V4_32K", "K4V4_G32", "decode_quant_kernel<4,4,128,4,4,false,false>")}


def record_traffic(fetch_csv: str, write_csv: str, workload: str = "k4v4-32k", log=print) -> int:
    """Turn the two counter runs of --probe-traffic into the workload's entry
    of profiles/traffic.json: each counter scaled by what it reads for the
    1 GiB copy of the same run, averaged over the three split launches.
    Entries of other workloads are kept while the kernel sources are those
    they were taken on."""
    import csv
    import hashlib

    import workloads as wl

    def per_kernel(path, counter):
        vals = {}
        for r in csv.DictReader(open(path)):
            if r["Counter_Name"] != counter:
                continue
            vals.setdefault(r["Kernel_Name"], []).append(float(r["Counter_Value"]) * 1024.0)  # KiB -> bytes
        return vals

    wname, mname, kernel = PROBE_WORKLOADS[workload]
    w, mode = getattr(wl, wname), getattr(wl, mname)
    counters = {}
    for name, path, counter, truth in (("fetch", fetch_csv, "FETCH_SIZE", 1 << 30), ("write", write_csv, "WRITE_SIZE", 1 << 30)):
        vals = per_kernel(path, counter)
        copy = max(v for k, v_ in vals.items() if "copyBuffer" in k or "copy" in k.lower() for v in v_)
        factor = truth / copy
        dec = [v for k, v_ in vals.items() if "decode_quant_kernel" in k for v in v_]
        prep = [v for k, v_ in vals.items() if "qprep_kernel" in k for v in v_]
        counters[name] = {"counter": counter, "copy_reads": copy, "factor": factor,
                          "decode_raw": sum(dec) / len(dec), "prep_raw": sum(prep) / len(prep) if prep else 0.0}
    h = hashlib.sha256()
    for f in TRAFFIC_SOURCES:
        h.update((ROOT / f).read_bytes())
    path = ROOT / "profiles" / "traffic.json"
    rec = json.loads(path.read_text()) if path.exists() else {}
    if rec.get("sha256") != h.hexdigest():
        rec = {}
    rec.update({
        "sources": TRAFFIC_SOURCES, "sha256": h.hexdigest(),
        "method": "rocprofv3 --pmc FETCH_SIZE, then --pmc WRITE_SIZE, of `python bench.py --probe-traffic "
                  "--probe-workload <workload>`; each counter scaled by its reading for a 1 GiB device copy in "
                  "the same run",
    })
    fetch = counters["fetch"]["decode_raw"] * counters["fetch"]["factor"]
    write = counters["write"]["decode_raw"] * counters["write"]["factor"]
    rec.setdefault("workloads", {})[f"{w.name}/{mode.name}"] = {
        "kernel": kernel,
        "bytes_per_launch": round(fetch) + round(write),
        "fetch_bytes": round(fetch),
        "write_bytes": round(write),
        "algorithmic_bytes": split_bytes(w, mode),
        "ratio_to_algorithmic": (fetch + write) / split_bytes(w, mode),
        "counters": counters,
    }
    (ROOT / "profiles").mkdir(exist_ok=True)
    path.write_text(json.dumps(rec, indent=1) + "\n")
    log(json.dumps(rec["workloads"], indent=1))
    return 0


def probe_traffic(chunk: int, workload: str = "k4v4-32k", log=print) -> int:
    """For a counter run (rocprofv3 --pmc FETCH_SIZE or WRITE_SIZE): a plain
    device copy of 1 GiB (the calibration), then three split-kernel launches
    of one 32K workload (the headline K4V4 one by default, or K8V4)."""
    import torch

    import decode_attention_quantized_kvq_amd as kvq
    import workloads as wl
    from workloads.device import fill, positions, queries

    wname, mname, _ = PROBE_WORKLOADS[workload]
    w, mode = getattr(wl, wname), getattr(wl, mname)
    cache = kvq.alloc_cache(w.batch, w.n_kv_heads, w.head_dim, w.capacity, mode.k_bits, mode.v_bits,
                            _group(mode, w), w.n_anchor, w.window)
    fill([cache], w, 0, w.n_pos)
    q = queries(w, 0)
    ch = kvq.kvq_chunk_tokens(cache, w.n_q_heads, w.n_pos) if chunk == 0 else chunk
    ws_bytes = kvq.kvq_workspace_bytes(cache, w.n_q_heads, w.n_pos, chunk)
    ws = torch.empty(ws_bytes // 4 + 64, dtype=torch.float32, device="cuda")
    lens = positions([w.n_pos] * w.batch)
    src = torch.ones(1 << 28, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    dst.copy_(src)                                   # 1 GiB read, 1 GiB written
    torch.cuda.synchronize()
    for _ in range(3):
        kvq.kvq_decode_partials(cache, q, w.n_q_heads, lens, w.n_pos, 0.0, chunk, ws, ws_bytes)
    torch.cuda.synchronize()
    log(f"[bench] traffic probe: copy 1 GiB, 3 launches of {w.name}/{mode.name} (chunk {ch})")
    return 0


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--chunk", type=int, default=0, help="split-K chunk (0 = the library's choice)")
    ap.add_argument("--modes", choices=["headline", "targets", "paged", "all"], default="all",
                    help="headline: the K4V4 32K line only; targets: + K8V4 at 32K; paged: + both 32K "
                         "workloads in 256-slot pages and bulk prefill; all: every workload")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--probe-traffic", action="store_true",
                    help="copy 1 GiB then launch the split kernel of --probe-workload 3 times (for counter runs)")
    ap.add_argument("--probe-workload", choices=sorted(PROBE_WORKLOADS), default="k4v4-32k",
                    help="the workload --probe-traffic launches and --record-traffic records")
    ap.add_argument("--record-traffic", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="write profiles/traffic.json from the two counter runs (CPU only)")
    ap.add_argument("--only", default="",
                    help="comma-separated workload names: time only these lines of --modes all (plus the headline)")
    ap.add_argument("--quiet", action="store_true")
    args = ap.parse_args()
    only = set(x for x in args.only.split(",") if x)

    if args.record_traffic:
        return record_traffic(*args.record_traffic, args.probe_workload)
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}, WORLD_SIZE {world}); "
              "the sharded design is described in DESIGN.md but not built", file=sys.stderr)
        return 2

    import torch
    import workloads as wl

    log = (lambda *a, **k: None) if args.quiet else (lambda *a, **k: print(*a, **k, file=sys.stderr, flush=True))
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 1
    import decode_attention_quantized_kvq_amd as kvq
    kvq.lib()
    dev = torch.cuda.get_device_properties(0)
    log(f"[bench] device: {dev.name} ({dev.multi_processor_count} CUs)")
    if args.probe_traffic:
        return probe_traffic(args.chunk, args.probe_workload, log=log)

    def want(name):
        return not only or name in only

    head_w, head_m = wl.K4V4_32K, wl.K4V4
    head = run_mode(head_w, head_m, args.steps, args.warmup, args.chunk, log=log)
    extra = []
    if args.modes in ("targets", "all") and want("k8v4-32k"):
        extra.append(run_mode(wl.K8V4_32K, wl.K8V4, args.steps, args.warmup, args.chunk, log=log))
    if args.modes in ("paged", "all") and want("paged"):
        extra.append(run_mode(wl.K4V4_32K, wl.K4V4, args.steps, args.warmup, args.chunk, log=log, page_size=256))
        extra.append(run_mode(wl.K8V4_32K, wl.K8V4, args.steps, args.warmup, args.chunk, log=log, page_size=256))
    if args.modes == "all":
        if want("k4v4-32k-modes"):
            extra.append(run_mode(wl.K4V4_32K, wl.FP16, args.steps, args.warmup, args.chunk, log=log))
            extra.append(run_mode(wl.K4V4_32K, wl.K4V4_G32, args.steps, args.warmup, args.chunk, log=log))
            extra.append(run_mode(wl.K4V4_32K, wl.K4V8, args.steps, args.warmup, args.chunk, log=log))
            extra.append(run_mode(wl.K4V4_32K, wl.K4V4_ZP, args.steps, args.warmup, args.chunk, log=log))
        if want("k4v4-window"):
            extra.append(run_mode(wl.K4V4_WINDOW, wl.K4V4, args.steps, args.warmup, args.chunk, flush=True, log=log))
        if want("k8v4-8k"):
            for m in wl.K8V4_8K.modes:
                extra.append(run_mode(wl.K8V4_8K, m, args.steps, args.warmup, args.chunk, flush=True, log=log))
        if want("tinyloop"):
            for m in wl.TINYLOOP.modes:
                extra.append(run_mode(wl.TINYLOOP, m, max(3, args.steps // 4), 2, args.chunk, log=log))
            # bit widths per layer: int8 in the first and last two layers, int4 between
            n_l = wl.TINYLOOP.n_layers
            per_layer = [wl.K8V8 if li < 2 or li >= n_l - 2 else wl.K4V4 for li in range(n_l)]
            extra.append(run_mode(wl.TINYLOOP, wl.Mode("k8v8-ends-k4v4", 4, 4), max(3, args.steps // 4), 2,
                                  args.chunk, log=log, layer_modes=per_layer))
        if want("tiny"):
            for m in wl.TINY.modes:
                extra.append(run_mode(wl.TINY, m, args.steps, args.warmup, args.chunk, log=log))
    gens = [generation_loop(wl.MNIML, m, log=log) for m in wl.MNIML.modes] \
        if args.modes == "all" and want("mniml") else []
    prefills = []
    if args.modes in ("paged", "all") and want("prefill"):
        prefills = [prefill(wl.K4V4_32K, wl.K4V4, log=log), prefill(wl.K8V4_32K, wl.K8V4, log=log),
                    prefill(wl.K4V4_32K, wl.FP16, log=log)]

    probe = read_probe(log=log)
    cpu = None if args.no_cpu_baseline else cpu_baseline(head_w, head_m, log=log)
    tr = traffic_record(f"{head_w.name}/{head_m.name}")
    traffic = None if tr is None else tr["bytes_per_launch"]
    for r in [head] + extra:
        # counted HBM bytes of the split kernel, where a counter run covers it
        t = traffic_record(f"{r['workload']}/{r['mode']}") if r["page_size"] == 0 else None
        r["split_traffic_bytes"] = None if t is None else t["bytes_per_launch"]

    line = {
        "metric": METRIC,
        "value": round(head["step_GBps"], 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(head["ms_per_step"], 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "int4 K/V codes, int32 dot products (i4 x i4 keys, u8 x u8 values), f32 softmax",
        "data": "synthetic: seeded N(0,1) K/V/q (numpy PCG64), no model weights",
        "config": {"workload": head["workload"], "mode": head["mode"], "batch": head["batch"],
                   "n_q_heads": head["n_q_heads"], "n_kv_heads": head["n_kv_heads"], "head_dim": head["head_dim"],
                   "context": head["context"], "group_size": head["group_size"],
                   "chunk_tokens": head["chunk_tokens"], "parallelism": "single GPU"},
        "tokens_per_s": round(head["tokens_per_s"], 1),
        "pct_of_peak": round(100.0 * head["step_GBps"] / PEAK_HBM_GBS, 2),
        "roofline": {
            "bound": "hbm",
            "kernel": PROBE_WORKLOADS["k4v4-32k"][2],
            "achieved": round(head["split_GBps"], 2),
            "peak": PEAK_HBM_GBS,
            "unit": "GB/s",
            "frac": round(head["split_GBps"] / PEAK_HBM_GBS, 4),
            "traffic": traffic,
            "us_per_launch": round(head["us_split_back_to_back"], 3),
            "bytes_per_launch": head["split_bytes"],
            "frac_of_read_probe": round(head["split_GBps"] / probe["GBps"], 4),
        },
        "read_probe": probe,
        "cpu_baseline": cpu,
        "modes": {f"{r['workload']}/{r['mode']}": {k: (round(v, 4) if isinstance(v, float) else v)
                                                   for k, v in r.items()} for r in [head] + extra},
        "prefill": {f"{r['workload']}/{r['mode']}": {k: (round(v, 4) if isinstance(v, float) else v)
                                                     for k, v in r.items()} for r in prefills},
        "generation": {f"{r['workload']}/{r['mode']}": {k: (round(v, 4) if isinstance(v, float) else v)
                                                        for k, v in r.items()} for r in gens},
    }
    # one row per mode: split kernel rate, step time and tokens/s
    line["summary"] = [
        {"line": f"{r['workload']}/{r['mode']}", "split_GBps": round(r["split_GBps"], 1),
         "split_pct_of_peak": round(r["split_pct_of_peak"], 2), "step_us": round(r["ms_per_step"] * 1e3, 2),
         "step_GBps": round(r["step_GBps"], 1), "tokens_per_s": round(r["tokens_per_s"], 1),
         "cold": r["mall_scrub"]} for r in [head] + extra
    ] + [
        {"line": f"generation {r['workload']}/{r['mode']}", "us_per_token": round(r["us_per_token_graph"], 2),
         "tokens_per_s": round(r["tokens_per_s_graph"], 1)} for r in gens
    ]
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
