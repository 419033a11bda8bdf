#!/usr/bin/env python3
"""Decode-attention throughput over a quantized KV cache on one MI355X.

One step = the whole hot path for one batch: quantize-append the step's new
K/V row of every sequence and KV head into the cache (kvq_append), split-K
decode attention over the cache (kvq_decode_partials) and the merge of the
chunk partials (kvq_combine).  Inputs are resident in HBM before timing.

The headline workload is 32 sequences x 32 query heads / 8 KV heads x
head_dim 128 at a 32K-token context with nibble-packed int4 K and V
(one fp16 scale per head and position).  `value` is whole-step throughput in
GB/s of algorithmic bytes (the bytes the method must move: the cache it
streams, q in, out, and the appended rows); `roofline` prices the split-K
kernel alone against MI355X's 8 TB/s HBM peak.

    python bench.py [--steps K] [--warmup W] [--modes headline|targets|all]

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
    """Cache bytes per position per KV head (fp16 scales included)."""
    import decode_attention_quantized_kvq_amd as kvq
    g = _group(mode, w)
    return kvq.kvq_bytes_per_token(mode.k_bits, mode.v_bits, w.n_kv_heads, w.head_dim, g) / w.n_kv_heads


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


def run_mode(w, mode, steps: int, warmup: int, chunk: int = 0, flush: bool = False, log=print) -> dict:
    import torch

    import decode_attention_quantized_kvq_amd as kvq
    from workloads.device import fill, positions, queries

    t_fill = time.perf_counter()
    layers = []
    for layer in range(w.n_layers):
        cache = kvq.alloc_cache(w.batch, w.n_kv_heads, w.head_dim, w.capacity, mode.k_bits, mode.v_bits,
                                _group(mode, w), w.n_anchor, w.window)
        k_last, v_last = fill([cache], w, layer, w.n_pos)
        q = queries(w, layer)
        layers.append((cache, k_last, v_last, q))
    log(f"[bench] {w.name} {mode.name}: {w.n_layers} layer(s) filled in {time.perf_counter() - t_fill:.1f} s")

    max_len = w.n_pos
    ch = kvq.kvq_chunk_tokens(layers[0][0], w.n_q_heads, max_len) if chunk == 0 else chunk
    n_chunks = -(-min(max_len, w.capacity) // ch)
    ws_bytes = kvq.kvq_workspace_bytes(layers[0][0], w.n_q_heads, max_len, ch)
    ws = torch.empty(ws_bytes // 4 + 64, dtype=torch.float32, device="cuda")
    out = torch.empty((w.batch, w.n_q_heads, w.head_dim), dtype=torch.float32, device="cuda")
    pos = positions([w.n_pos - 1] * w.batch)
    lens = positions([w.n_pos] * w.batch)
    scrub = torch.empty(1 << 28, dtype=torch.float32, device="cuda") if flush else None   # 1 GiB > 256 MB MALL
    stream = torch.cuda.current_stream()

    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(steps * w.n_layers)]

    def one_step(record):
        for li, (cache, k_last, v_last, q) in enumerate(layers):
            e = ev[record * w.n_layers + li] if record is not None else None
            if scrub is not None:
                scrub.zero_()
            if e: e[0].record(stream)
            kvq.kvq_append(cache, k_last, v_last, 1, pos, stream)
            if e: e[1].record(stream)
            kvq.kvq_decode_partials(cache, q, w.n_q_heads, lens, max_len, 0.0, ch, ws, ws_bytes, stream)
            if e: e[2].record(stream)
            kvq.kvq_combine(w.batch, w.n_q_heads, w.head_dim, n_chunks, ws, ws_bytes, out, stream)
            if e: e[3].record(stream)

    for _ in range(warmup):
        one_step(None)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s in range(steps):
        one_step(s)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0

    t_app = sum(e[0].elapsed_time(e[1]) for e in ev) / len(ev)
    t_split = sum(e[1].elapsed_time(e[2]) for e in ev) / len(ev)
    t_comb = sum(e[2].elapsed_time(e[3]) for e in ev) / len(ev)
    ms_step_wall = wall / steps * 1e3
    ms_step_gpu = (t_app + t_split + t_comb) * w.n_layers
    sbytes = step_bytes(w, mode) * w.n_layers
    # with the MALL scrub inside the loop, wall time includes it: rate from kernel events then
    ms_step = ms_step_gpu if flush else ms_step_wall
    res = {
        "workload": w.name, "mode": mode.name, "batch": w.batch, "n_q_heads": w.n_q_heads,
        "n_kv_heads": w.n_kv_heads, "head_dim": w.head_dim, "context": attended(w), "n_layers": w.n_layers,
        "capacity": w.capacity, "n_anchor": w.n_anchor, "window": w.window, "group_size": _group(mode, w),
        "chunk_tokens": ch, "n_chunks": n_chunks, "mall_scrub": flush,
        "ms_per_step": ms_step, "ms_per_step_wall": ms_step_wall, "ms_per_step_kernels": ms_step_gpu,
        "step_GBps": sbytes / (ms_step * 1e-3) / 1e9,
        "tokens_per_s": w.batch / (ms_step * 1e-3),
        "us_append": t_app * 1e3, "us_split": t_split * 1e3, "us_combine": t_comb * 1e3,
        "split_bytes": split_bytes(w, mode), "split_GBps": split_bytes(w, mode) / (t_split * 1e-3) / 1e9,
    }
    res["split_pct_of_peak"] = 100.0 * res["split_GBps"] / PEAK_HBM_GBS
    log(f"[bench] {w.name} {mode.name}: step {ms_step * 1e3:.1f} us ({res['step_GBps']:.0f} GB/s, "
        f"{res['tokens_per_s']:.0f} tok/s); split {t_split * 1e3:.1f} us = {res['split_GBps']:.0f} GB/s "
        f"({res['split_pct_of_peak']:.1f}% of peak); append {t_app * 1e3:.1f} us, combine {t_comb * 1e3:.1f} us")
    del layers, ws, out, scrub
    torch.cuda.empty_cache()
    return res


def cpu_baseline(w, mode, log=print) -> dict:
    """The CPU oracle's decode step, untuned, on a bounded sample of the
    workload: whole sequences (every KV and query head, the full context),
    one per thread."""
    import numpy as np

    import oracle
    import workloads as wl

    oracle.lib()
    cores = max(1, min(16, os.cpu_count() or 1, w.batch))
    seqs = list(range(cores))
    data = {}
    for b in seqs:
        data[b] = (wl.rows(w, wl.K_STREAM, 0, b, w.n_pos), wl.rows(w, wl.V_STREAM, 0, b, w.n_pos), wl.query(w, 0, b))
    g = _group(mode, w)
    scale = 1.0 / np.sqrt(w.head_dim)

    def work(b):
        K, V, q = data[b]
        oracle.decode_step(mode.k_bits, mode.v_bits, g, w.n_anchor, w.window, K, V, q, scale)

    threads = [threading.Thread(target=work, args=(b,)) for b in seqs]
    t0 = time.perf_counter()
    for t in threads:
        t.start()
    for t in threads:
        t.join()
    dt = time.perf_counter() - t0
    frac = len(seqs) / w.batch
    sample_bytes = step_bytes(w, mode) * frac
    log(f"[bench] cpu oracle: {len(seqs)} sequence(s) on {cores} thread(s) in {dt:.2f} s")
    return {
        "value": sample_bytes / dt / 1e9, "unit": "GB/s", "cores": cores, "kind": "oracle",
        "sample": f"{len(seqs)} of {w.batch} sequences of {w.name} ({mode.name}), every head, "
                  f"full {attended(w)}-position context, one sequence per thread; float64 oracle "
                  f"(encode every row, then softmax attention); {dt:.2f} s wall",
        "tokens_per_s": len(seqs) / dt,
    }


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--chunk", type=int, default=0, help="split-K chunk (0 = the library's choice)")
    ap.add_argument("--modes", choices=["headline", "targets", "all"], default="targets",
                    help="headline: the K4V4 32K line only; targets: + K8V4 at 32K; all: every workload")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--quiet", action="store_true")
    args = ap.parse_args()

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

    head_w, head_m = wl.K4V4_32K, wl.K4V4
    head = run_mode(head_w, head_m, args.steps, args.warmup, args.chunk, log=log)
    extra = []
    if args.modes in ("targets", "all"):
        extra.append(run_mode(wl.K8V4_32K, wl.K8V4, args.steps, args.warmup, args.chunk, log=log))
    if args.modes == "all":
        extra.append(run_mode(wl.K4V4_32K, wl.FP16, args.steps, args.warmup, args.chunk, log=log))
        extra.append(run_mode(wl.K4V4_WINDOW, wl.K4V4, args.steps, args.warmup, args.chunk, flush=True, log=log))
        for m in wl.K8V4_8K.modes:
            extra.append(run_mode(wl.K8V4_8K, m, args.steps, args.warmup, args.chunk, flush=True, log=log))
        for m in wl.TINYLOOP.modes:
            extra.append(run_mode(wl.TINYLOOP, m, max(3, args.steps // 4), 2, args.chunk, log=log))
        for m in wl.TINY.modes:
            extra.append(run_mode(wl.TINY, m, args.steps, args.warmup, args.chunk, log=log))

    cpu = None if args.no_cpu_baseline else cpu_baseline(head_w, head_m, log=log)

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
        "dtype": "int4 (i32 dot on K codes, f16->f32 on V codes)",
        "data": "synthetic: seeded N(0,1) K/V/q (numpy PCG64), no model weights",
        "config": {"workload": head["workload"], "mode": head["mode"], "batch": head["batch"],
                   "n_q_heads": head["n_q_heads"], "n_kv_heads": head["n_kv_heads"], "head_dim": head["head_dim"],
                   "context": head["context"], "group_size": head["group_size"],
                   "chunk_tokens": head["chunk_tokens"], "parallelism": "single GPU"},
        "tokens_per_s": round(head["tokens_per_s"], 1),
        "pct_of_peak": round(100.0 * head["step_GBps"] / PEAK_HBM_GBS, 2),
        "roofline": {
            "bound": "hbm",
            "kernel": "decode_split_kernel<4,4,128,4>",
            "achieved": round(head["split_GBps"], 2),
            "peak": PEAK_HBM_GBS,
            "unit": "GB/s",
            "frac": round(head["split_GBps"] / PEAK_HBM_GBS, 4),
            "traffic": None,
            "us_per_launch": round(head["us_split"], 3),
            "bytes_per_launch": head["split_bytes"],
        },
        "cpu_baseline": cpu,
        "modes": {f"{r['workload']}/{r['mode']}": {k: (round(v, 4) if isinstance(v, float) else v)
                                                   for k, v in r.items()} for r in [head] + extra},
    }
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
