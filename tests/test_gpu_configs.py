"""GPU parity on the five workloads at their full shapes, in the launch
configuration the bench times (library-chosen chunks): codes and scales
bit-exact and attention outputs within tolerance, on every sequence for the
small workloads and on sampled sequences (recomputed by the oracle one by
one) for the large ones."""
import numpy as np
import pytest

import workloads as wl
from gpu_util import (assert_close, assert_same_storage, cache_arrays, check_codes, group_size_of, linear_slots, need_gpu,
                      paged_table, window_slots)

pytestmark = pytest.mark.gpu


def _alloc(kvq, w, mode):
    gs = group_size_of(mode.k_bits, mode.v_bits, mode.group, w.n_kv_heads, w.head_dim)
    return kvq.alloc_cache(w.batch, w.n_kv_heads, w.head_dim, w.capacity, mode.k_bits, mode.v_bits, gs,
                           w.n_anchor, w.window), gs


def _check_sequence(oq, w, cache, gs, mode, layer, b, out_b, n_pos, q_b):
    K = wl.rows(w, wl.K_STREAM, layer, b, n_pos)
    V = wl.rows(w, wl.V_STREAM, layer, b, n_pos)
    # codes and scales of this sequence, bit-exact
    seq = cache.sequence(b)
    slots = window_slots(oq, n_pos, w.n_anchor, w.window) if w.window else linear_slots(n_pos, w.capacity)
    check_codes(oq, seq, K[None], V[None], slots)
    want = oq.decode_step(mode.k_bits, mode.v_bits, gs, w.n_anchor, w.window, K, V, q_b,
                          1.0 / np.sqrt(w.head_dim))
    return assert_close(out_b, want, f"{w.name} {mode.name} layer={layer} b={b}")


def _run(oq, w, modes, sample_b, layers=(0,)):
    kvq = need_gpu()
    import torch
    from workloads.device import decode, fill, positions, queries
    for layer in layers:
        made = [(_alloc(kvq, w, m), m) for m in modes]
        caches = [c for (c, _), _ in made]
        # positions 0 .. n_pos-2 as the cached context, then the step's row
        fill(caches, w, layer, w.n_pos)
        q = queries(w, layer)
        qn = q.cpu().numpy()
        lens = positions([w.n_pos] * w.batch)
        for (cache, gs), m in made:
            out = decode(cache, q, w.n_q_heads, lens, w.n_pos).cpu().numpy()
            for b in sample_b:
                _check_sequence(oq, w, cache, gs, m, layer, b, out[b], w.n_pos, qn[b])
        del made, caches
        torch.cuda.empty_cache()


def test_tiny(oq):
    w = wl.TINY
    _run(oq, w, w.modes, sample_b=range(w.batch))


def test_tinyloop(oq):
    w = wl.TINYLOOP
    _run(oq, w, w.modes, sample_b=(0, 5, 7), layers=(0, 33))


def test_k8v4_8k(oq):
    w = wl.K8V4_8K
    _run(oq, w, w.modes, sample_b=(0, 9, 15))


def test_k8v4_32k(oq):
    w = wl.K8V4_32K
    _run(oq, w, w.modes, sample_b=(0, 15))


def test_k4v4_32k(oq):
    w = wl.K4V4_32K
    _run(oq, w, w.modes, sample_b=(0, 31))


def test_k4v4_32k_ragged(oq):
    """The library's chunks over a 32K context with per-sequence lengths that
    end inside a chunk, on a chunk boundary, in the last chunk, or at 0 and
    1 (empty chunks write empty partials)."""
    kvq = need_gpu()
    import torch
    from workloads.device import decode, fill, positions, queries
    w = wl.K4V4_32K
    (cache, gs), mode = _alloc(kvq, w, wl.K4V4), wl.K4V4
    fill([cache], w, 0, w.n_pos)
    q = queries(w, 0)
    qn = q.cpu().numpy()
    lens = [w.n_pos - 97 * b for b in range(w.batch)]
    special = {1: 30001, 2: 24577, 3: 24576, 4: 20000, 5: 513, 6: 1, 7: 0, 8: 4096}
    for b, L in special.items():
        lens[b] = L
    out = decode(cache, q, w.n_q_heads, positions(lens), w.n_pos).cpu().numpy()
    sc = 1.0 / np.sqrt(w.head_dim)
    for b in sorted(special) + [20]:
        L = lens[b]
        if L == 0:
            assert np.all(out[b] == 0)
            continue
        K = wl.rows(w, wl.K_STREAM, 0, b, L)
        V = wl.rows(w, wl.V_STREAM, 0, b, L)
        want = oq.decode_step(mode.k_bits, mode.v_bits, gs, 0, 0, K, V, qn[b], sc)
        assert_close(out[b], want, f"ragged b={b} L={L}")
    del cache
    torch.cuda.empty_cache()


@pytest.mark.parametrize("w,mode", [(wl.K4V4_32K, wl.K4V4), (wl.K8V4_32K, wl.K8V4)], ids=["k4v4-32k", "k8v4-32k"])
def test_32k_paged(oq, w, mode):
    """The 32K workloads in 256-slot pages, assigned in a random order (as
    the paged bench lines run them): the pages hold bit for bit what the
    contiguous cache holds, the outputs are bit for bit the contiguous
    cache's, and sampled sequences match the oracle."""
    kvq = need_gpu()
    import torch
    from workloads.device import decode, fill, positions, queries, to_device
    P = 256
    pps = w.capacity // P
    table = paged_table(w.batch, pps, w.batch * pps, 90)
    (contig, gs) = _alloc(kvq, w, mode)
    paged = kvq.alloc_cache(w.batch, w.n_kv_heads, w.head_dim, w.capacity, mode.k_bits, mode.v_bits, gs,
                            page_size=P, n_pages=w.batch * pps, block_table=to_device(table))
    fill([contig, paged], w, 0, w.n_pos)
    assert_same_storage(paged, table, contig)
    q = queries(w, 0)
    lens = positions([w.n_pos] * w.batch)
    oc, op = (decode(c, q, w.n_q_heads, lens, w.n_pos) for c in (contig, paged))
    torch.cuda.synchronize()
    assert torch.equal(oc, op)
    out, qn = op.cpu().numpy(), q.cpu().numpy()
    for b in (0, w.batch - 1):
        K = wl.rows(w, wl.K_STREAM, 0, b, w.n_pos)
        V = wl.rows(w, wl.V_STREAM, 0, b, w.n_pos)
        want = oq.decode_step(mode.k_bits, mode.v_bits, gs, 0, 0, K, V, qn[b], 1.0 / np.sqrt(w.head_dim))
        assert_close(out[b], want, f"{w.name} paged b={b}")
    del contig, paged
    torch.cuda.empty_cache()


@pytest.mark.parametrize("kb,vb", [(4, 4), (8, 8), (16, 16)])
def test_maximum_units(oq, kb, vb):
    """The largest grid the library launches: 8191 sequences x 8 KV heads =
    65528 (sequence, KV head) units (the limit is 65535), a 64-slot context
    appended in one bulk call and decoded; sampled sequences against the
    oracle, codes bit for bit."""
    kvq = need_gpu()
    import torch
    from workloads.device import decode, positions
    B, H, G, HD, n = 8191, 8, 1, 64, 64
    gen = torch.Generator(device="cuda").manual_seed(77 + kb)
    K = torch.randn((B, H, n, HD), device="cuda", generator=gen)
    V = torch.randn((B, H, n, HD), device="cuda", generator=gen)
    q = torch.randn((B, H * G, HD), device="cuda", generator=gen)
    cache = kvq.alloc_cache(B, H, HD, n, kb, vb, HD)
    kvq.kvq_append(cache, K, V, n, positions([0] * B))
    out = decode(cache, q, H * G, positions([n] * B), n).cpu().numpy()
    for b in (0, 4095, B - 1):
        Kb, Vb, qb = K[b].cpu().numpy(), V[b].cpu().numpy(), q[b].cpu().numpy()
        check_codes(oq, cache.sequence(b), Kb[None], Vb[None], linear_slots(n, n))
        want = oq.decode_step(kb, vb, HD, 0, 0, Kb, Vb, qb, 1.0 / np.sqrt(HD))
        assert_close(out[b], want, f"max units kb={kb} vb={vb} b={b}")
    del cache, K, V
    torch.cuda.empty_cache()


@pytest.mark.parametrize("kb,vb", [(4, 4), (8, 4), (16, 16)])
def test_million_position_context(oq, kb, vb):
    """One sequence and KV head with 2^20 positions (4 query heads): a bulk
    append of the whole context, then 1024 chunks of 1024 slots (2048 of 512
    for fp16) merged by the combine; the output against the oracle, codes
    bit for bit on 2000 sampled slots."""
    kvq = need_gpu()
    import torch
    from workloads.device import decode, positions, to_device
    B, H, G, HD, n = 1, 1, 4, 128, 1 << 20
    rng = np.random.default_rng(99 + kb)
    K = rng.standard_normal((B, H, n, HD), dtype=np.float32)
    V = rng.standard_normal((B, H, n, HD), dtype=np.float32)
    q = rng.standard_normal((B, H * G, HD), dtype=np.float32)
    cache = kvq.alloc_cache(B, H, HD, n, kb, vb, HD)
    kvq.kvq_append(cache, to_device(K), to_device(V), n, positions([0]))
    # >= 1024 workgroups for integer caches, >= 2048 for float ones
    assert kvq.kvq_chunk_tokens(cache, H * G, n) == (1024 if kb < 16 else 512)
    out = decode(cache, to_device(q), H * G, positions([n]), n).cpu().numpy()
    sample = {int(t): int(t) for t in np.unique(np.concatenate([rng.integers(0, n, 1990), np.arange(5), n - 5 + np.arange(5)]))}
    check_codes(oq, cache, K, V, sample)
    want = oq.decode_step(kb, vb, HD, 0, 0, K[0], V[0], q[0], 1.0 / np.sqrt(HD))
    assert_close(out[0], want, f"1M positions kb={kb} vb={vb}")
    del cache
    torch.cuda.empty_cache()


def test_k4v4_window(oq):
    w = wl.K4V4_WINDOW
    _run(oq, w, w.modes, sample_b=(0, 13, 31))


@pytest.mark.parametrize("mode", wl.MNIML.modes, ids=lambda m: m.name)
def test_mniml_generation_loop(oq, mode):
    """4-token prompt, then 252 steps of (append one row, attend); every
    step's output against the oracle."""
    kvq = need_gpu()
    import torch
    from workloads.device import positions, to_device
    w = wl.MNIML
    cache, gs = _alloc(kvq, w, mode)
    K = wl.rows(w, wl.K_STREAM, 0, 0, w.n_pos)
    V = wl.rows(w, wl.V_STREAM, 0, 0, w.n_pos)
    kvq.kvq_append(cache, to_device(K[None, :, :w.prompt]), to_device(V[None, :, :w.prompt]), w.prompt,
                   positions([0]))
    ws_bytes = kvq.kvq_workspace_bytes(cache, w.n_q_heads, w.capacity, 0)
    ws = torch.empty(ws_bytes // 4 + 64, device="cuda")
    out = torch.empty((1, w.n_q_heads, w.head_dim), device="cuda")
    worst = 0.0
    for step in range(w.n_pos - w.prompt):
        pos = w.prompt + step
        kvq.kvq_append(cache, to_device(np.ascontiguousarray(K[None, :, pos:pos + 1])),
                       to_device(np.ascontiguousarray(V[None, :, pos:pos + 1])), 1, positions([pos]))
        q = wl.query(w, 0, 0, step)
        kvq.kvq_decode_attn(cache, to_device(q[None]), w.n_q_heads, positions([pos + 1]), w.capacity, 0.0, 0, out,
                            ws, ws_bytes)
        got = out.cpu().numpy()[0]
        want = oq.decode_step(mode.k_bits, mode.v_bits, gs, 0, 0, K[:, :pos + 1], V[:, :pos + 1], q,
                              1.0 / np.sqrt(w.head_dim))
        worst = max(worst, assert_close(got, want, f"mniml {mode.name} step {step}")[0])
    check_codes(oq, cache, K[None], V[None], linear_slots(w.n_pos, w.capacity))
