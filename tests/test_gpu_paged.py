"""Paged storage on the GPU: a cache whose buffers are pools of pages,
addressed through a block table, holds bit for bit what a contiguous cache
holds once its pages are gathered in table order, and decodes to the same
outputs bit for bit (and within tolerance of the oracle), for every kernel
instantiation, window mode, ragged lengths, appends that cross pages, the
fused step, table entries that name no page, and the zero-point codec."""
import numpy as np
import pytest

from gpu_util import (BUFFERS, assert_close, assert_same_storage, group_size_of, need_gpu, paged_table,
                      softmax_default, unit_view)

pytestmark = pytest.mark.gpu

MODES = [(32, 32, 0), (16, 16, 0), (8, 8, 0), (8, 4, 0), (4, 4, 0), (4, 8, 0)]


def _data(B, H, n_pos, HD, Hq, seed):
    rng = np.random.default_rng(seed)
    K = rng.standard_normal((B, H, n_pos, HD)).astype(np.float32)
    V = rng.standard_normal((B, H, n_pos, HD)).astype(np.float32)
    q = rng.standard_normal((B, Hq, HD)).astype(np.float32)
    return K, V, q


def _paged(kvq, table, n_pages, B, H, HD, cap, kb, vb, gs, P, n_anchor=0, window=0, zp=0):
    from workloads.device import to_device
    bt = to_device(np.ascontiguousarray(table, np.int32))
    return kvq.alloc_cache(B, H, HD, cap, kb, vb, gs, n_anchor, window, page_size=P, n_pages=n_pages,
                           block_table=bt, zero_point=zp)


def _append_pieces(kvq, caches, K, V, pieces):
    from workloads.device import positions, to_device
    B, n_pos = K.shape[0], K.shape[2]
    p0 = 0
    for i, frac in enumerate(pieces):
        n = n_pos - p0 if i == len(pieces) - 1 else max(1, int(round(frac * n_pos)))
        kk, vv = to_device(K[:, :, p0:p0 + n]), to_device(V[:, :, p0:p0 + n])
        for c in caches:
            kvq.kvq_append(c, kk, vv, n, positions([p0] * B))
        p0 += n
    assert p0 == n_pos


def run_paged(oq, kb, vb, group, B=3, H=2, G=4, HD=128, P=64, n_pos=700, pieces=(0.3, 0.002, 0.5, 1.0),
              seq_lens=None, chunk=0, n_anchor=0, window=0, spare=5, seed=0, zp=0):
    kvq = need_gpu()
    import torch
    from workloads.device import decode, positions, to_device
    Hq = H * G
    K, V, q = _data(B, H, n_pos, HD, Hq, seed)
    if zp:
        # asymmetric ranges, so that the zero points matter
        rng = np.random.default_rng(seed + 1)
        K += np.float32(1.5) * rng.standard_normal((B, H, 1, HD)).astype(np.float32)
        V += np.float32(-0.8) + np.float32(0.5) * rng.standard_normal((B, H, n_pos, 1)).astype(np.float32)
    cap = n_anchor + window if window else (n_pos + P - 1) // P * P
    assert cap % P == 0
    pps = cap // P
    n_pages = B * pps + spare
    table = paged_table(B, pps, n_pages, seed)
    gs = group_size_of(kb, vb, group, H, HD)
    contig = kvq.alloc_cache(B, H, HD, cap, kb, vb, gs, n_anchor, window, zero_point=zp)
    paged = _paged(kvq, table, n_pages, B, H, HD, cap, kb, vb, gs, P, n_anchor, window, zp)
    _append_pieces(kvq, [contig, paged], K, V, pieces)
    torch.cuda.synchronize()
    assert_same_storage(paged, table, contig)

    lens = seq_lens if seq_lens is not None else [n_pos] * B
    qd = to_device(q)
    outs = [decode(c, qd, Hq, positions(lens), max(max(lens), 1), 0.0, chunk) for c in (contig, paged)]
    torch.cuda.synchronize()
    assert torch.equal(outs[0], outs[1]), "paged output differs from the contiguous cache's"
    got = outs[1].cpu().numpy()
    sc = softmax_default(HD)
    for b in range(B):
        L = n_pos if window else min(max(lens[b], 0), cap)
        if L == 0:
            assert np.all(got[b] == 0)
            continue
        want = oq.decode_step(kb, vb, gs, n_anchor, window, K[b][:, :L], V[b][:, :L], q[b], sc, asym=bool(zp))
        assert_close(got[b], want, f"paged P={P} kb={kb} vb={vb} HD={HD} G={G} zp={zp} b={b} L={L}")


@pytest.mark.parametrize("kb,vb,group", MODES)
@pytest.mark.parametrize("HD", [64, 128])
@pytest.mark.parametrize("P", [64, 256])
def test_paged_matches_contiguous(oq, kb, vb, group, HD, P):
    run_paged(oq, kb, vb, group, HD=HD, P=P, seq_lens=[700, 333, 1], seed=kb * 10 + vb + HD + P)


@pytest.mark.parametrize("kb,vb", [(4, 4), (8, 4), (16, 16)])
@pytest.mark.parametrize("G", [1, 2, 8])
def test_paged_gqa_groups(oq, kb, vb, G):
    run_paged(oq, kb, vb, 0, B=2, H=2, G=G, HD=128, P=128, n_pos=901, seed=G + kb)


@pytest.mark.parametrize("chunk", [256, 512, 2048])
def test_paged_chunks(oq, chunk):
    """Chunks smaller, equal and larger than the page; the wave ranges start
    inside pages and span several."""
    run_paged(oq, 4, 4, 0, B=2, H=2, G=4, HD=128, P=512, n_pos=3001, chunk=chunk, seq_lens=[3001, 2050],
              seed=chunk)
    run_paged(oq, 8, 4, 0, B=2, H=2, G=4, HD=64, P=64, n_pos=3001, chunk=chunk, seed=chunk + 1)


@pytest.mark.parametrize("kb,vb", [(8, 8), (4, 4)])
def test_paged_group_scales(oq, kb, vb):
    run_paged(oq, kb, vb, 32, B=2, H=2, G=4, HD=128, P=64, n_pos=515, seed=40 + kb)


@pytest.mark.parametrize("kb,vb", [(8, 8), (8, 4), (4, 4), (4, 8)])
def test_paged_per_row_scale(oq, kb, vb):
    run_paged(oq, kb, vb, -1, B=2, H=4, G=1, HD=64, P=64, n_pos=300, seed=41 + kb + vb)
    run_paged(oq, kb, vb, -1, B=2, H=2, G=4, HD=128, P=128, n_pos=600, seed=43 + kb + vb)


@pytest.mark.parametrize("kb,vb", [(4, 4), (16, 16)])
def test_paged_window(oq, kb, vb):
    """Anchors and a ring over pages: capacity 64 + 192 slots in 64-slot
    pages, a context that wraps the ring several times."""
    run_paged(oq, kb, vb, 0, B=2, H=2, G=4, HD=128, P=64, n_pos=700, n_anchor=64, window=192, seed=50 + kb)


ZP_PAIRS = [(8, 8), (8, 4), (4, 4), (4, 8)]


@pytest.mark.parametrize("kb,vb", ZP_PAIRS)
@pytest.mark.parametrize("group", [0, 32, -1])
@pytest.mark.parametrize("P", [64, 256])
def test_paged_zero_point(oq, kb, vb, group, P):
    """The zero-point codec on paged storage: per-head, 32-value group and
    per-position scale words, pages of 64 and 256 slots, ragged lengths."""
    H, G = (4, 1) if group == -1 else (2, 4)
    run_paged(oq, kb, vb, group, H=H, G=G, HD=128, P=P, seq_lens=[700, 333, 1], zp=1,
              seed=80 + kb * 10 + vb + P + max(group, 0))


@pytest.mark.parametrize("kb,vb", [(4, 4), (8, 4)])
def test_paged_zero_point_shapes(oq, kb, vb):
    """head_dim 64 with two scale groups, G = 2 and 8, a window over pages,
    and chunks that start inside pages."""
    run_paged(oq, kb, vb, 32, B=2, H=2, G=2, HD=64, P=64, n_pos=515, zp=1, seed=90 + kb)
    run_paged(oq, kb, vb, 0, B=2, H=2, G=8, HD=128, P=128, n_pos=901, zp=1, seed=91 + kb)
    run_paged(oq, kb, vb, 0, B=2, H=2, G=4, HD=128, P=64, n_pos=700, n_anchor=64, window=192, zp=1, seed=92 + kb)
    run_paged(oq, kb, vb, 0, B=2, H=2, G=4, HD=128, P=512, n_pos=3001, chunk=256, seq_lens=[3001, 2050], zp=1,
              seed=93 + kb)


@pytest.mark.parametrize("kb,vb,group", [(4, 4, 0), (8, 8, 0), (16, 16, 0), (8, 4, 0)])
def test_paged_invalid_entries(oq, kb, vb, group):
    """Table entries outside [0, n_pages) are skipped by the append and read
    as zero codes and scales: the cache and the output equal those of a
    cache whose entries name pages that are zeroed after the append."""
    kvq = need_gpu()
    import torch
    from workloads.device import decode, positions, to_device
    B, H, G, HD, P, n_pos = 2, 2, 4, 128, 64, 450
    K, V, q = _data(B, H, n_pos, HD, H * G, 60 + kb)
    cap = 512
    pps, n_pages = cap // P, B * (cap // P) + 4
    table = paged_table(B, pps, n_pages, 60 + kb)
    used = set(table.reshape(-1).tolist())
    spare = [u for u in range(n_pages) if u not in used]
    bad = table.copy()
    bad[1, 2], bad[1, 5], bad[0, 0] = -1, n_pages, -7
    good = table.copy()
    good[1, 2], good[1, 5], good[0, 0] = spare[0], spare[1], spare[2]
    gs = group_size_of(kb, vb, group, H, HD)
    cx = _paged(kvq, bad, n_pages, B, H, HD, cap, kb, vb, gs, P)
    cy = _paged(kvq, good, n_pages, B, H, HD, cap, kb, vb, gs, P)
    _append_pieces(kvq, [cx, cy], K, V, (0.5, 1.0))
    for name in BUFFERS:
        if getattr(cy, name) is not None:
            unit_view(cy, name)[torch.as_tensor(spare[:3], device="cuda")] = 0
    torch.cuda.synchronize()
    for name in BUFFERS:
        if getattr(cx, name) is not None:
            assert torch.equal(getattr(cx, name), getattr(cy, name)), f"{name}: an invalid page entry was written"
    qd = to_device(q)
    lens = positions([n_pos, n_pos - 10])
    ox, oy = (decode(c, qd, H * G, lens, n_pos) for c in (cx, cy))
    torch.cuda.synchronize()
    assert torch.equal(ox, oy)
    assert torch.all(torch.isfinite(ox))


@pytest.mark.parametrize("kb,vb,group,zp", [(4, 4, 0, 0), (8, 4, 0, 0), (16, 16, 0, 0), (4, 4, 32, 1), (8, 8, 0, 1)])
@pytest.mark.parametrize("n_new", [1, 3])
def test_paged_decode_step(oq, kb, vb, group, zp, n_new):
    """kvq_decode_step on a paged cache, its new rows crossing a page
    boundary, equals the separate calls on the same pages and on a
    contiguous cache (symmetric and zero-point codecs)."""
    kvq = need_gpu()
    import torch
    from workloads.device import positions, to_device
    B, H, G, HD, P = 2, 2, 4, 128, 64
    n0 = 3 * P - 1
    n = n0 + n_new
    cap = 4 * P
    pps, n_pages = 4, 2 * 4 + 3
    table = paged_table(B, pps, n_pages, 70 + n_new)
    gs = group_size_of(kb, vb, group, H, HD)
    K, V, q = _data(B, H, n, HD, H * G, 70 + n_new + kb)
    ps = [_paged(kvq, table, n_pages, B, H, HD, cap, kb, vb, gs, P, zp=zp) for _ in range(2)]
    contig = kvq.alloc_cache(B, H, HD, cap, kb, vb, gs, zero_point=zp)
    caches = ps + [contig]
    for c in caches:
        kvq.kvq_append(c, to_device(K[:, :, :n0]), to_device(V[:, :, :n0]), n0, positions([0] * B))
    kn, vn, qd = to_device(K[:, :, n0:]), to_device(V[:, :, n0:]), to_device(q)
    pos, lens = positions([n0] * B), positions([n] * B)
    ws_bytes = kvq.kvq_workspace_bytes(contig, H * G, n, 0)
    outs = [torch.full((B, H * G, HD), 7.0, dtype=torch.float32, device="cuda") for _ in range(3)]
    wss = [torch.empty(ws_bytes // 4 + 64, dtype=torch.float32, device="cuda") for _ in range(3)]
    wss[0].zero_()                                   # kvq_decode_step takes a zero-filled workspace
    kvq.kvq_decode_step(ps[0], kn, vn, n_new, pos, qd, H * G, lens, n, 0.0, 0, outs[0], wss[0], ws_bytes)
    for i in (1, 2):
        kvq.kvq_append(caches[i], kn, vn, n_new, pos)
        kvq.kvq_decode_attn(caches[i], qd, H * G, lens, n, 0.0, 0, outs[i], wss[i], ws_bytes)
    torch.cuda.synchronize()
    assert torch.equal(outs[0], outs[1]) and torch.equal(outs[0], outs[2])
    for name in BUFFERS:
        if getattr(contig, name) is not None:
            assert torch.equal(getattr(ps[0], name), getattr(ps[1], name)), name
    assert_same_storage(ps[0], table, contig)
    got = outs[0].cpu().numpy()
    for b in range(B):
        want = oq.decode_step(kb, vb, gs, 0, 0, K[b], V[b], q[b], softmax_default(HD), asym=bool(zp))
        assert_close(got[b], want, f"paged step kb={kb} vb={vb} zp={zp} n_new={n_new} b={b}")
