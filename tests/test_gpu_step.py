"""The short decode step: when a step's context spans at most 2 chunks per
(sequence, KV head) on an 8/4-bit cache, kvq_decode_step runs as a single
kernel whose workgroups store the new rows of their chunk, prepare their
query and write the output (one chunk) or partials that the last workgroup
of the (sequence, KV head) merges, setting its ticket counter back to zero;
at 3 or 4 chunks as two launches, the split kernel merging in its last
workgroups.  Either must leave the cache and the output bit for bit as
kvq_append followed by kvq_decode_attn with the same chunk does (a split
launch and the combine), and match the oracle."""
import numpy as np
import pytest

from gpu_util import assert_close, check_codes, linear_slots, need_gpu, paged_table, softmax_default, window_slots

pytestmark = pytest.mark.gpu

PAIRS = [(8, 8), (8, 4), (4, 4), (4, 8)]


def _data(B, H, n, HD, Hq, seed):
    rng = np.random.default_rng(seed)
    K = rng.standard_normal((B, H, n, HD)).astype(np.float32)
    V = rng.standard_normal((B, H, n, HD)).astype(np.float32)
    q = rng.standard_normal((B, Hq, HD)).astype(np.float32)
    return K, V, q


def _pair(oq, kb, vb, gs, B, H, G, HD, n, n_new, chunk, seed, n_anchor=0, window=0, lens=None, page=0,
          scale=0.0, reps=1):
    """One step through kvq_decode_step on one cache and through kvq_append +
    kvq_decode_attn on another; the two must agree bit for bit."""
    kvq = need_gpu()
    import torch
    from workloads.device import positions, to_device
    Hq = H * G
    K, V, q = _data(B, H, n, HD, Hq, seed)
    cap = n_anchor + window if window else n
    if page:
        cap = (cap + page - 1) // page * page
        pps = cap // page
        table = paged_table(B, pps, B * pps + 2, seed)   # the same pages for both caches
        tables = [table, table.copy()]
        caches = [kvq.alloc_cache(B, H, HD, cap, kb, vb, gs, n_anchor, window, page_size=page,
                                  n_pages=B * pps + 2, block_table=to_device(t)) for t in tables]
    else:
        caches = [kvq.alloc_cache(B, H, HD, cap, kb, vb, gs, n_anchor, window) for _ in range(2)]
    n0 = n - n_new
    for c in caches:
        if n0:
            kvq.kvq_append(c, to_device(K[:, :, :n0]), to_device(V[:, :, :n0]), n0, positions([0] * B))
    kn, vn, qd = to_device(K[:, :, n0:]), to_device(V[:, :, n0:]), to_device(q)
    lens = lens or [n] * B
    pos, sl = positions([n0] * B), positions(lens)
    max_len = max(max(lens), 1)
    ws_bytes = kvq.kvq_workspace_bytes(caches[0], Hq, max_len, chunk)
    assert kvq.kvq_chunk_count(caches[0], Hq, max_len, chunk) <= 4     # the one-launch path
    outs = [torch.full((B, Hq, HD), 7.0, dtype=torch.float32, device="cuda") for _ in range(2)]
    # the step's workspace zero-filled (its ticket counters), the separate calls' any
    wss = [torch.full((ws_bytes // 4 + 64,), v, dtype=torch.float32, device="cuda") for v in (0.0, 3.0)]
    for _ in range(reps):                            # later steps find the counters back at zero
        kvq.kvq_decode_step(caches[0], kn, vn, n_new, pos, qd, Hq, sl, max_len, scale, chunk, outs[0], wss[0],
                            ws_bytes)
    kvq.kvq_append(caches[1], kn, vn, n_new, pos)
    kvq.kvq_decode_attn(caches[1], qd, Hq, sl, max_len, scale, chunk, outs[1], wss[1], ws_bytes)
    torch.cuda.synchronize()
    assert torch.equal(outs[0], outs[1]), "one-launch step differs from append + decode_attn"
    for name in ("k_codes", "v_codes", "k_scales", "v_scales"):
        a, b_ = getattr(caches[0], name), getattr(caches[1], name)
        if a is not None:
            assert torch.equal(a, b_), name
    got = outs[0].cpu().numpy()
    if not page:
        slots = window_slots(oq, n, n_anchor, window) if window else linear_slots(n, cap)
        check_codes(oq, caches[0], K, V, slots)
    sigma = scale or softmax_default(HD)
    for b in range(B):
        Lb = n if window else min(lens[b], cap)
        if Lb == 0:
            assert np.all(got[b] == 0)
            continue
        want = oq.decode_step(kb, vb, gs, n_anchor, window, K[b][:, :Lb], V[b][:, :Lb], q[b], sigma)
        assert_close(got[b], want, f"one-launch step kb={kb} vb={vb} g={gs} b={b}")
    return caches[0], outs[0]


@pytest.mark.parametrize("kb,vb", PAIRS)
@pytest.mark.parametrize("group", [0, 32, -1])
@pytest.mark.parametrize("G", [1, 4, 8])
@pytest.mark.parametrize("n_new", [0, 1, 3])
def test_one_launch_step(oq, kb, vb, group, G, n_new):
    HD = 64 if G == 8 else 128
    H = 2
    gs = HD if group == 0 else (H * HD if group == -1 else group)
    _pair(oq, kb, vb, gs, B=2, H=H, G=G, HD=HD, n=700, n_new=n_new, chunk=1024, seed=kb * 13 + vb + G + n_new)


@pytest.mark.parametrize("kb,vb", [(8, 8), (4, 4)])
def test_one_launch_step_library_chunk(oq, kb, vb):
    """Short contexts (Tiny: 257 positions; the mni-ml-like loop's 256) take
    the one-launch path with the library's own chunk."""
    _pair(oq, kb, vb, 64, B=1, H=4, G=1, HD=64, n=257, n_new=1, chunk=0, seed=3)
    _pair(oq, kb, vb, 8 * 64, B=1, H=8, G=1, HD=64, n=256, n_new=1, chunk=0, seed=4)


@pytest.mark.parametrize("kb,vb", [(8, 4), (4, 4)])
def test_one_launch_step_window(oq, kb, vb):
    """Anchors + ring (64 + 512 slots) after 1500 positions, three rows per step."""
    _pair(oq, kb, vb, 128, B=2, H=2, G=4, HD=128, n=1500, n_new=3, chunk=1024, seed=11, n_anchor=64, window=512)


@pytest.mark.parametrize("kb,vb", [(8, 8), (4, 4)])
def test_one_launch_step_paged(oq, kb, vb):
    _pair(oq, kb, vb, 128, B=3, H=2, G=4, HD=128, n=640, n_new=1, chunk=1024, seed=12, page=128)


def test_one_launch_step_ragged(oq):
    """A sequence that attends nothing (its rows are still stored), one that
    attends a prefix, and an explicit softmax scale."""
    _pair(oq, 8, 4, 128, B=3, H=2, G=4, HD=128, n=600, n_new=1, chunk=1024, seed=13, lens=[600, 0, 300])
    _pair(oq, 4, 4, 32, B=2, H=2, G=4, HD=128, n=600, n_new=1, chunk=1024, seed=14, scale=0.5)


def test_one_launch_step_graph(oq):
    """The one-launch step captured in a HIP graph gives the eager output bit
    for bit on every replay, with eager work between replays."""
    kvq = need_gpu()
    import torch
    from workloads.device import positions, to_device
    B, H, G, HD, n = 2, 2, 4, 128, 400
    cache = kvq.alloc_cache(B, H, HD, n, 4, 4, HD)
    K, V, q = _data(B, H, n, HD, H * G, 21)
    kvq.kvq_append(cache, to_device(K[:, :, : n - 1]), to_device(V[:, :, : n - 1]), n - 1, positions([0, 0]))
    k1, v1, qd = to_device(K[:, :, n - 1:]), to_device(V[:, :, n - 1:]), to_device(q)
    pos, lens = positions([n - 1] * B), positions([n] * B)
    assert kvq.kvq_chunk_tokens(cache, H * G, n) >= n          # one chunk: the one-launch path
    ws_bytes = kvq.kvq_workspace_bytes(cache, H * G, n, 0)
    ws = torch.empty(ws_bytes // 4 + 64, dtype=torch.float32, device="cuda")
    out = torch.zeros((B, H * G, HD), dtype=torch.float32, device="cuda")

    def step(st):
        kvq.kvq_decode_step(cache, k1, v1, 1, pos, qd, H * G, lens, n, 0.0, 0, out, ws, ws_bytes, st)

    step(torch.cuda.current_stream())
    torch.cuda.synchronize()
    want = out.clone()
    g = torch.cuda.CUDAGraph()
    cs = torch.cuda.Stream()
    cs.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(cs):
        step(cs)
    torch.cuda.synchronize()
    with torch.cuda.graph(g, stream=cs):
        step(cs)
    for r in range(3):
        out.zero_()
        ws.fill_(float(r + 1))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, want), f"replay {r}"
    got = want.cpu().numpy()
    for b in range(B):
        ref = oq.decode_step(4, 4, HD, 0, 0, K[b], V[b], q[b], softmax_default(HD))
        assert_close(got[b], ref, f"graph one-launch b={b}")


@pytest.mark.parametrize("kb,vb", PAIRS)
@pytest.mark.parametrize("n,n_new,chunk", [(700, 1, 512), (1024, 3, 512), (513, 1, 512), (600, 0, 512),
                                           (700, 1, 256), (1024, 3, 256)])
def test_one_launch_step_chunks(oq, kb, vb, n, n_new, chunk):
    """Two chunks per (sequence, KV head) in one launch (512-slot chunks):
    the new rows are stored by the workgroup of their chunk, the last
    workgroup merges; three or four (256-slot chunks) in two launches.
    Three steps in a row on one workspace (the counters come back to zero)."""
    _pair(oq, kb, vb, 128, B=2, H=2, G=4, HD=128, n=n, n_new=n_new, chunk=chunk, seed=kb + vb + n + n_new,
          reps=3)


@pytest.mark.parametrize("kb,vb", [(8, 4), (4, 4)])
def test_one_launch_step_chunks_window(oq, kb, vb):
    """Anchors + ring (64 + 512 slots: two 512-slot chunks, one launch, or
    three 256-slot ones); the step's rows land in the ring wherever the wrap
    puts them."""
    for n, seed, ch in ((1500, 51, 512), (1777, 52, 512), (1777, 53, 256)):
        _pair(oq, kb, vb, 128, B=2, H=2, G=4, HD=128, n=n, n_new=3, chunk=ch, seed=seed + kb, n_anchor=64,
              window=512, reps=2)


def test_one_launch_step_chunks_ragged_paged(oq):
    """Sequences attending nothing, a prefix, or all of four chunks (the rows
    are stored all the same); paged storage; group and per-position scales;
    an explicit softmax scale."""
    _pair(oq, 8, 4, 128, B=3, H=2, G=4, HD=128, n=1000, n_new=1, chunk=512, seed=61, lens=[1000, 0, 300])
    _pair(oq, 8, 4, 128, B=3, H=2, G=4, HD=128, n=1000, n_new=1, chunk=256, seed=65, lens=[1000, 0, 300])
    _pair(oq, 4, 4, 128, B=3, H=2, G=4, HD=128, n=1000, n_new=1, chunk=512, seed=62, page=128, reps=2)
    _pair(oq, 4, 8, 32, B=2, H=2, G=4, HD=128, n=900, n_new=2, chunk=512, seed=63, scale=0.5)
    _pair(oq, 8, 8, 2 * 64, B=2, H=2, G=1, HD=64, n=800, n_new=1, chunk=512, seed=64)


def test_one_launch_step_chunks_graph(oq):
    """Two chunks per (sequence, KV head), one launch, captured in a HIP
    graph: every replay gives the eager output bit for bit (the merge's
    ticket counters are back at zero after each), with eager work on other
    memory between replays."""
    kvq = need_gpu()
    import torch
    from workloads.device import positions, to_device
    B, H, G, HD, n, ch = 2, 2, 4, 128, 700, 512
    cache = kvq.alloc_cache(B, H, HD, n, 4, 4, HD)
    K, V, q = _data(B, H, n, HD, H * G, 22)
    kvq.kvq_append(cache, to_device(K[:, :, : n - 1]), to_device(V[:, :, : n - 1]), n - 1, positions([0, 0]))
    k1, v1, qd = to_device(K[:, :, n - 1:]), to_device(V[:, :, n - 1:]), to_device(q)
    pos, lens = positions([n - 1] * B), positions([n] * B)
    assert kvq.kvq_chunk_count(cache, H * G, n, ch) == 2
    ws_bytes = kvq.kvq_workspace_bytes(cache, H * G, n, ch)
    ws = torch.zeros(ws_bytes // 4 + 64, dtype=torch.float32, device="cuda")
    out = torch.zeros((B, H * G, HD), dtype=torch.float32, device="cuda")
    other = torch.zeros(1 << 20, dtype=torch.float32, device="cuda")

    def step(st):
        kvq.kvq_decode_step(cache, k1, v1, 1, pos, qd, H * G, lens, n, 0.0, ch, out, ws, ws_bytes, st)

    step(torch.cuda.current_stream())
    torch.cuda.synchronize()
    want = out.clone()
    g = torch.cuda.CUDAGraph()
    cs = torch.cuda.Stream()
    cs.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(cs):
        step(cs)
    torch.cuda.synchronize()
    with torch.cuda.graph(g, stream=cs):
        step(cs)
    for r in range(4):
        out.zero_()
        other.fill_(float(r + 1))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, want), f"replay {r}"
    got = want.cpu().numpy()
    for b in range(B):
        ref = oq.decode_step(4, 4, HD, 0, 0, K[b], V[b], q[b], softmax_default(HD))
        assert_close(got[b], ref, f"graph two-chunk step b={b}")


def test_shared_workspace_float_and_integer_layers(oq):
    """Layers of an FP16 cache and of 8/4-bit caches (one-launch steps over
    two chunks) sharing one workspace, sized by the largest need (the FP16
    layer's: its partials reach the end of its data), never cleared after
    the first step: several decode steps in a row, each layer's output bit
    for bit that of the same layer on a workspace of its own, and the cache
    contents the same."""
    kvq = need_gpu()
    import torch
    from workloads.device import positions, to_device
    B, H, G, HD, n0, steps = 4, 4, 1, 128, 900, 3
    modes = [(16, 16, HD), (8, 8, HD), (4, 4, 32)]
    Hq = H * G
    layers = []
    for li, (kb, vb, gs) in enumerate(modes):
        K, V, q = _data(B, H, n0 + steps, HD, Hq, 90 + li)
        pair = [kvq.alloc_cache(B, H, HD, n0 + steps, kb, vb, gs) for _ in range(2)]
        for c in pair:
            kvq.kvq_append(c, to_device(K[:, :, :n0]), to_device(V[:, :, :n0]), n0, positions([0] * B))
        layers.append((pair, K, V, q))
    n_max = n0 + steps
    needs = [kvq.kvq_workspace_bytes(p[0], Hq, n_max, 0) for p, *_ in layers]
    assert needs[0] == max(needs)                    # the FP16 layer's partials fill the shared extent
    for (p, *_), (kb, _, _) in zip(layers, modes):
        if kb < 16:
            assert kvq.kvq_chunk_count(p[0], Hq, n_max, 0) == 2   # one launch, merged by the last workgroup
    shared_bytes = max(needs)
    shared = torch.zeros(shared_bytes // 4 + 64, dtype=torch.float32, device="cuda")
    own = [torch.zeros(nb // 4 + 64, dtype=torch.float32, device="cuda") for nb in needs]
    for s in range(steps):
        t = n0 + s
        pos, lens = positions([t] * B), positions([t + 1] * B)
        for li, (pair, K, V, q) in enumerate(layers):
            k1, v1 = to_device(K[:, :, t:t + 1]), to_device(V[:, :, t:t + 1])
            qd = to_device(q * np.float32(1.0 + 0.1 * s))
            outs = [torch.full((B, Hq, HD), 9.0, dtype=torch.float32, device="cuda") for _ in range(2)]
            kvq.kvq_decode_step(pair[0], k1, v1, 1, pos, qd, Hq, lens, n_max, 0.0, 0, outs[0], shared, shared_bytes)
            kvq.kvq_decode_step(pair[1], k1, v1, 1, pos, qd, Hq, lens, n_max, 0.0, 0, outs[1], own[li], needs[li])
            torch.cuda.synchronize()
            assert torch.equal(outs[0], outs[1]), f"step {s} layer {li}: the shared workspace changed the output"
            if s == steps - 1:
                kb, vb, gs = modes[li]
                got = outs[0].cpu().numpy()
                for b in range(B):
                    ref = oq.decode_step(kb, vb, gs, 0, 0, K[b][:, :t + 1], V[b][:, :t + 1],
                                         q[b] * np.float32(1.0 + 0.1 * s), softmax_default(HD))
                    assert_close(got[b], ref, f"shared workspace layer {li} b={b}")
    for pair, *_ in layers:
        for name in ("k_codes", "v_codes", "k_scales", "v_scales"):
            a, b_ = getattr(pair[0], name), getattr(pair[1], name)
            assert (a is None and b_ is None) or torch.equal(a, b_), name


@pytest.mark.parametrize("kb,vb", PAIRS)
@pytest.mark.parametrize("group,chunk", [(32, 512), (64, 256), (32, 0)])
def test_split_head_step(oq, kb, vb, group, chunk):
    """Eight query heads per KV head with scale groups inside the head run as
    two workgroup heads of four per cache head: one launch merging two
    chunks, two launches over three, and the library's chunk."""
    _pair(oq, kb, vb, group, B=2, H=2, G=8, HD=128, n=700, n_new=1, chunk=chunk, seed=kb * 7 + vb + group + chunk)


def test_split_head_step_window_paged(oq):
    """The split heads over a ring with anchors (three rows a step) and over
    pages."""
    _pair(oq, 4, 4, 32, B=2, H=2, G=8, HD=128, n=1500, n_new=3, chunk=512, seed=31, n_anchor=64, window=512)
    _pair(oq, 8, 4, 64, B=3, H=2, G=8, HD=128, n=640, n_new=1, chunk=512, seed=32, page=128)
    _pair(oq, 4, 8, 32, B=2, H=2, G=8, HD=64, n=900, n_new=1, chunk=256, seed=33, page=64)
