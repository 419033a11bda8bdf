"""GPU parity of the HIP path (through the C ABI) against the CPU oracle at
sizes the oracle finishes in seconds: several chunks, a ragged tail, every
kernel instantiation (widths x head_dim x GQA group), windows, groups."""
import numpy as np
import pytest

from gpu_util import (assert_close, cache_arrays, check_codes, group_size_of, linear_slots, need_gpu, softmax_default,
                      window_slots)

pytestmark = pytest.mark.gpu

MODES = [(32, 32, 0), (16, 16, 0), (8, 8, 0), (8, 4, 0), (4, 4, 0), (4, 8, 0)]


def _data(B, H, n_pos, HD, Hq, seed, outliers=False):
    rng = np.random.default_rng(seed)
    K = rng.standard_normal((B, H, n_pos, HD)).astype(np.float32)
    if outliers:
        K[:, :, :, ::23] *= np.float32(10.0)
    V = rng.standard_normal((B, H, n_pos, HD)).astype(np.float32)
    q = rng.standard_normal((B, Hq, HD)).astype(np.float32)
    return K, V, q


def run_case(oq, kb, vb, group, B=2, H=2, G=4, HD=128, n_pos=700, n_anchor=0, window=0, pieces=(1.0,),
             seq_lens=None, chunk=0, seed=0, outliers=False, check_all_codes=True):
    kvq = need_gpu()
    import torch
    from workloads.device import decode, positions, to_device

    Hq = H * G
    K, V, q = _data(B, H, n_pos, HD, Hq, seed, outliers)
    cap = n_anchor + window if window else n_pos
    gs = group_size_of(kb, vb, group, H, HD)
    cache = kvq.alloc_cache(B, H, HD, cap, kb, vb, gs, n_anchor, window)
    # append in pieces (fractions of n_pos), all sequences per call
    p0 = 0
    for i, frac in enumerate(pieces):
        n = n_pos - p0 if i == len(pieces) - 1 else max(1, int(round(frac * n_pos)))
        kvq.kvq_append(cache, to_device(K[:, :, p0:p0 + n]), to_device(V[:, :, p0:p0 + n]), n,
                       positions([p0] * B))
        p0 += n
    assert p0 == n_pos
    lens = seq_lens if seq_lens is not None else [n_pos] * B
    out = decode(cache, to_device(q), Hq, positions(lens), max(max(lens), 1), 0.0, chunk)
    torch.cuda.synchronize()
    got = out.cpu().numpy()

    if check_all_codes:
        slots = window_slots(oq, n_pos, n_anchor, window) if window else linear_slots(n_pos, cap)
        check_codes(oq, cache, K, V, slots)
    sc = softmax_default(HD)
    for b in range(B):
        L = min(max(lens[b], 0), cap) if not window else n_pos
        if L == 0:
            assert np.all(got[b] == 0)
            continue
        want = oq.decode_step(kb, vb, gs, n_anchor, window, K[b][:, :L], V[b][:, :L], q[b], sc)
        assert_close(got[b], want, f"kb={kb} vb={vb} g={gs} HD={HD} G={G} b={b} L={L}")
    return cache, got


@pytest.mark.parametrize("kb,vb,group", MODES)
@pytest.mark.parametrize("HD", [64, 128])
@pytest.mark.parametrize("G", [1, 2, 4, 8])
def test_every_instantiation(oq, kb, vb, group, HD, G):
    run_case(oq, kb, vb, group, B=2, H=2, G=G, HD=HD, n_pos=333, seed=kb * 100 + vb + HD + G)


@pytest.mark.parametrize("kb,vb", [(8, 8), (8, 4), (4, 4), (4, 8)])
@pytest.mark.parametrize("group", [32, 64])
def test_group_scales(oq, kb, vb, group):
    """Several fp16 scales per head row (the KVSplit-style group layout)."""
    run_case(oq, kb, vb, group, B=2, H=2, G=4, HD=128, n_pos=515, seed=7 + group, outliers=True)


@pytest.mark.parametrize("kb,vb", [(8, 8), (8, 4), (4, 4), (4, 8)])
@pytest.mark.parametrize("H,G,HD", [(4, 1, 64), (2, 4, 128), (2, 8, 64)])
def test_per_row_scale(oq, kb, vb, H, G, HD):
    """One scale per position over all KV heads (mni-ml's per-tensor INT8),
    at every integer width pair the descriptor accepts it for."""
    run_case(oq, kb, vb, -1, B=2, H=H, G=G, HD=HD, n_pos=300, seed=3 + kb * 10 + vb + G)


@pytest.mark.parametrize("chunk", [256, 512, 1024, 2048])
def test_chunk_sizes(oq, chunk):
    run_case(oq, 4, 4, 0, B=1, H=2, G=4, HD=128, n_pos=3001, chunk=chunk, seed=11)


@pytest.mark.parametrize("chunk", [64, 128, 512])
def test_chunk_sizes_float(oq, chunk):
    run_case(oq, 16, 16, 0, B=1, H=2, G=4, HD=128, n_pos=1001, chunk=chunk, seed=12)


@pytest.mark.parametrize("chunk", [4096, 8192])
def test_long_chunks(oq, chunk):
    """Chunks of several sub-chunks per wave (running maxima merged), int8 keys."""
    run_case(oq, 8, 4, 0, B=1, H=2, G=4, HD=128, n_pos=9000, chunk=chunk, seed=13, outliers=True)


def test_ragged_lengths(oq):
    """Different lengths per sequence, zero length, and lengths past capacity."""
    run_case(oq, 8, 4, 0, B=4, H=2, G=4, HD=128, n_pos=1000, seq_lens=[1000, 1, 0, 777], seed=5)
    run_case(oq, 16, 16, 0, B=3, H=1, G=2, HD=64, n_pos=130, seq_lens=[65, 5000, 129], seed=6)


def test_pieces_equal_one_call(oq):
    c1, o1 = run_case(oq, 4, 4, 0, B=2, H=2, G=2, HD=128, n_pos=500, pieces=(1.0,), seed=9)
    c2, o2 = run_case(oq, 4, 4, 0, B=2, H=2, G=2, HD=128, n_pos=500, pieces=(0.3, 0.002, 0.5, 1.0), seed=9)
    assert np.array_equal(o1, o2)
    assert np.array_equal(c1.k_codes.cpu().numpy(), c2.k_codes.cpu().numpy())


@pytest.mark.parametrize("n_pos", [5, 11, 12, 13, 40, 101])
def test_window_edges(oq, n_pos):
    """Anchors 3 + window 9 (capacity 12): before filling, exactly full, one
    past, and many wraps, with single-row and multi-row appends."""
    run_case(oq, 4, 4, 0, B=2, H=1, G=4, HD=64, n_pos=n_pos, n_anchor=3, window=9, seed=n_pos)
    run_case(oq, 8, 8, 0, B=1, H=1, G=1, HD=64, n_pos=n_pos, n_anchor=3, window=9, seed=n_pos,
             pieces=tuple([1.0 / n_pos] * (n_pos - 1) + [1.0]))


def test_window_page_shape(oq):
    """64 anchors + 1536 recent (on-device page), 5000 positions in mixed calls."""
    run_case(oq, 4, 4, 0, B=2, H=2, G=4, HD=128, n_pos=5000, n_anchor=64, window=1536,
             pieces=(0.01, 0.4, 0.0002, 1.0), seed=21)


def test_determinism(oq):
    _, a = run_case(oq, 4, 4, 0, B=2, H=2, G=4, HD=128, n_pos=2000, seed=13)
    _, b = run_case(oq, 4, 4, 0, B=2, H=2, G=4, HD=128, n_pos=2000, seed=13)
    assert np.array_equal(a, b)


def test_special_rows(oq):
    """All-zero rows, tiny rows (subnormal or zero scale), huge rows (scale
    saturation), exact ties."""
    kvq = need_gpu()
    import torch
    from workloads.device import decode, positions, to_device
    B, H, HD, n = 1, 2, 64, 8
    K = np.random.default_rng(1).standard_normal((B, H, n, HD)).astype(np.float32)
    K[0, 0, 0] = 0.0
    K[0, 0, 1] *= np.float32(1e-6)
    K[0, 0, 2] *= np.float32(1e-4)
    K[0, 0, 3] *= np.float32(1e6)
    s = np.float32(0.142822265625)            # fp16 scale of amax 1, qmax 7
    K[0, 1, 4] = 0.0
    K[0, 1, 4, 0] = 1.0
    K[0, 1, 4, 1:4] = [s / 2, 1.5 * s, 2.5 * s]
    V = K.copy()
    for kb, vb in [(8, 8), (4, 4), (16, 16)]:
        cache = kvq.alloc_cache(B, H, HD, n, kb, vb, HD)
        kvq.kvq_append(cache, to_device(K), to_device(V), n, positions([0]))
        torch.cuda.synchronize()
        check_codes(oq, cache, K, V, linear_slots(n, n))


def test_append_skips_out_of_range(oq):
    """Rows at negative positions or at/after capacity are not stored."""
    kvq = need_gpu()
    import torch
    from workloads.device import positions, to_device
    B, H, HD, cap = 2, 1, 64, 10
    cache = kvq.alloc_cache(B, H, HD, cap, 8, 8, HD)
    cache.k_codes.fill_(0x5A)
    x = np.ones((B, H, 4, HD), np.float32)
    kvq.kvq_append(cache, to_device(x), to_device(x), 4, positions([-2, 8]))
    torch.cuda.synchronize()
    kc = cache_arrays(cache)[0]
    assert np.all(kc[0, 0, :2] == 127) and np.all(kc[0, 0, 2:] == 0x5A)
    assert np.all(kc[1, 0, 8:] == 127) and np.all(kc[1, 0, :8] == 0x5A)


@pytest.mark.parametrize("kb,vb", [(4, 4), (8, 4), (8, 8), (4, 8)])
@pytest.mark.parametrize("HD,group", [(128, 0), (128, 32), (64, 0), (64, 32)])
def test_bulk_append_matches_rows(oq, kb, vb, HD, group):
    """A bulk append (the 64-slot tile kernel) stores bit for bit what one
    append per row (the row kernel) stores, for tiles cut by unaligned and
    negative starts and by the capacity, contiguous and paged."""
    kvq = need_gpu()
    import torch
    from gpu_util import assert_same_storage, paged_table
    from workloads.device import positions, to_device
    B, H, cap, n = 4, 2, 512, 300
    gs = group or HD
    starts = [37, 0, -5, cap - 200]                  # the last runs 100 rows past the capacity
    rng = np.random.default_rng(kb * 7 + vb + HD + gs)
    K = (rng.standard_normal((B, H, n, HD)) * rng.uniform(0.1, 4.0, (B, H, n, 1))).astype(np.float32)
    V = rng.standard_normal((B, H, n, HD)).astype(np.float32)
    bulk = kvq.alloc_cache(B, H, HD, cap, kb, vb, gs)
    rows = kvq.alloc_cache(B, H, HD, cap, kb, vb, gs)
    P, pps = 64, cap // 64
    table = paged_table(B, pps, B * pps + 2, kb + vb)
    paged = kvq.alloc_cache(B, H, HD, cap, kb, vb, gs, page_size=P, n_pages=B * pps + 2,
                            block_table=to_device(table))
    kd, vd = to_device(K), to_device(V)
    for c in (bulk, paged):
        kvq.kvq_append(c, kd, vd, n, positions(starts))
    for i in range(n):
        kvq.kvq_append(rows, kd[:, :, i:i + 1].contiguous(), vd[:, :, i:i + 1].contiguous(), 1,
                       positions([s0 + i for s0 in starts]))
    torch.cuda.synchronize()
    for name in ("k_codes", "v_codes", "k_scales", "v_scales"):
        assert torch.equal(getattr(bulk, name), getattr(rows, name)), name
    assert_same_storage(paged, table, rows)
    # and the stored rows are the oracle's codes
    for b, s0 in enumerate(starts):
        slots = {s0 + i: s0 + i for i in range(n) if 0 <= s0 + i < cap}
        Kp = np.zeros((1, H, cap, HD), np.float32)
        Vp = np.zeros((1, H, cap, HD), np.float32)
        for sl in slots:
            Kp[0, :, sl], Vp[0, :, sl] = K[b, :, sl - s0], V[b, :, sl - s0]
        check_codes(oq, bulk.sequence(b), Kp, Vp, slots)


@pytest.mark.parametrize("kb,vb", [(4, 4), (8, 8)])
def test_codes_near_half_integers(oq, kb, vb):
    """Values whose quotient by the scale lies within a few ulps of k + 1/2
    (the rounding boundary), for normal and subnormal fp16 scales and a
    scale rounded down from 1.45 * 2^-24: both append kernels store the
    oracle's codes, decided by the IEEE quotient."""
    kvq = need_gpu()
    import torch
    from workloads.device import positions, to_device
    B, H, HD, n, g = 2, 2, 128, 128, 32
    qmax = 127 if kb == 8 else 7
    rng = np.random.default_rng(91 + kb)
    f16 = lambda v: np.float32(np.float16(v))
    scales = [f16(1.0), f16(0.0371), f16(3.3e-3), f16(7.1e-5), np.float32(3 * 2.0 ** -24),
              np.float32(2.0 ** -24), f16(250.0)]
    X = np.zeros((B, H, n, HD), np.float32)
    for idx in np.ndindex(B, H, n, HD // g):
        S = scales[rng.integers(len(scales))]
        grp = np.empty(g, np.float32)
        grp[0] = np.float32(qmax) * S                   # amax / qmax = S exactly
        if S == np.float32(2.0 ** -24) and rng.random() < 0.5:
            grp[0] = np.float32(1.45 * 2.0 ** -24) * np.float32(qmax)   # scale rounds down to 2^-24
        k = rng.integers(-qmax, qmax, g - 1)
        # half of them just outside the window where the exact divide decides
        off = np.where(rng.random(g - 1) < 0.5, 0.0, rng.uniform(0.8e-4, 3e-4, g - 1) * rng.choice([-1, 1], g - 1))
        x = ((k + 0.5 + off) * np.float64(S)).astype(np.float32)
        for _ in range(3):                              # nudge by -3 .. 3 ulps
            step = rng.integers(-1, 2, g - 1)
            x = np.where(step > 0, np.nextafter(x, np.float32(np.inf)),
                         np.where(step < 0, np.nextafter(x, np.float32(-np.inf)), x)).astype(np.float32)
        grp[1:] = np.clip(x, -grp[0], grp[0])
        rng.shuffle(grp)
        b, h, t, j = idx
        X[b, h, t, j * g:(j + 1) * g] = grp
    bulk = kvq.alloc_cache(B, H, HD, n, kb, vb, g)
    rows = kvq.alloc_cache(B, H, HD, n, kb, vb, g)
    xd = to_device(X)
    kvq.kvq_append(bulk, xd, xd, n, positions([0, 0]))
    for p0 in range(0, n, 16):
        part = to_device(X[:, :, p0:p0 + 16])
        kvq.kvq_append(rows, part, part, 16, positions([p0, p0]))
    torch.cuda.synchronize()
    slots = {t: t for t in range(n)}
    check_codes(oq, bulk, X, X, slots)
    check_codes(oq, rows, X, X, slots)


def test_guard_bands_untouched(oq):
    """Buffers placed between guard bytes: append and decode write only
    their own ranges."""
    kvq = need_gpu()
    import torch
    from workloads.device import positions, to_device
    B, H, HD, cap, G = 2, 2, 128, 300, 4
    d0 = kvq.alloc_cache(B, H, HD, cap, 4, 4, HD)
    sizes = kvq.kvq_cache_sizes(d0)
    guard = 4096
    big = [torch.full((s + 2 * guard,), 0xA5, dtype=torch.uint8, device="cuda") for s in sizes]
    d = kvq.kvq_cache.from_buffer_copy(d0.desc)
    d.k_codes, d.v_codes, d.k_scales, d.v_scales = (t.data_ptr() + guard for t in big)
    K, V, q = _data(B, H, cap, HD, H * G, 4)
    kvq.kvq_append(d, to_device(K), to_device(V), cap, positions([0, 0]))
    ws_bytes = kvq.kvq_workspace_bytes(d, H * G, cap, 256)
    ws = torch.full((ws_bytes + 2 * guard,), 0xA5, dtype=torch.uint8, device="cuda")
    out = torch.full((B * H * G * HD + 2 * 64,), 7.0, device="cuda")
    kvq.kvq_decode_attn(d, to_device(q), H * G, positions([cap, cap]), cap, 0.0, 256, out.data_ptr() + 256,
                        ws.data_ptr() + guard, ws_bytes)
    torch.cuda.synchronize()
    for t in big + [ws]:
        a = t.cpu().numpy()
        assert np.all(a[:guard] == 0xA5) and np.all(a[-guard:] == 0xA5)
    o = out.cpu().numpy()
    assert np.all(o[:64] == 7.0) and np.all(o[-64:] == 7.0)


def test_combine_matches_single_chunk(oq):
    """Split-K partials merged by kvq_combine equal a one-chunk run."""
    _, a = run_case(oq, 8, 8, 0, B=1, H=1, G=2, HD=128, n_pos=4000, chunk=256, seed=17)
    _, b = run_case(oq, 8, 8, 0, B=1, H=1, G=2, HD=128, n_pos=4000, chunk=2048, seed=17)
    np.testing.assert_allclose(a, b, rtol=0, atol=2e-4)


def _fp16_patterns(kvq, u):
    """Store float32 bit patterns `u` (uint32 numpy) through the FP16 cache
    mode and compare with numpy's nearest-even cast (any NaN == any NaN)."""
    import torch
    from workloads.device import positions
    HD = 128
    n = u.size // HD * HD
    u = u[:n]
    cache = kvq.alloc_cache(1, 1, HD, n // HD, 16, 16, HD)
    x = torch.from_numpy(u.view(np.int32)).cuda().view(torch.float32)
    kvq.kvq_append(cache, x, x, n // HD, positions([0]))
    got = cache.k_codes.view(torch.int16).cpu().numpy().view(np.uint16)
    with np.errstate(over="ignore", invalid="ignore"):
        ref = u.view(np.float32).astype(np.float16).view(np.uint16)
    ref_nan = ((ref & 0x7C00) == 0x7C00) & ((ref & 0x3FF) != 0)
    got_nan = ((got & 0x7C00) == 0x7C00) & ((got & 0x3FF) != 0)
    assert np.array_equal(ref_nan, got_nan)
    bad = np.flatnonzero(got[~ref_nan] != ref[~ref_nan])
    assert bad.size == 0, (u[~ref_nan][bad[:4]], got[~ref_nan][bad[:4]], ref[~ref_nan][bad[:4]])


def test_fp16_conversion_rounding_neighbourhoods():
    """The FP16 cache mode rounds like IEEE binary16 nearest-even: every
    sign x exponent x top-10-fraction-bit pattern with the dropped bits at
    and around the ties, all results in the subnormal range, and a strided
    sweep of all 2^32 patterns."""
    kvq = need_gpu()
    low = np.array([0, 1, 2, 0x0FFE, 0x0FFF, 0x1000, 0x1001, 0x1002, 0x1FFE, 0x1FFF], np.uint32)
    top = np.arange(1 << 19, dtype=np.uint32) << np.uint32(13)
    _fp16_patterns(kvq, (top[:, None] | low[None, :]).ravel())
    e = np.arange(102, 114, dtype=np.uint32)
    m = np.arange(1 << 23, dtype=np.uint32)[::3]
    sub = ((e[:, None] << np.uint32(23)) | m[None, :]).ravel()
    _fp16_patterns(kvq, np.concatenate([sub, sub | np.uint32(0x80000000)]))
    _fp16_patterns(kvq, np.arange(0, 1 << 32, 4099, dtype=np.uint64).astype(np.uint32))


@pytest.mark.skipif(not __import__("os").environ.get("KVQ_EXHAUSTIVE_FP16"), reason="set KVQ_EXHAUSTIVE_FP16=1")
def test_fp16_conversion_exhaustive():
    """All 2^32 float32 patterns through the FP16 cache mode."""
    kvq = need_gpu()
    step = 1 << 25
    for hi in range(0, 1 << 32, step):
        _fp16_patterns(kvq, np.arange(hi, hi + step, dtype=np.uint64).astype(np.uint32))


@pytest.mark.parametrize("kb,vb,group", MODES)
@pytest.mark.parametrize("n_new", [0, 1, 3])
def test_decode_step_matches_separate_calls(oq, kb, vb, group, n_new):
    """kvq_decode_step leaves the cache and the output bit for bit as
    kvq_append followed by kvq_decode_attn does, and matches the oracle."""
    kvq = need_gpu()
    import torch
    from workloads.device import positions, to_device
    B, H, G, HD, n0 = 2, 2, 4, 128, 650
    n = n0 + n_new
    gs = group_size_of(kb, vb, group, H, HD)
    K, V, q = _data(B, H, n, HD, H * G, 31 + n_new)
    caches = [kvq.alloc_cache(B, H, HD, n, kb, vb, gs) for _ in range(2)]
    for c in caches:
        kvq.kvq_append(c, to_device(K[:, :, :n0]), to_device(V[:, :, :n0]), n0, positions([0] * B))
    kn, vn, qd = to_device(K[:, :, n0:]), to_device(V[:, :, n0:]), to_device(q)
    pos, lens = positions([n0] * B), positions([n] * B)
    ws_bytes = kvq.kvq_workspace_bytes(caches[0], H * G, n, 0)
    outs = [torch.full((B, H * G, HD), 7.0, dtype=torch.float32, device="cuda") for _ in range(2)]
    wss = [torch.empty(ws_bytes // 4 + 64, dtype=torch.float32, device="cuda") for _ in range(2)]
    wss[0].zero_()                                   # kvq_decode_step takes a zero-filled workspace
    kvq.kvq_decode_step(caches[0], kn, vn, n_new, pos, qd, H * G, lens, n, 0.0, 0, outs[0], wss[0], ws_bytes)
    kvq.kvq_append(caches[1], kn, vn, n_new, pos)
    kvq.kvq_decode_attn(caches[1], qd, H * G, lens, n, 0.0, 0, outs[1], wss[1], ws_bytes)
    torch.cuda.synchronize()
    assert torch.equal(outs[0], outs[1])
    for name in ("k_codes", "v_codes", "k_scales", "v_scales"):
        a, b = getattr(caches[0], name), getattr(caches[1], name)
        if a is not None:
            assert torch.equal(a, b), name
    got = outs[0].cpu().numpy()
    sc = softmax_default(HD)
    for b in range(B):
        want = oq.decode_step(kb, vb, gs, 0, 0, K[b], V[b], q[b], sc)
        assert_close(got[b], want, f"step kb={kb} vb={vb} n_new={n_new} b={b}")


@pytest.mark.parametrize("kb,vb", [(4, 4), (8, 4)])
@pytest.mark.parametrize("n", [1023, 1024, 1025, 2100])
def test_decode_step_merge_rule(oq, kb, vb, n):
    """Contexts of 4 chunks (merged inside the split kernel), 5 and 9 chunks
    (merged by the combine launch), with one row appended by the step: both
    forms equal the separate calls bit for bit."""
    kvq = need_gpu()
    import torch
    from workloads.device import positions, to_device
    B, H, G, HD, ch = 2, 2, 4, 128, 256
    n0 = n - 1
    K, V, q = _data(B, H, n, HD, H * G, 80 + n)
    caches = [kvq.alloc_cache(B, H, HD, n, kb, vb, HD) for _ in range(2)]
    for c in caches:
        kvq.kvq_append(c, to_device(K[:, :, :n0]), to_device(V[:, :, :n0]), n0, positions([0] * B))
    kn, vn, qd = to_device(K[:, :, n0:]), to_device(V[:, :, n0:]), to_device(q)
    pos, lens = positions([n0] * B), positions([n, n - 300])
    ws_bytes = kvq.kvq_workspace_bytes(caches[0], H * G, n, ch)
    outs = [torch.full((B, H * G, HD), 7.0, dtype=torch.float32, device="cuda") for _ in range(2)]
    # the step's workspace zero-filled (its ticket counters), the separate calls' any
    wss = [torch.full((ws_bytes // 4 + 64,), v, dtype=torch.float32, device="cuda") for v in (0.0, 3.0)]
    for _ in range(2):                                  # the second step reuses the workspace's counters
        kvq.kvq_decode_step(caches[0], kn, vn, 1, pos, qd, H * G, lens, n, 0.0, ch, outs[0], wss[0], ws_bytes)
    kvq.kvq_append(caches[1], kn, vn, 1, pos)
    kvq.kvq_decode_attn(caches[1], qd, H * G, lens, n, 0.0, ch, outs[1], wss[1], ws_bytes)
    torch.cuda.synchronize()
    assert torch.equal(outs[0], outs[1])
    got = outs[0].cpu().numpy()
    for b, L in ((0, n), (1, n - 300)):
        want = oq.decode_step(kb, vb, HD, 0, 0, K[b][:, :L], V[b][:, :L], q[b], softmax_default(HD))
        assert_close(got[b], want, f"merge rule n={n} b={b}")


@pytest.mark.parametrize("fused", [False, True])
def test_graph_replay_matches_eager(oq, fused):
    """A step captured in a HIP graph (append + decode + combine, as separate
    calls or as one kvq_decode_step) gives the eager result bit for bit on
    every replay, with eager work in between."""
    kvq = need_gpu()
    import torch
    from workloads.device import positions, to_device
    B, H, G, HD, n = 2, 2, 4, 128, 700
    cache = kvq.alloc_cache(B, H, HD, n, 4, 4, HD)
    K, V, q = _data(B, H, n, HD, H * G, 21)
    kvq.kvq_append(cache, to_device(K[:, :, : n - 1]), to_device(V[:, :, : n - 1]), n - 1, positions([0, 0]))
    k1, v1, qd = to_device(K[:, :, n - 1:]), to_device(V[:, :, n - 1:]), to_device(q)
    pos, lens = positions([n - 1] * B), positions([n] * B)
    ws_bytes = kvq.kvq_workspace_bytes(cache, H * G, n, 0)
    ws = torch.zeros(ws_bytes // 4 + 64, dtype=torch.float32, device="cuda")   # zero-filled for kvq_decode_step
    out = torch.zeros((B, H * G, HD), dtype=torch.float32, device="cuda")

    def step(st):
        if fused:
            kvq.kvq_decode_step(cache, k1, v1, 1, pos, qd, H * G, lens, n, 0.0, 0, out, ws, ws_bytes, st)
        else:
            kvq.kvq_append(cache, k1, v1, 1, pos, st)
            kvq.kvq_decode_attn(cache, qd, H * G, lens, n, 0.0, 0, out, ws, ws_bytes, st)

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
        # eager work between replays (the step's workspace comes back
        # zero-filled, as kvq_decode_step takes it; the separate calls' any)
        ws.fill_(0.0 if fused else float(r + 1))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, want), f"replay {r}"


def test_layers_of_mixed_widths_in_one_graph(oq):
    """Bit widths chosen per layer (KVSplit's per-layer roadmap): four layers
    with K8V8, K4V4 in 32-value groups, K8V4 and FP16 caches, one decode step
    each, captured together in one HIP graph sharing one workspace; every
    replay gives each layer's eager output bit for bit, and each matches the
    oracle."""
    kvq = need_gpu()
    import torch
    from workloads.device import positions, to_device
    B, H, G, HD, n = 2, 2, 4, 128, 600
    modes = [(8, 8, HD), (4, 4, 32), (8, 4, HD), (16, 16, HD)]
    layers = []
    for li, (kb, vb, gs) in enumerate(modes):
        K, V, q = _data(B, H, n, HD, H * G, 40 + li)
        cache = kvq.alloc_cache(B, H, HD, n, kb, vb, gs)
        kvq.kvq_append(cache, to_device(K[:, :, : n - 1]), to_device(V[:, :, : n - 1]), n - 1, positions([0, 0]))
        out = torch.zeros((B, H * G, HD), dtype=torch.float32, device="cuda")
        layers.append((cache, to_device(K[:, :, n - 1:]), to_device(V[:, :, n - 1:]), to_device(q), out, K, V, q))
    pos, lens = positions([n - 1] * B), positions([n] * B)
    ws_bytes = max(kvq.kvq_workspace_bytes(c, H * G, n, 0) for c, *_ in layers)
    ws = torch.zeros(ws_bytes // 4 + 64, dtype=torch.float32, device="cuda")   # zero-filled for kvq_decode_step

    def step(st):
        for cache, k1, v1, qd, out, *_ in layers:
            kvq.kvq_decode_step(cache, k1, v1, 1, pos, qd, H * G, lens, n, 0.0, 0, out, ws, ws_bytes, st)

    step(torch.cuda.current_stream())
    torch.cuda.synchronize()
    want = [l[4].clone() for l in layers]
    for (kb, vb, gs), (_, _, _, _, _, K, V, q), w in zip(modes, layers, want):
        got = w.cpu().numpy()
        for b in range(B):
            ref = oq.decode_step(kb, vb, gs, 0, 0, K[b], V[b], q[b], softmax_default(HD))
            assert_close(got[b], ref, f"layer kb={kb} vb={vb} g={gs} b={b}")
    # more steps on the same workspace, never cleared again: the FP16 layer's
    # partials (the largest need, so they reach the end of the data) leave
    # the integer layers' ticket counters alone, and every step leaves them
    # zero
    for r in range(2):
        for l in layers:
            l[4].zero_()
        step(torch.cuda.current_stream())
        torch.cuda.synchronize()
        for li, l in enumerate(layers):
            assert torch.equal(l[4], want[li]), f"eager step {r + 2} layer {li}"
    g = torch.cuda.CUDAGraph()
    cs = torch.cuda.Stream()
    cs.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(cs):
        step(cs)
    torch.cuda.synchronize()
    with torch.cuda.graph(g, stream=cs):
        step(cs)
    for r in range(3):
        for l in layers:
            l[4].zero_()                             # eager work between replays (the workspace is not cleared)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for li, l in enumerate(layers):
            assert torch.equal(l[4], want[li]), f"replay {r} layer {li}"


def test_read_probe_runs():
    """The read-bandwidth probe reads every block it is given (an all-zero
    buffer folds to zero in every workgroup) and rejects bad sizes."""
    kvq = need_gpu()
    import torch
    buf = torch.zeros(1 << 20, dtype=torch.uint8, device="cuda")
    sink = torch.full((64,), -1, dtype=torch.int32, device="cuda")
    kvq.kvq_read_probe(buf, buf.numel(), sink, sink.numel() * 4)
    torch.cuda.synchronize()
    assert torch.all(sink == 0)
    with pytest.raises(kvq.KvqError):
        kvq.kvq_read_probe(buf, 1000, sink, sink.numel() * 4)


@pytest.mark.parametrize("kb,vb", [(4, 4), (8, 4), (8, 8), (4, 8)])
def test_prepared_halves_match_partials(oq, kb, vb):
    """kvq_prepare_query + kvq_decode_partials_prepared (run twice on one
    preparation) write the same partials, bit for bit, as
    kvq_decode_partials."""
    kvq = need_gpu()
    import torch
    from workloads.device import positions, to_device
    B, H, G, HD, n = 2, 2, 4, 128, 900
    cache = kvq.alloc_cache(B, H, HD, n, kb, vb, HD)
    K, V, q = _data(B, H, n, HD, H * G, 41)
    kvq.kvq_append(cache, to_device(K), to_device(V), n, positions([0] * B))
    qd, lens = to_device(q), positions([n, n - 301])
    ws_bytes = kvq.kvq_workspace_bytes(cache, H * G, n, 0)
    ws = [torch.full((ws_bytes // 4 + 64,), 3.0, dtype=torch.float32, device="cuda") for _ in range(2)]
    kvq.kvq_decode_partials(cache, qd, H * G, lens, n, 0.0, 0, ws[0], ws_bytes)
    kvq.kvq_prepare_query(cache, qd, H * G, n, 0.0, 0, ws[1], ws_bytes)
    for _ in range(2):
        kvq.kvq_decode_partials_prepared(cache, H * G, lens, n, 0, ws[1], ws_bytes)
    torch.cuda.synchronize()
    # (raw words: the workspace also holds the query's integer digits)
    assert torch.equal(ws[0].view(torch.int32), ws[1].view(torch.int32))
