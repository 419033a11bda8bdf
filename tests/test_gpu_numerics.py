"""GPU parity on inputs that stress the integer path's fixed-point arithmetic,
beyond N(0, 1) rows and the default softmax scale.

The integer split kernel holds the query as 16-bit fixed point (plus one
extra low digit when a channel stands out) and each sub-chunk's value
weights p * s_v as 16-bit fixed point relative to the sub-chunk's largest
one.  These cases are the method's own edge cases: explicit softmax scales
and a scaled-up query (peaked softmax); an anchor row that carries most of
the attention mass while its values are small (the on-device page keeps the
first 64 tokens as anchors for this, and notes that values need more
precision than keys); rows of near-zero weight whose value scale is far
larger than the rest; a query with one large channel.  Each is compared with
the oracle at the path's tolerance for the four integer width pairs, per-head
and 32-value scale groups, at a few hundred positions and at 32K."""
import numpy as np
import pytest

from gpu_util import assert_close, check_codes, linear_slots, need_gpu, window_slots

pytestmark = pytest.mark.gpu

PAIRS = [(8, 8), (8, 4), (4, 4), (4, 8)]
GROUPS = [0, 32]            # 0: one scale per head (group = head_dim)


def _base(B, H, G, n_pos, HD, seed):
    rng = np.random.default_rng(seed)
    K = rng.standard_normal((B, H, n_pos, HD)).astype(np.float32)
    V = rng.standard_normal((B, H, n_pos, HD)).astype(np.float32)
    q = rng.standard_normal((B, H * G, HD)).astype(np.float32)
    return K, V, q


def _dir(q, G, kvh):
    """Unit direction shared by the G query heads of KV head kvh (the mean of
    their unit vectors), and each head's component along it."""
    qs = q[kvh * G:(kvh + 1) * G].astype(np.float64)
    u = (qs / np.linalg.norm(qs, axis=1, keepdims=True)).sum(0)
    u /= np.linalg.norm(u)
    return u, qs @ u


def _mass(q, K, sigma, t, G, kvh):
    """Softmax mass of position t for each of the G heads (float64, raw rows)."""
    z = sigma * (K[kvh].astype(np.float64) @ q[kvh * G:(kvh + 1) * G].T.astype(np.float64))
    z -= z.max(0)
    p = np.exp(z)
    return p[t] / p.sum(0)


def _make_sink(K, V, q, G, sigma, t_sink, v_factor, target=0.92):
    """Give position t_sink of every (sequence, KV head) a key along the
    heads' common direction, long enough that each head puts at least
    `target` of its mass on it, and shrink its value row by v_factor."""
    B, H = K.shape[:2]
    for b in range(B):
        for kvh in range(H):
            u, comp = _dir(q[b], G, kvh)
            assert np.all(comp > 0)
            lo, hi = 0.0, 400.0
            for _ in range(60):
                a = 0.5 * (lo + hi)
                K[b, kvh, t_sink] = (a * u).astype(np.float32)
                if _mass(q[b], K[b], sigma, t_sink, G, kvh).min() < target:
                    lo = a
                else:
                    hi = a
            K[b, kvh, t_sink] = (hi * u).astype(np.float32)
            m = _mass(q[b], K[b], sigma, t_sink, G, kvh)
            assert m.min() >= 0.9, m
            V[b, kvh, t_sink] *= np.float32(v_factor)


def _make_faint(K, V, q, G, sigma, every, v_factor):
    """One row per `every` positions (at offset 7) whose key points away from
    the heads' common direction (logit about -4, a near-zero weight) and whose
    value row is v_factor times larger."""
    B, H, n = K.shape[:3]
    for b in range(B):
        for kvh in range(H):
            u, comp = _dir(q[b], G, kvh)
            beta = 4.0 / (sigma * comp.min())
            for t in range(7, n, every):
                K[b, kvh, t] = (-beta * u).astype(np.float32)
                V[b, kvh, t] *= np.float32(v_factor)


def _run(oq, kb, vb, group, K, V, q, sigma, n_anchor=0, window=0, chunk=0, fused=False, codes=True):
    """Append every row (the last one through the step when fused), decode,
    compare with the oracle; explicit softmax scale sigma."""
    kvq = need_gpu()
    import torch
    from workloads.device import positions, to_device
    B, H, n_pos, HD = K.shape
    Hq = q.shape[1]
    gs = group or HD
    cap = n_anchor + window if window else n_pos
    cache = kvq.alloc_cache(B, H, HD, cap, kb, vb, gs, n_anchor, window)
    n0 = n_pos - 1
    kvq.kvq_append(cache, to_device(K[:, :, :n0]), to_device(V[:, :, :n0]), n0, positions([0] * B))
    kn, vn, qd = to_device(K[:, :, n0:]), to_device(V[:, :, n0:]), to_device(q)
    pos, lens = positions([n0] * B), positions([n_pos] * B)
    ws_bytes = kvq.kvq_workspace_bytes(cache, Hq, n_pos, chunk)
    # (kvq_decode_step takes a zero-filled workspace)
    ws = (torch.zeros if fused else torch.empty)(ws_bytes // 4 + 64, dtype=torch.float32, device="cuda")
    out = torch.full((B, Hq, HD), 5.0, dtype=torch.float32, device="cuda")
    if fused:
        kvq.kvq_decode_step(cache, kn, vn, 1, pos, qd, Hq, lens, n_pos, sigma, chunk, out, ws, ws_bytes)
    else:
        kvq.kvq_append(cache, kn, vn, 1, pos)
        kvq.kvq_decode_attn(cache, qd, Hq, lens, n_pos, sigma, chunk, out, ws, ws_bytes)
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    if codes:
        slots = window_slots(oq, n_pos, n_anchor, window) if window else linear_slots(n_pos, cap)
        check_codes(oq, cache, K, V, slots)
    res = []
    for b in range(B):
        want = oq.decode_step(kb, vb, gs, n_anchor, window, K[b], V[b], q[b], sigma)
        res.append(assert_close(got[b], want, f"kb={kb} vb={vb} g={gs} b={b} sigma={sigma}"))
    return res


SMALL = dict(B=2, H=2, G=4, n_pos=600, HD=128)


@pytest.mark.parametrize("kb,vb", PAIRS)
@pytest.mark.parametrize("group", GROUPS)
@pytest.mark.parametrize("sigma", [0.02, 0.5, 1.0])
def test_explicit_softmax_scale(oq, kb, vb, group, sigma):
    """softmax_scale given by the caller (1.0 makes logits of spread ~11):
    through kvq_decode_attn with 2048-slot chunks (512-position sub-chunks)
    and through kvq_decode_step with the library's chunk."""
    c = SMALL
    K, V, q = _base(c["B"], c["H"], c["G"], c["n_pos"], c["HD"], 600 + kb + vb + group)
    _run(oq, kb, vb, group, K, V, q, sigma, chunk=2048)
    _run(oq, kb, vb, group, K, V, q, sigma, fused=True, codes=False)


@pytest.mark.parametrize("kb,vb", PAIRS)
@pytest.mark.parametrize("group", GROUPS)
def test_scaled_query(oq, kb, vb, group):
    """q x 8: a peaked softmax at the default scale."""
    c = SMALL
    K, V, q = _base(c["B"], c["H"], c["G"], c["n_pos"], c["HD"], 610 + kb + vb + group)
    _run(oq, kb, vb, group, K, V, q * np.float32(8.0), 1.0 / np.sqrt(c["HD"]), chunk=2048)


@pytest.mark.parametrize("kb,vb", PAIRS)
@pytest.mark.parametrize("group", GROUPS)
def test_sink_row_small_values(oq, kb, vb, group):
    """Position 0 carries >= 90 % of every head's mass, its values x 0.05."""
    c = SMALL
    sigma = 1.0 / np.sqrt(c["HD"])
    K, V, q = _base(c["B"], c["H"], c["G"], c["n_pos"], c["HD"], 620 + kb + vb + group)
    _make_sink(K, V, q, c["G"], sigma, 0, 0.05)
    _run(oq, kb, vb, group, K, V, q, sigma, chunk=2048)
    _run(oq, kb, vb, group, K, V, q, sigma, fused=True, codes=False)


@pytest.mark.parametrize("kb,vb", PAIRS)
@pytest.mark.parametrize("group", GROUPS)
def test_sink_among_window_anchors(oq, kb, vb, group):
    """The same anchor row at position 3 of a window cache (64 anchors + 512
    recent slots) after 1500 positions, so the ring has wrapped."""
    B, H, G, n, HD = 2, 2, 4, 1500, 128
    sigma = 1.0 / np.sqrt(HD)
    K, V, q = _base(B, H, G, n, HD, 630 + kb + vb + group)
    # mass computed over the attended positions only
    Ka = np.concatenate([K[:, :, :64], K[:, :, n - 512:]], axis=2)
    Va = np.concatenate([V[:, :, :64], V[:, :, n - 512:]], axis=2)
    _make_sink(Ka, Va, q, G, sigma, 3, 0.05)
    K[:, :, 3], V[:, :, 3] = Ka[:, :, 3], Va[:, :, 3]
    _run(oq, kb, vb, group, K, V, q, sigma, n_anchor=64, window=512)
    _run(oq, kb, vb, group, K, V, q, sigma, n_anchor=64, window=512, fused=True, codes=False)


@pytest.mark.parametrize("kb,vb", PAIRS)
@pytest.mark.parametrize("group", GROUPS)
@pytest.mark.parametrize("v_factor", [30.0, 1000.0])
def test_faint_rows_large_values(oq, kb, vb, group, v_factor):
    """One near-zero-weight row per 512 positions whose values are 30x or
    1000x the others'."""
    c = SMALL
    sigma = 1.0 / np.sqrt(c["HD"])
    K, V, q = _base(c["B"], c["H"], c["G"], c["n_pos"], c["HD"], 640 + kb + vb + group + int(v_factor))
    _make_faint(K, V, q, c["G"], sigma, 512, v_factor)
    _run(oq, kb, vb, group, K, V, q, sigma, chunk=2048)
    _run(oq, kb, vb, group, K, V, q, sigma, chunk=512)


@pytest.mark.parametrize("kb,vb", PAIRS)
@pytest.mark.parametrize("group", GROUPS + [64])
@pytest.mark.parametrize("factor", [4.0, 100.0])
def test_query_outlier_channel(oq, kb, vb, group, factor):
    """One query channel x 100 (the query takes its extra low digit) and
    x 4 (it does not)."""
    c = SMALL
    K, V, q = _base(c["B"], c["H"], c["G"], c["n_pos"], c["HD"], 650 + kb + vb + group + int(factor))
    q[:, :, 5] *= np.float32(factor)
    _run(oq, kb, vb, group, K, V, q, 1.0 / np.sqrt(c["HD"]), chunk=2048)
    _run(oq, kb, vb, group, K, V, q, 1.0 / np.sqrt(c["HD"]), fused=True, codes=False)


@pytest.mark.parametrize("kb,vb", PAIRS)
@pytest.mark.parametrize("group", GROUPS)
@pytest.mark.parametrize("factor", [4.0, 100.0])
def test_query_outlier_channel_eight_heads(oq, kb, vb, group, factor):
    """The same with eight query heads per KV head: with one scale per head
    they are one unit of eight (the extra digit a product of its own on the
    matrix cores), with 32-value groups two workgroup heads of four."""
    K, V, q = _base(2, 2, 8, 600, 128, 660 + kb + vb + group + int(factor))
    q[:, :, 5] *= np.float32(factor)
    _run(oq, kb, vb, group, K, V, q, 1.0 / np.sqrt(128), chunk=2048)
    _run(oq, kb, vb, group, K, V, q, 1.0 / np.sqrt(128), fused=True, codes=False)


LONG = dict(B=1, H=2, G=4, n_pos=32768, HD=128)


@pytest.mark.parametrize("kb,vb", PAIRS)
@pytest.mark.parametrize("group", GROUPS)
@pytest.mark.parametrize("case", ["sink", "faint30", "faint1000", "qx100", "scale1"])
def test_stress_32k(oq, kb, vb, group, case):
    """The stress cases at 32K positions, library chunk and 2048-slot chunks."""
    c = LONG
    sigma = 1.0 / np.sqrt(c["HD"])
    K, V, q = _base(c["B"], c["H"], c["G"], c["n_pos"], c["HD"], 700 + kb + vb + group + len(case))
    if case == "sink":
        _make_sink(K, V, q, c["G"], sigma, 0, 0.05)
    elif case.startswith("faint"):
        _make_faint(K, V, q, c["G"], sigma, 512, float(case[5:]))
    elif case == "qx100":
        q[:, :, 5] *= np.float32(100.0)
    elif case == "scale1":
        sigma = 1.0
    _run(oq, kb, vb, group, K, V, q, sigma, chunk=2048, codes=False)
    _run(oq, kb, vb, group, K, V, q, sigma, fused=True, codes=False)
