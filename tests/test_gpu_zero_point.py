"""GPU parity of the zero-point (asymmetric) codec: the appended rows' codes,
fp16 scales and zero points bit for bit against the oracle's codec, and the
decode outputs within tolerance of the oracle's decode step with the same
codec, over every integer width pair, head_dim, GQA group and scale grouping,
with shifted (asymmetric) value ranges, windows, the one-launch and the
multi-launch decode step, and the fixed-point stress inputs."""
import numpy as np
import pytest

from gpu_util import assert_close, check_codes_zp, linear_slots, need_gpu, softmax_default, window_slots

pytestmark = pytest.mark.gpu

PAIRS = [(8, 8), (8, 4), (4, 4), (4, 8)]


def _data(B, H, n, HD, Hq, seed, shift=True):
    rng = np.random.default_rng(seed)
    K = rng.standard_normal((B, H, n, HD)).astype(np.float32)
    V = rng.standard_normal((B, H, n, HD)).astype(np.float32)
    if shift:
        # asymmetric ranges: the zero point matters
        K += np.float32(1.5) * rng.standard_normal((B, H, 1, HD)).astype(np.float32)
        V += np.float32(-0.8) + np.float32(0.5) * rng.standard_normal((B, H, n, 1)).astype(np.float32)
    q = rng.standard_normal((B, Hq, HD)).astype(np.float32)
    return K, V, q


def run_zp(oq, kb, vb, gs, B, H, G, HD, n, seed, n_anchor=0, window=0, chunk=0, fused=False, pieces=1,
           sigma=None, data=None, lens=None, codes=True):
    kvq = need_gpu()
    import torch
    from workloads.device import positions, to_device
    Hq = H * G
    K, V, q = data if data is not None else _data(B, H, n, HD, Hq, seed)
    cap = n_anchor + window if window else n
    cache = kvq.alloc_cache(B, H, HD, cap, kb, vb, gs, n_anchor, window, zero_point=1)
    n0 = n - 1
    cuts = np.linspace(0, n0, pieces + 1).astype(int)
    for a, b in zip(cuts[:-1], cuts[1:]):
        if b > a:
            kvq.kvq_append(cache, to_device(K[:, :, a:b]), to_device(V[:, :, a:b]), int(b - a), positions([int(a)] * B))
    kn, vn, qd = to_device(K[:, :, n0:]), to_device(V[:, :, n0:]), to_device(q)
    lens = lens or [n] * B
    pos, sl = positions([n0] * B), positions(lens)
    max_len = max(max(lens), 1)
    ws_bytes = kvq.kvq_workspace_bytes(cache, Hq, max_len, chunk)
    # (kvq_decode_step takes a zero-filled workspace; the separate calls any)
    ws = torch.full((ws_bytes // 4 + 64,), 0.0 if fused else 3.0, dtype=torch.float32, device="cuda")
    out = torch.full((B, Hq, HD), 5.0, dtype=torch.float32, device="cuda")
    sc = sigma or softmax_default(HD)
    if fused:
        kvq.kvq_decode_step(cache, kn, vn, 1, pos, qd, Hq, sl, max_len, sc, chunk, out, ws, ws_bytes)
    else:
        kvq.kvq_append(cache, kn, vn, 1, pos)
        kvq.kvq_decode_attn(cache, qd, Hq, sl, max_len, sc, chunk, out, ws, ws_bytes)
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    if codes:
        slots = window_slots(oq, n, n_anchor, window) if window else linear_slots(n, cap)
        check_codes_zp(oq, cache, K, V, slots)
    for b in range(B):
        L = n if window else min(lens[b], cap)
        if L == 0:
            assert np.all(got[b] == 0)
            continue
        want = oq.decode_step(kb, vb, gs, n_anchor, window, K[b][:, :L], V[b][:, :L], q[b], sc, asym=True)
        assert_close(got[b], want, f"zp kb={kb} vb={vb} g={gs} b={b}")
    return cache, got


@pytest.mark.parametrize("kb,vb", PAIRS)
@pytest.mark.parametrize("HD", [64, 128])
@pytest.mark.parametrize("G", [1, 4, 8])
@pytest.mark.parametrize("group", [0, 32])
def test_zero_point_every_instantiation(oq, kb, vb, HD, G, group):
    gs = group or HD
    run_zp(oq, kb, vb, gs, B=2, H=2, G=G, HD=HD, n=777, seed=kb * 7 + vb + HD + G + gs, chunk=512)


@pytest.mark.parametrize("kb,vb", PAIRS)
def test_zero_point_per_position_scale(oq, kb, vb):
    """One scale and zero point per position over all KV heads."""
    run_zp(oq, kb, vb, 4 * 64, B=2, H=4, G=1, HD=64, n=300, seed=21 + kb + vb)
    run_zp(oq, kb, vb, 2 * 128, B=2, H=2, G=4, HD=128, n=600, seed=22 + kb + vb, pieces=3)


@pytest.mark.parametrize("kb,vb", PAIRS)
@pytest.mark.parametrize("group", [0, 64])
def test_zero_point_128_group(oq, kb, vb, group):
    """head_dim 128 with 2 scale groups; 2048-slot chunks (512-position sub-chunks)."""
    run_zp(oq, kb, vb, group or 128, B=2, H=2, G=4, HD=128, n=2100, seed=31 + kb + vb + group, chunk=2048)


@pytest.mark.parametrize("kb,vb", [(4, 4), (8, 4)])
def test_zero_point_window(oq, kb, vb):
    run_zp(oq, kb, vb, 128, B=2, H=2, G=4, HD=128, n=1700, seed=41 + kb, n_anchor=64, window=512, pieces=4)


@pytest.mark.parametrize("kb,vb", PAIRS)
@pytest.mark.parametrize("n", [400, 3000])
def test_zero_point_decode_step(oq, kb, vb, n):
    """The one-launch step (400 positions) and the split + merge step (3000),
    against the separate calls bit for bit and the oracle."""
    kvq = need_gpu()
    import torch
    from workloads.device import positions, to_device
    B, H, G, HD = 2, 2, 4, 128
    K, V, q = _data(B, H, n, HD, H * G, 50 + n + kb + vb)
    caches = [kvq.alloc_cache(B, H, HD, n, kb, vb, HD, zero_point=1) for _ in range(2)]
    for c in caches:
        kvq.kvq_append(c, to_device(K[:, :, :n - 1]), to_device(V[:, :, :n - 1]), n - 1, positions([0] * B))
    kn, vn, qd = to_device(K[:, :, n - 1:]), to_device(V[:, :, n - 1:]), to_device(q)
    pos, sl = positions([n - 1] * B), positions([n, n - 77])
    ws_bytes = kvq.kvq_workspace_bytes(caches[0], H * G, n, 0)
    outs = [torch.full((B, H * G, HD), 7.0, device="cuda") for _ in range(2)]
    wss = [torch.full((ws_bytes // 4 + 64,), v, device="cuda") for v in (0.0, 3.0)]   # the step's zero-filled
    kvq.kvq_decode_step(caches[0], kn, vn, 1, pos, qd, H * G, sl, n, 0.0, 0, outs[0], wss[0], ws_bytes)
    kvq.kvq_append(caches[1], kn, vn, 1, pos)
    kvq.kvq_decode_attn(caches[1], qd, H * G, sl, n, 0.0, 0, outs[1], wss[1], ws_bytes)
    torch.cuda.synchronize()
    assert torch.equal(outs[0], outs[1])
    for name in ("k_codes", "v_codes", "k_scales", "v_scales"):
        assert torch.equal(getattr(caches[0], name), getattr(caches[1], name)), name
    got = outs[0].cpu().numpy()
    for b, L in ((0, n), (1, n - 77)):
        want = oq.decode_step(kb, vb, HD, 0, 0, K[b][:, :L], V[b][:, :L], q[b], softmax_default(HD), asym=True)
        assert_close(got[b], want, f"zp step kb={kb} vb={vb} b={b}")


@pytest.mark.parametrize("kb,vb", [(8, 8), (4, 4)])
@pytest.mark.parametrize("case", ["scale1", "qx100", "faint1000", "unshifted"])
def test_zero_point_stress(oq, kb, vb, case):
    """Peaked softmax, a query outlier channel (the extra low digit with the
    zero point's correction), near-zero-weight rows with values x 1000, and
    zero-mean data."""
    B, H, G, HD, n = 2, 2, 4, 128, 1500
    K, V, q = _data(B, H, n, HD, H * G, 60 + kb + vb + len(case), shift=case != "unshifted")
    sigma = None
    if case == "scale1":
        sigma = 1.0
    elif case == "qx100":
        q[:, :, 5] *= np.float32(100.0)
    elif case == "faint1000":
        from test_gpu_numerics import _make_faint
        _make_faint(K, V, q, G, softmax_default(HD), 512, 1000.0)
    run_zp(oq, kb, vb, 128, B=B, H=H, G=G, HD=HD, n=n, seed=0, chunk=2048, sigma=sigma, data=(K, V, q), codes=False)
    run_zp(oq, kb, vb, 32, B=B, H=H, G=G, HD=HD, n=n, seed=0, sigma=sigma, data=(K, V, q), fused=True, codes=False)


@pytest.mark.parametrize("kb,vb", PAIRS)
def test_zero_point_split_heads(oq, kb, vb):
    """Eight query heads per KV head with 32-value groups (two workgroup heads
    of four per cache head): the separate calls and the one-launch step."""
    run_zp(oq, kb, vb, 32, B=2, H=2, G=8, HD=128, n=900, seed=70 + kb + vb, chunk=512)
    run_zp(oq, kb, vb, 32, B=2, H=2, G=8, HD=128, n=900, seed=71 + kb + vb, chunk=512, fused=True, codes=False)
