"""Seeded random configurations on the GPU: widths, head_dim, GQA group,
scale groups, window with anchors, paged storage, chunk sizes, ragged
lengths, appends in pieces and the fused decode step, drawn together so that
combinations the targeted tests do not spell out are run too.  Each draw is
checked against the oracle (outputs within tolerance; stored codes bit for
bit where the cache is contiguous)."""
import os

import numpy as np
import pytest

from gpu_util import (assert_close, check_codes, check_codes_zp, linear_slots, need_gpu, paged_table, softmax_default,
                      window_slots)

pytestmark = pytest.mark.gpu

WIDTHS = [(32, 32), (16, 16), (8, 8), (8, 4), (4, 4), (4, 8)]


def draw(seed):
    rng = np.random.default_rng(5000 + seed)
    kb, vb = WIDTHS[rng.integers(len(WIDTHS))]
    HD = int(rng.choice([64, 128]))
    G = int(rng.choice([1, 2, 4, 8]))
    H = int(rng.integers(1, 4))
    B = int(rng.integers(1, 4))
    quant = kb < 16
    gs = HD
    if quant:
        gs = int(rng.choice([g for g in (32, 64, HD) if HD % g == 0]))
        if H > 1 and rng.random() < 0.2:
            gs = H * HD                              # one scale per position over all heads
    P = int(rng.choice([0, 64, 128, 256]))
    window = rng.random() < 0.3
    if window:
        cap = int(rng.integers(2, 9)) * (P or 64)
        A = int(rng.choice([0, 16, 48]))
        W = cap - A
        n_pos = int(rng.integers(1, 3 * cap))
    else:
        A = W = 0
        n_pos = int(rng.integers(1, 1600))
        cap = ((n_pos + (P or 1) - 1) // (P or 1)) * (P or 1) + int(rng.choice([0, P or 7]))
    zp = bool(quant and rng.random() < 0.25)          # the zero-point codec
    chunk = int(rng.choice([0, 256, 512, 1024]))
    if not quant and chunk:
        chunk = int(rng.choice([64, 128, 256]))
    n_pieces = int(rng.integers(1, 4))
    return dict(kb=kb, vb=vb, HD=HD, G=G, H=H, B=B, gs=gs, P=P, A=A, W=W, cap=cap, n_pos=n_pos, chunk=chunk,
                n_pieces=n_pieces, fused=bool(rng.random() < 0.5), zp=zp, rng=rng)


# KVQ_RANDOM_SEEDS sets the number of draws (1200 run in about 20 s)
@pytest.mark.parametrize("seed", range(int(os.environ.get("KVQ_RANDOM_SEEDS", "1200"))))
def test_random_configuration(oq, seed):
    kvq = need_gpu()
    import torch
    from workloads.device import positions, to_device
    c = draw(seed)
    kb, vb, HD, G, H, B, gs, P, A, W, cap, n_pos = (c[k] for k in
                                                    ("kb", "vb", "HD", "G", "H", "B", "gs", "P", "A", "W", "cap",
                                                     "n_pos"))
    rng = c["rng"]
    desc = f"seed {seed}: {dict((k, v) for k, v in c.items() if k != 'rng')}"
    print(desc, flush=True)
    Hq = H * G
    K = rng.standard_normal((B, H, n_pos, HD)).astype(np.float32)
    V = rng.standard_normal((B, H, n_pos, HD)).astype(np.float32)
    q = rng.standard_normal((B, Hq, HD)).astype(np.float32)
    if P:
        pps = cap // P
        table = paged_table(B, pps, B * pps + 3, seed)
        cache = kvq.alloc_cache(B, H, HD, cap, kb, vb, gs, A, W, page_size=P, n_pages=B * pps + 3,
                                block_table=to_device(table), zero_point=int(c["zp"]))
    else:
        cache = kvq.alloc_cache(B, H, HD, cap, kb, vb, gs, A, W, zero_point=int(c["zp"]))
    # the context before the step's row, appended in pieces
    n0 = n_pos - 1
    cuts = sorted(set([0, n0] + [int(x) for x in rng.integers(0, n0 + 1, c["n_pieces"] - 1)]))
    for a, b in zip(cuts[:-1], cuts[1:]):
        if b > a:
            kvq.kvq_append(cache, to_device(K[:, :, a:b]), to_device(V[:, :, a:b]), b - a, positions([a] * B))
    lens = [n_pos] * B
    if not W and B > 1:
        lens[-1] = int(rng.integers(0, n_pos + 1))   # a sequence attending a prefix (or nothing)
    max_len = max(max(lens), 1)
    ws_bytes = kvq.kvq_workspace_bytes(cache, Hq, max_len, c["chunk"])
    # (kvq_decode_step takes a zero-filled workspace)
    ws = (torch.zeros if c["fused"] else torch.empty)(ws_bytes // 4 + 64, dtype=torch.float32, device="cuda")
    out = torch.full((B, Hq, HD), 5.0, dtype=torch.float32, device="cuda")
    kn, vn, qd = to_device(K[:, :, n0:]), to_device(V[:, :, n0:]), to_device(q)
    pos, sl = positions([n0] * B), positions(lens)
    if c["fused"]:
        kvq.kvq_decode_step(cache, kn, vn, 1, pos, qd, Hq, sl, max_len, 0.0, c["chunk"], out, ws, ws_bytes)
    else:
        kvq.kvq_append(cache, kn, vn, 1, pos)
        kvq.kvq_decode_attn(cache, qd, Hq, sl, max_len, 0.0, c["chunk"], out, ws, ws_bytes)
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    if not P:
        slots = window_slots(oq, n_pos, A, W) if W else linear_slots(n_pos, cap)
        (check_codes_zp if c["zp"] else check_codes)(oq, cache, K, V, slots)
    for b in range(B):
        L = n_pos if W else min(lens[b], cap)
        if L == 0:
            assert np.all(got[b] == 0), desc
            continue
        want = oq.decode_step(kb, vb, gs, A, W, K[b][:, :L], V[b][:, :L], q[b], softmax_default(HD), asym=c["zp"])
        assert_close(got[b], want, f"{desc} b={b} L={L}")
