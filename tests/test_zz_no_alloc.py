"""kvq_decode_step_static (the decode step that allocates nothing: its
workspace is the library's static device array) against kvq_decode_step
with a caller-allocated workspace: the same output and cache bit for bit, on
two steps in a row through the static array, the second one smaller, and
within tolerance of the oracle."""
import numpy as np
import pytest

from gpu_util import assert_close, need_gpu, softmax_default

pytestmark = pytest.mark.gpu


def _step_pair(oq, kvq, kb, vb, B, H, G, HD, n, seed, chunk=0):
    import torch
    from workloads.device import positions, to_device
    rng = np.random.default_rng(seed)
    K = rng.standard_normal((B, H, n, HD)).astype(np.float32)
    V = rng.standard_normal((B, H, n, HD)).astype(np.float32)
    q = rng.standard_normal((B, H * G, HD)).astype(np.float32)
    n0 = n - 1
    caches = [kvq.alloc_cache(B, H, HD, n, kb, vb, HD) for _ in range(2)]
    for c in caches:
        kvq.kvq_append(c, to_device(K[:, :, :n0]), to_device(V[:, :, :n0]), n0, positions([0] * B))
    kn, vn, qd = to_device(K[:, :, n0:]), to_device(V[:, :, n0:]), to_device(q)
    pos, lens = positions([n0] * B), positions([n] * B)
    outs = [torch.full((B, H * G, HD), 7.0, dtype=torch.float32, device="cuda") for _ in range(2)]
    ws_bytes = kvq.kvq_workspace_bytes(caches[0], H * G, n, chunk)
    assert ws_bytes <= kvq.KVQ_STATIC_SCRATCH_BYTES
    ws = torch.zeros(ws_bytes // 4 + 64, dtype=torch.float32, device="cuda")   # zero-filled, as the step takes it
    kvq.kvq_decode_step(caches[0], kn, vn, 1, pos, qd, H * G, lens, n, 0.0, chunk, outs[0], ws, ws_bytes)
    kvq.kvq_decode_step_static(caches[1], kn, vn, 1, pos, qd, H * G, lens, n, 0.0, chunk, outs[1])
    torch.cuda.synchronize()
    assert torch.equal(outs[0], outs[1]), f"kb={kb} vb={vb} B={B} n={n}"
    for name in ("k_codes", "v_codes", "k_scales", "v_scales"):
        a, b = getattr(caches[0], name), getattr(caches[1], name)
        if a is not None:
            assert torch.equal(a, b), name
    got = outs[1].cpu().numpy()
    for b in range(B):
        want = oq.decode_step(kb, vb, HD, 0, 0, K[b], V[b], q[b], softmax_default(HD))
        assert_close(got[b], want, f"static step kb={kb} vb={vb} b={b}")


@pytest.mark.parametrize("kb,vb", [(4, 4), (8, 4), (16, 16)])
def test_static_step_matches_step(oq, kb, vb):
    """A large step (9 chunks: split + combine launches), then a smaller one
    (one chunk: the merge inside the split kernel) through the same array."""
    kvq = need_gpu()
    _step_pair(oq, kvq, kb, vb, B=3, H=2, G=4, HD=128, n=4500, seed=900 + kb + vb, chunk=512)
    _step_pair(oq, kvq, kb, vb, B=1, H=1, G=2, HD=64, n=301, seed=901 + kb + vb)

