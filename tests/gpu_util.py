"""Shared helpers of the GPU tests: run the HIP path through the C ABI and
compare it with the CPU oracle."""
from __future__ import annotations

import math

import numpy as np
import pytest

ATOL = 2e-3      # max |gpu - oracle| on attention outputs
RTOL_L2 = 1e-3   # ||gpu - oracle||_2 / ||oracle||_2


def need_gpu():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import decode_attention_quantized_kvq_amd as kvq
    kvq.lib()                       # raises if libkvq.so is missing: no fallback
    return kvq


def assert_close(got, want, ctx=""):
    got = np.asarray(got, np.float64)
    want = np.asarray(want, np.float64)
    assert got.shape == want.shape, (got.shape, want.shape)
    assert np.all(np.isfinite(got)), f"{ctx}: non-finite output"
    d = np.abs(got - want)
    nrm = np.linalg.norm(want)
    rel = np.linalg.norm(got - want) / nrm if nrm > 0 else np.linalg.norm(got - want)
    assert d.max() <= ATOL and rel <= RTOL_L2, f"{ctx}: max|d|={d.max():.3e} relL2={rel:.3e}"
    return float(d.max()), float(rel)


def group_size_of(kb, vb, group, hkv, hd):
    if kb >= 16:
        return hd
    if group == -1:
        return hkv * hd
    return group or hd


def cache_arrays(cache):
    """(k_codes, v_codes, k_scales, v_scales) of a cache as numpy arrays,
    codes shaped [B][Hkv][cap][row bytes], scales [B][Hkv][cap][groups] or
    [B][cap] for one scale per position."""
    d = cache.desc
    B, H, HD, cap = d.batch, d.n_kv_heads, d.head_dim, d.capacity
    KR = HD * d.k_bits // 8
    kraw = cache.k_codes.cpu().numpy()
    if d.k_bits < 16:
        # 8/4-bit keys: tiles of 64 slots, slice-major (kvq.h): byte j of slot s at
        # ((s & ~63) * KR + (j // 16) * 1024 + (s & 63) * 16 + j % 16) within a (b, head)
        cap64 = (cap + 63) // 64 * 64
        kc = (kraw.reshape(B, H, cap64 // 64, KR // 16, 64, 16).transpose(0, 1, 2, 4, 3, 5)
              .reshape(B, H, cap64, KR)[:, :, :cap])
    else:
        kc = kraw.reshape(B, H, cap, KR)
    vraw = cache.v_codes.cpu().numpy()
    R = HD * d.v_bits // 8
    if d.v_bits < 16:
        # 8/4-bit values: four positions interleaved per byte (kvq.h):
        # byte j of slot s at ((s & ~3) * R + 4 * j + (s & 3)) within a (b, head)
        # stored offset binary: code + 128 per byte (8-bit), code + 8 per nibble (4-bit)
        cap4 = (cap + 3) // 4 * 4
        vc = vraw.reshape(B, H, cap4 // 4, R, 4).transpose(0, 1, 2, 4, 3).reshape(B, H, cap4, R)[:, :, :cap]
        vc = vc ^ np.uint8(0x80 if d.v_bits == 8 else 0x88)
    else:
        vc = vraw.reshape(B, H, cap, R)
    out = [kc, vc]
    per_row = d.group_size == H * HD and H > 1
    for t in (cache.k_scales, cache.v_scales):
        if t is None:
            out.append(None)
        else:
            a = t.cpu().numpy().view(np.uint16)
            out.append(a.reshape(B, cap) if per_row else a.reshape(B, H, cap, HD // d.group_size))
    return out


def check_codes(oq, cache, K, V, positions_of_slot):
    """Bit-exact check of every stored row: K, V float32 [B][Hkv][n_pos][HD];
    positions_of_slot: {slot: position} that the cache must hold."""
    d = cache.desc
    B, H, HD = d.batch, d.n_kv_heads, d.head_dim
    kc, vc, ks, vs = cache_arrays(cache)
    slots = np.array(sorted(positions_of_slot), dtype=np.int64)
    pos = np.array([positions_of_slot[s] for s in slots], dtype=np.int64)
    per_row = d.group_size == H * HD and H > 1
    for side, (src, codes, scales, bits) in enumerate(((K, kc, ks, d.k_bits), (V, vc, vs, d.v_bits))):
        name = "K" if side == 0 else "V"
        if per_row and bits < 16:
            for b in range(B):
                rows_ = src[b][:, pos, :].transpose(1, 0, 2).reshape(len(pos), H * HD)
                p, s = oq.encode_rows(rows_, H * HD, bits)
                got = codes[b][:, slots, :].transpose(1, 0, 2).reshape(len(pos), -1)
                assert np.array_equal(got, p), f"{name} codes differ (b={b}, per-row)"
                assert np.array_equal(scales[b][slots], s[:, 0]), f"{name} scales differ (b={b})"
        else:
            g = d.group_size if bits < 16 else HD
            p, s = oq.encode_rows(src[:, :, pos, :], g, bits)
            got = codes[:, :, slots, :]
            if not np.array_equal(got, p):
                bad = np.argwhere(got != p)[:5]
                raise AssertionError(f"{name} codes differ at {bad.tolist()} (bits={bits})")
            if bits < 16:
                assert np.array_equal(scales[:, :, slots, :], s), f"{name} scales differ"


def linear_slots(n_pos, cap):
    return {p: p for p in range(min(n_pos, cap))}


def window_slots(oq, n_pos, A, W):
    held = oq.attended_positions(n_pos - 1, A, W)
    return {oq.slot_of(int(p), A, W): int(p) for p in held}


def softmax_default(hd):
    return 1.0 / math.sqrt(hd)


# ---------------------------------------------------------------- paged caches
BUFFERS = ("k_codes", "v_codes", "k_scales", "v_scales")


def paged_table(B, pps, n_pages, seed):
    """A random assignment of distinct pool pages to the logical pages."""
    rng = np.random.default_rng(1000 + seed)
    return rng.permutation(n_pages)[: B * pps].reshape(B, pps).astype(np.int32)


def unit_view(cache, name):
    """The pool `name` as [n_pages][heads][elements per page and head]
    (heads 1 for one scale per slot over all heads)."""
    import decode_attention_quantized_kvq_amd as kvq
    d = cache.desc
    t = getattr(cache, name)
    size = kvq.kvq_cache_sizes(d)[BUFFERS.index(name)] // t.element_size()
    per_row = name.endswith("scales") and d.group_size == d.n_kv_heads * d.head_dim and d.n_kv_heads > 1
    return t[:size].view(d.n_pages, 1 if per_row else d.n_kv_heads, -1)


def gathered(cache, table, name):
    """Pool `name` gathered in table order: the contiguous cache's layout,
    [batch][heads][elements per sequence and head]."""
    import torch
    u = unit_view(cache, name)
    B, pps = table.shape
    g = u[torch.as_tensor(table.reshape(-1).astype(np.int64), device=u.device)]
    return g.view(B, pps, u.shape[1], -1).permute(0, 2, 1, 3).reshape(B, u.shape[1], -1)


def _contig_view(cache, name, heads):
    import decode_attention_quantized_kvq_amd as kvq
    d = cache.desc
    t = getattr(cache, name)
    size = kvq.kvq_cache_sizes(d)[BUFFERS.index(name)] // t.element_size()
    return t[:size].view(d.batch, heads, -1)


def assert_same_storage(paged, table, contig):
    import torch
    for name in BUFFERS:
        if getattr(contig, name) is None:
            assert getattr(paged, name) is None
            continue
        g = gathered(paged, table, name)
        c = _contig_view(contig, name, g.shape[1])
        assert torch.equal(g, c), f"{name}: gathered pages differ from the contiguous cache"
        spare = sorted(set(range(paged.desc.n_pages)) - set(table.reshape(-1).tolist()))
        if spare:
            u = unit_view(paged, name)
            assert not torch.any(u[torch.as_tensor(spare, device=u.device)]), f"{name}: a spare page was written"


# ---------------------------------------------------------------- zero-point codec
def zp_arrays(cache):
    """(k_codes, v_codes, k_scales, k_zeros, v_scales, v_zeros) of a zero-point
    cache as the oracle's unsigned codes: keys are stored as code - 2^(bits-1)
    (two's complement, so code XOR 0x80 per byte or 0x8 per nibble), values as
    the code; scale words hold the fp16 scale in the low and the zero point in
    the high half."""
    d = cache.desc
    B, H, HD, cap = d.batch, d.n_kv_heads, d.head_dim, d.capacity
    KR = HD * d.k_bits // 8
    cap64 = (cap + 63) // 64 * 64
    kraw = cache.k_codes.cpu().numpy()
    kc = (kraw[:B * H * cap64 * KR].reshape(B, H, cap64 // 64, KR // 16, 64, 16).transpose(0, 1, 2, 4, 3, 5)
          .reshape(B, H, cap64, KR)[:, :, :cap]) ^ np.uint8(0x80 if d.k_bits == 8 else 0x88)
    VR = HD * d.v_bits // 8
    cap4 = (cap + 3) // 4 * 4
    vraw = cache.v_codes.cpu().numpy()
    vc = vraw[:B * H * cap4 * VR].reshape(B, H, cap4 // 4, VR, 4).transpose(0, 1, 2, 4, 3).reshape(B, H, cap4, VR)[:, :, :cap]
    per_row = d.group_size == H * HD and H > 1
    out = [kc, vc]
    for t in (cache.k_scales, cache.v_scales):
        w = t.cpu().numpy().view(np.uint32)
        w = w.reshape(B, cap) if per_row else w.reshape(B, H, cap, HD // d.group_size)
        out += [(w & 0xFFFF).astype(np.uint16), (w >> 16).astype(np.uint8)]
    return out


def check_codes_zp(oq, cache, K, V, positions_of_slot):
    """Bit-exact check of every stored row of a zero-point cache against the
    oracle's asymmetric codec: codes, fp16 scales and zero points."""
    d = cache.desc
    B, H, HD = d.batch, d.n_kv_heads, d.head_dim
    kc, vc, ks, kz, vs, vz = zp_arrays(cache)
    slots = np.array(sorted(positions_of_slot), dtype=np.int64)
    pos = np.array([positions_of_slot[s] for s in slots], dtype=np.int64)
    per_row = d.group_size == H * HD and H > 1
    for name, src, codes, scales, zeros, bits in (("K", K, kc, ks, kz, d.k_bits), ("V", V, vc, vs, vz, d.v_bits)):
        if per_row:
            for b in range(B):
                rows_ = src[b][:, pos, :].transpose(1, 0, 2).reshape(len(pos), H * HD)
                p, s, z = oq.encode_rows_asym(rows_, H * HD, bits)
                got = codes[b][:, slots, :].transpose(1, 0, 2).reshape(len(pos), -1)
                assert np.array_equal(got, p), f"{name} codes differ (b={b}, per-row)"
                assert np.array_equal(scales[b][slots], s[:, 0]), f"{name} scales differ (b={b})"
                assert np.array_equal(zeros[b][slots], z[:, 0]), f"{name} zero points differ (b={b})"
        else:
            p, s, z = oq.encode_rows_asym(src[:, :, pos, :], d.group_size, bits)
            got = codes[:, :, slots, :]
            if not np.array_equal(got, p):
                bad = np.argwhere(got != p)[:5]
                raise AssertionError(f"{name} codes differ at {bad.tolist()} (bits={bits})")
            assert np.array_equal(scales[:, :, slots, :], s), f"{name} scales differ"
            assert np.array_equal(zeros[:, :, slots, :], z), f"{name} zero points differ"
