"""Pins for the oracle's attention and its decode step.

The decode step follows the mni-ml page ("how the KV cache creates speed":
each step adds one K and one V row and reuses the cached ones) and the
aihot.vn page (Q is used only at the current position): the current query
attends, by softmax, over every cached row including the one just appended.
Pins: closed forms, a 50-digit brute force, and torch's
scaled_dot_product_attention in float64 on the CPU (a library routine) over
the stored rows.
"""
import math

import mpmath
import numpy as np
import pytest
import torch

import workloads as wl


def _sdpa(q, K, V, scale):
    """q [Hq][d], K/V [Hkv][n][d] float64 -> [Hq][d] via torch SDPA with
    query head h reading KV head h // (Hq/Hkv) (repeat_interleave)."""
    Hq, Hkv = q.shape[0], K.shape[0]
    Kt = torch.from_numpy(np.ascontiguousarray(K)).repeat_interleave(Hq // Hkv, dim=0)
    Vt = torch.from_numpy(np.ascontiguousarray(V)).repeat_interleave(Hq // Hkv, dim=0)
    qt = torch.from_numpy(np.ascontiguousarray(q))[:, None, :]
    o = torch.nn.functional.scaled_dot_product_attention(qt, Kt, Vt, scale=scale)
    return o[:, 0, :].numpy()


# ------------------------------------------------------------ closed forms
def test_single_row_returns_its_value(oq):
    rng = np.random.default_rng(0)
    K, V, q = rng.standard_normal((1, 16)), rng.standard_normal((1, 16)), rng.standard_normal(16)
    assert np.array_equal(oq.attend(q, K, V, 0.25), V[0])


def test_zero_query_gives_mean(oq):
    rng = np.random.default_rng(1)
    K, V = rng.standard_normal((37, 8)), rng.standard_normal((37, 8))
    np.testing.assert_allclose(oq.attend(np.zeros(8), K, V, 1.0), V.mean(0), rtol=0, atol=1e-14)


def test_equal_keys_give_mean(oq):
    rng = np.random.default_rng(2)
    K = np.tile(rng.standard_normal((1, 8)), (20, 1))
    V = rng.standard_normal((20, 8))
    np.testing.assert_allclose(oq.attend(rng.standard_normal(8), K, V, 0.7), V.mean(0), atol=1e-14)


def test_two_rows_sigmoid(oq):
    q = np.array([1.0, 2.0])
    K = np.array([[0.5, -1.0], [2.0, 1.0]])
    V = np.array([[1.0, 0.0], [0.0, 1.0]])
    s = 0.3
    z0, z1 = s * (q @ K[0]), s * (q @ K[1])
    w1 = 1.0 / (1.0 + math.exp(z0 - z1))
    np.testing.assert_allclose(oq.attend(q, K, V, s), [1 - w1, w1], atol=1e-15)


def test_shift_and_permutation_invariance(oq):
    rng = np.random.default_rng(3)
    q, K, V = rng.standard_normal(8), rng.standard_normal((50, 8)), rng.standard_normal((50, 8))
    base = oq.attend(q, K, V, 0.4)
    u = rng.standard_normal(8)
    np.testing.assert_allclose(oq.attend(q, K + u, V, 0.4), base, atol=1e-13)  # shifts every z by q.u
    perm = rng.permutation(50)
    np.testing.assert_allclose(oq.attend(q, K[perm], V[perm], 0.4), base, atol=1e-14)
    # large scores do not overflow (max subtracted first)
    np.testing.assert_allclose(oq.attend(q, K * 1e3, V, 1.0), oq.attend(q, K * 1e3, V, 1.0))
    assert np.all(np.isfinite(oq.attend(q, K * 1e4, V, 1.0)))


def test_brute_force_50_digits(oq):
    mpmath.mp.dps = 50
    rng = np.random.default_rng(4)
    for n in range(1, 9):
        for d in (1, 3, 8):
            q, K, V = rng.standard_normal(d), rng.standard_normal((n, d)), rng.standard_normal((n, d))
            s = 1 / math.sqrt(d)
            z = [mpmath.mpf(s) * mpmath.fsum(mpmath.mpf(q[c]) * mpmath.mpf(K[t, c]) for c in range(d))
                 for t in range(n)]
            w = [mpmath.e ** zt for zt in z]
            tot = mpmath.fsum(w)
            want = [float(mpmath.fsum(w[t] * mpmath.mpf(V[t, c]) for t in range(n)) / tot) for c in range(d)]
            np.testing.assert_allclose(oq.attend(q, K, V, s), want, rtol=0, atol=1e-14)


# ------------------------------------------------------------ decode step
def _mk(hkv, n, hd, hq, seed, outliers=False):
    rng = np.random.default_rng(seed)
    K = rng.standard_normal((hkv, n, hd)).astype(np.float32)
    if outliers:
        K[:, :, ::17] *= np.float32(10.0)
    V = rng.standard_normal((hkv, n, hd)).astype(np.float32)
    q = rng.standard_normal((hq, hd)).astype(np.float32)
    return K, V, q


@pytest.mark.parametrize("hkv,hq", [(4, 4), (2, 8), (1, 4)])
def test_fp16_mode_equals_dense_sdpa(oq, hkv, hq):
    """FP16 mode is plain softmax attention over fp16-rounded K/V."""
    K, V, q = _mk(hkv, 70, 64, hq, 10)
    got = oq.decode_step(16, 16, 0, 0, 0, K, V, q, 1 / 8)
    want = _sdpa(q.astype(np.float64), K.astype(np.float16).astype(np.float64),
                 V.astype(np.float16).astype(np.float64), 1 / 8)
    np.testing.assert_allclose(got, want, rtol=0, atol=1e-12)


def test_fp32_mode_equals_dense_sdpa(oq):
    K, V, q = _mk(2, 33, 16, 4, 11)
    got = oq.decode_step(32, 32, 0, 0, 0, K, V, q, 0.25)
    want = _sdpa(q.astype(np.float64), K.astype(np.float64), V.astype(np.float64), 0.25)
    np.testing.assert_allclose(got, want, rtol=0, atol=1e-12)


@pytest.mark.parametrize("kb,vb,g", [(8, 8, 64), (8, 4, 64), (4, 4, 64), (4, 8, 32), (8, 8, 32)])
def test_quantized_mode_is_sdpa_over_stored_rows(oq, kb, vb, g):
    """Quantized modes attend over code * scale of each stored row."""
    K, V, q = _mk(2, 45, 64, 8, 12, outliers=True)

    def stored(x, bits):
        out = np.zeros(x.shape, np.float64)
        for h in range(x.shape[0]):
            for t in range(x.shape[1]):
                p, s = oq.encode_row(x[h, t], g, bits)
                out[h, t] = oq.decode_row(p, s, x.shape[2], g, bits)
        return out

    got = oq.decode_step(kb, vb, g, 0, 0, K, V, q, 0.125)
    want = _sdpa(q.astype(np.float64), stored(K, kb), stored(V, vb), 0.125)
    np.testing.assert_allclose(got, want, rtol=0, atol=1e-12)


def test_per_row_scale_mode(oq):
    """One scale over the whole position row of all KV heads (mni-ml's
    per-tensor INT8, read as one scale per appended row)."""
    hkv, hd, n = 4, 16, 20
    K, V, q = _mk(hkv, n, hd, hkv, 13)
    D = hkv * hd

    def stored(x):
        out = np.zeros(x.shape, np.float64)
        for t in range(n):
            row = np.ascontiguousarray(x[:, t, :].reshape(D))
            p, s = oq.encode_row(row, D, 8)
            assert s.size == 1
            out[:, t, :] = oq.decode_row(p, s, D, D, 8).reshape(hkv, hd)
        return out

    got = oq.decode_step(8, 8, D, 0, 0, K, V, q, 0.25)
    want = _sdpa(q.astype(np.float64), stored(K), stored(V), 0.25)
    np.testing.assert_allclose(got, want, rtol=0, atol=1e-12)


def test_window_mode_restricts_positions(oq):
    A, W, n = 3, 5, 20
    K, V, q = _mk(1, n, 8, 2, 14)
    keep = list(range(A)) + list(range(n - W, n))
    got = oq.decode_step(16, 16, 0, A, W, K, V, q, 0.5)
    want = _sdpa(q.astype(np.float64), K[:, keep].astype(np.float16).astype(np.float64),
                 V[:, keep].astype(np.float16).astype(np.float64), 0.5)
    np.testing.assert_allclose(got, want, rtol=0, atol=1e-12)
    # before any eviction the window is the whole prefix
    got2 = oq.decode_step(16, 16, 0, A, W, K[:, :7], V[:, :7], q, 0.5)
    np.testing.assert_allclose(got2, oq.decode_step(16, 16, 0, 0, 0, K[:, :7], V[:, :7], q, 0.5), atol=0)


def test_head_subset_matches_full(oq):
    K, V, q = _mk(2, 30, 16, 8, 15)
    full = oq.decode_step(8, 4, 16, 0, 0, K, V, q, 0.25)
    part = oq.decode_step(8, 4, 16, 0, 0, K, V, q, 0.25, hq_begin=3, hq_end=6)
    np.testing.assert_array_equal(part, full[3:6])


def test_gqa_grouping_is_contiguous(oq):
    """Query heads 0..G-1 share KV head 0: changing KV head 1 leaves them alone."""
    K, V, q = _mk(2, 12, 8, 4, 16)
    a = oq.decode_step(16, 16, 0, 0, 0, K, V, q, 0.3)
    K2, V2 = K.copy(), V.copy()
    K2[1] += 1
    V2[1] -= 2
    b = oq.decode_step(16, 16, 0, 0, 0, K2, V2, q, 0.3)
    np.testing.assert_array_equal(a[:2], b[:2])
    assert not np.allclose(a[2:], b[2:])


def test_workload_generator_prefix_stable():
    w = wl.TINY
    a = wl.rows(w, wl.K_STREAM, 0, 0, 100)
    b = wl.rows(w, wl.K_STREAM, 0, 0, 257)
    np.testing.assert_array_equal(a, b[:, :100])
    c = wl.rows(w, wl.K_STREAM, 0, 0, 57, start=100)
    np.testing.assert_array_equal(c, b[:, 100:157])
    w3 = wl.TINYLOOP
    ch = wl.outlier_channels(w3)
    assert ch.size == 20
    r = wl.rows(w3, wl.K_STREAM, 0, 0, 64).transpose(1, 0, 2).reshape(64, -1)
    big = np.abs(r[:, ch]).mean()
    small = np.abs(np.delete(r, ch, axis=1)).mean()
    assert 6 < big / small < 10
