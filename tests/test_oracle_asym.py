"""Pins for the oracle's asymmetric (zero-point) codec.

Source: the mni-ml page ("why INT8 loses no speed") names scale/zero-point
metadata next to the INT8 cache without fixing a form; the reading taken is
the affine min/max codec with the range widened to contain zero, one fp16
scale and one integer zero point per group (stated in
tests/golden/asym_examples.txt).  Pins: worked examples derived by hand from
IEEE rules; the range, the exact zero, the end codes, the error bound that
follows from the definition, the exact-rational nearest grid point; the
comparison with the symmetric codec's step on the same data; and torch's
scaled_dot_product_attention in float64 over the stored rows for the decode
step.
"""
from fractions import Fraction
from pathlib import Path

import numpy as np
import pytest
import torch

GOLD = Path(__file__).parent / "golden"


def _cases():
    for line in (GOLD / "asym_examples.txt").read_text().splitlines():
        if not line.strip() or line.startswith("#"):
            continue
        L, xs, sc, zp, codes, packed = [p.strip() for p in line.split("|")]
        yield (int(L), np.array([float(v) for v in xs.split()], np.float32), int(sc, 16), int(zp),
               [int(c) for c in codes.split()], None if packed == "-" else [int(b, 16) for b in packed.split()])


@pytest.mark.parametrize("case", list(_cases()), ids=lambda c: f"L{c[0]}-{c[1][:2]}")
def test_worked_examples(oq, case):
    L, x, scale_bits, zero, codes, packed = case
    got_codes, got_scale, got_zero = oq.quantize_group_asym(x, L)
    assert got_scale == scale_bits
    assert got_zero == zero
    assert got_codes.tolist() == codes
    if packed is not None:
        bits = 4 if L == 15 else 8
        p, s, z = oq.encode_rows_asym(x, x.size, bits)
        assert p.tolist() == packed and s.tolist() == [scale_bits] and z.tolist() == [zero]


def _f16(bits):
    return float(np.array([bits], np.uint16).view(np.float16)[0])


@pytest.mark.parametrize("bits,L", [(8, 255), (4, 15)])
def test_codec_invariants(oq, bits, L):
    """Codes and zero point in [0, L]; an exact zero decodes to exactly 0;
    the group minimum (when negative) takes code 0 and the maximum (when
    positive) code L or L - 1; |x - xhat| <= s/2 + max(0, (hi - lo) - L*s),
    the bound the definition gives (the second term is where the fp16 scale's
    span falls short of the range); decode_row_asym is (code - zero) * s."""
    rng = np.random.default_rng(17)
    x = rng.standard_normal((600, 64)).astype(np.float32)
    x[::5] += np.float32(2.0)                        # shifted rows: asymmetric ranges
    x[::7] = np.abs(x[::7])                          # all-positive rows
    x[::9] = -np.abs(x[::9])                         # all-negative rows
    x[::11, 3] = np.float32(0.0)
    x[::13] *= np.float32(1e-3)
    p, S, Z = oq.encode_rows_asym(x, 64, bits)
    for i in range(x.shape[0]):
        xi = x[i].astype(np.float64)
        if bits == 8:
            codes = p[i].astype(np.int64)
        else:
            codes = np.stack([p[i] & 0xF, p[i] >> 4], axis=1).reshape(-1).astype(np.int64)
        s, z = _f16(S[i, 0]), int(Z[i, 0])
        assert codes.min() >= 0 and codes.max() <= L and 0 <= z <= L
        xhat = (codes - z) * s
        lo, hi = min(0.0, float(x[i].min())), max(0.0, float(x[i].max()))
        span = float(np.float32(np.float32(hi) - np.float32(lo)))
        bound = s / 2 + max(0.0, span - L * s)
        assert np.abs(xi - xhat).max() <= bound * (1 + 2.0 ** -30)
        zeros = xi == 0.0
        assert np.all(xhat[zeros] == 0.0)
        if lo < 0:
            assert codes[int(np.argmin(xi))] == 0
        if hi > 0:
            assert codes[int(np.argmax(xi))] in (L, L - 1)
        dec = oq.decode_row_asym(p[i], S[i], Z[i], 64, 64, bits)
        assert np.array_equal(dec, xhat)


def _exact_nearest(x, s, z, L):
    """argmin over codes c in [0, L] of |x - (c - z) s| in exact rationals, ties
    to the code whose offset c - z is even (rounding x / s half to even)."""
    X, S = Fraction(x), Fraction(s)
    best = None
    for c in range(L + 1):
        d = abs(X - (c - z) * S)
        if best is None or d < best[0] or (d == best[0] and (c - z) % 2 == 0):
            best = (d, c)
    return best[1]


@pytest.mark.parametrize("L", [255, 15])
def test_codes_are_nearest_grid_points(oq, L):
    """Each code is the exact nearest point of the grid (c - z) s, except where
    the fp32 quotient x / s rounds across a half-integer (the reading decides
    in fp32); such cases lie within 2^-20 of a tie."""
    rng = np.random.default_rng(23)
    n_mismatch = 0
    for trial in range(40 if L == 255 else 300):
        x = (rng.standard_normal(24) + rng.uniform(-1.5, 1.5)).astype(np.float32)
        x *= np.float32(rng.choice([1e-3, 1.0, 30.0]))
        codes, sb, z = oq.quantize_group_asym(x, L)
        s = _f16(sb)
        for xi, ci in zip(x.tolist(), codes.tolist()):
            want = _exact_nearest(xi, s, z, L)
            if want != ci:
                n_mismatch += 1
                r = Fraction(xi) / Fraction(s)
                frac = abs(r - (r.numerator // r.denominator)) - Fraction(1, 2)
                assert abs(frac) < Fraction(1, 1 << 20) * max(abs(r), 1), (xi, s, ci, want)
    assert n_mismatch <= 2


@pytest.mark.parametrize("bits", [8, 4])
def test_requantize_is_identity(oq, bits):
    """Quantizing the decoded row again reproduces codes, scale and zero point
    (rows whose minimum is negative and maximum positive)."""
    rng = np.random.default_rng(29)
    x = rng.standard_normal((1500, 32)).astype(np.float32)
    x[:, 0] = -np.abs(x[:, 0]) - np.float32(0.5)
    x[:, 1] = np.abs(x[:, 1]) + np.float32(0.5)
    p1, s1, z1 = oq.encode_rows_asym(x, 32, bits)
    xhat = np.stack([oq.decode_row_asym(p1[i], s1[i], z1[i], 32, 32, bits) for i in range(len(x))])
    p2, s2, z2 = oq.encode_rows_asym(xhat.astype(np.float32), 32, bits)
    same = np.all(p1 == p2, axis=1) & np.all(s1 == s2, axis=1) & np.all(z1 == z2, axis=1)
    # the fp16 rounding of (hi - lo) / L can move the scale by one ulp on the
    # second pass; everything else must round-trip
    assert same.mean() > 0.9


@pytest.mark.parametrize("bits", [8, 4])
def test_step_is_finer_than_symmetric(oq, bits):
    """On the same groups the asymmetric step (hi - lo) / L is never coarser
    than the symmetric step max|x| / qmax = 2 max|x| / (L - 1), since
    hi - lo <= 2 max|x|; so its round-trip error on N(0,1) rows is smaller."""
    rng = np.random.default_rng(31)
    x = rng.standard_normal((2000, 128)).astype(np.float32)
    pa, sa, za = oq.encode_rows_asym(x, 128, bits)
    ps, ss = oq.encode_rows(x, 128, bits)
    step_a = np.array([_f16(v) for v in sa[:, 0]])
    step_s = np.array([_f16(v) for v in ss[:, 0]])
    assert np.all(step_a <= step_s)
    err_a = np.linalg.norm(np.stack([oq.decode_row_asym(pa[i], sa[i], za[i], 128, 128, bits) for i in range(200)])
                           - x[:200])
    err_s = np.linalg.norm(np.stack([oq.decode_row(ps[i], ss[i], 128, 128, bits) for i in range(200)]) - x[:200])
    assert err_a < err_s


def test_bytes_per_token_zp(oq):
    """The asymmetric codec's metadata as stored: a 32-bit word (fp16 scale +
    zero point field) per group and quantized side, so 2 bytes more per group
    and side than the symmetric layout; 16/32-bit sides are unchanged."""
    for kb, vb, hkv, hd, g in [(8, 8, 16, 128, 128), (4, 4, 8, 128, 128), (8, 4, 8, 128, 32), (4, 8, 8, 64, 64)]:
        sym = oq.bytes_per_token(kb, vb, hkv, hd, g)
        assert oq.bytes_per_token_zp(kb, vb, hkv, hd, g, 0) == sym
        assert oq.bytes_per_token_zp(kb, vb, hkv, hd, g, 1) == sym + 2 * 2 * (hkv * hd // g)
    # K4V4 per head at head_dim 128: 64 + 64 code bytes + 2 words of 4 bytes
    assert oq.bytes_per_token_zp(4, 4, 1, 128, 128, 1) == 136
    assert oq.bytes_per_token_zp(16, 16, 16, 128, 128, 1) == 8192


def _sdpa(q, K, V, scale):
    Hq, Hkv = q.shape[0], K.shape[0]
    Kt = torch.from_numpy(np.ascontiguousarray(K)).repeat_interleave(Hq // Hkv, dim=0)
    Vt = torch.from_numpy(np.ascontiguousarray(V)).repeat_interleave(Hq // Hkv, dim=0)
    qt = torch.from_numpy(np.ascontiguousarray(q))[:, None, :]
    return torch.nn.functional.scaled_dot_product_attention(qt, Kt, Vt, scale=scale)[:, 0, :].numpy()


@pytest.mark.parametrize("kb,vb,g", [(8, 8, 64), (8, 4, 32), (4, 4, 64), (4, 8, 32)])
def test_decode_step_is_sdpa_over_stored_rows(oq, kb, vb, g):
    """With asym the decode step attends over (code - zero) * scale of each
    stored row: torch SDPA in float64 over rows encoded and decoded one by one."""
    rng = np.random.default_rng(kb * 10 + vb + g)
    hkv, n, hd, hq = 2, 37, 64, 8
    K = (rng.standard_normal((hkv, n, hd)) + 0.7).astype(np.float32)
    V = (rng.standard_normal((hkv, n, hd)) - 0.4).astype(np.float32)
    q = rng.standard_normal((hq, hd)).astype(np.float32)

    def stored(x, bits):
        out = np.zeros(x.shape, np.float64)
        for h in range(x.shape[0]):
            for t in range(x.shape[1]):
                p, s, z = oq.encode_rows_asym(x[h, t], g, bits)
                out[h, t] = oq.decode_row_asym(p, s, z, hd, g, bits)
        return out

    got = oq.decode_step(kb, vb, g, 0, 0, K, V, q, 0.125, asym=True)
    want = _sdpa(q.astype(np.float64), stored(K, kb), stored(V, vb), 0.125)
    np.testing.assert_allclose(got, want, rtol=0, atol=1e-12)
    # and it is not the symmetric step
    sym = oq.decode_step(kb, vb, g, 0, 0, K, V, q, 0.125)
    assert np.abs(sym - got).max() > 1e-6


@pytest.mark.parametrize("bits,L", [(8, 255), (4, 15)])
def test_codes_follow_fp32_division(oq, bits, L):
    """The reading decides every rounding in IEEE fp32: recomputed here with
    numpy's correctly rounded float32 arithmetic and its nearest-even binary16
    cast (library routines), on groups whose values sit within a few ulps of
    the half-integer boundaries x / s = k + 1/2, where a reciprocal-multiply
    or a float64 quotient would round the other way."""
    rng = np.random.default_rng(37)
    f32 = np.float32
    n_near = 0
    for trial in range(400):
        g = 16
        x = (rng.standard_normal(g) * rng.choice([0.01, 1.0, 40.0]) + rng.uniform(-1, 1)).astype(f32)
        lo, hi = min(f32(0), x.min()), max(f32(0), x.max())
        s = f32(np.float16(f32(f32(hi - lo) / f32(L))))
        if not np.isfinite(s) or s == 0:
            continue
        # move most values next to a tie of the grid they will be coded on
        k = rng.integers(-L // 2, L // 2, g)
        near = ((k + 0.5) * np.float64(s)).astype(f32)
        for _ in range(int(rng.integers(0, 3))):
            near = np.nextafter(near, np.where(rng.random(g) < 0.5, f32(-np.inf), f32(np.inf))).astype(f32)
        keep = np.zeros(g, bool)
        keep[[int(np.argmin(x)), int(np.argmax(x))]] = True    # the range stays as drawn
        x = np.where(keep, x, np.clip(near, lo, hi)).astype(f32)
        codes, sb, z = oq.quantize_group_asym(x, L)
        lo, hi = min(f32(0), x.min()), max(f32(0), x.max())
        s = f32(np.float16(f32(f32(hi - lo) / f32(L))))
        assert sb == int(np.float16(s).view(np.uint16))
        zw = int(min(max(np.rint(f32(-lo) / s), 0), L))
        want = np.clip(np.rint(x / s) + zw, 0, L).astype(np.int64)
        assert z == zw
        assert codes.tolist() == want.tolist(), (x, s)
        q = (x / s).astype(np.float64)
        n_near += int(np.sum(np.abs(np.abs(q - np.floor(q)) - 0.5) < 1e-5))
    assert n_near > 1000                                        # the boundaries were exercised
