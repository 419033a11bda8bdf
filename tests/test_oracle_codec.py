"""Pins for the oracle's symmetric quantizer, packer and row codec.

Sources: TinyLoop "KV Cache 模式" five-modes table (INT8 = 255 levels, INT4
symmetric = 15 levels, nibble-packed, one FP16 scale per head; relative L2
error about 0.6 % / 10 %); mni-ml page (symmetric INT8 with a scale);
KVSplit page (separate K and V widths).
"""
from fractions import Fraction
from pathlib import Path

import numpy as np
import pytest

GOLD = Path(__file__).parent / "golden"


def _cases():
    for line in (GOLD / "codec_examples.txt").read_text().splitlines():
        if not line.strip() or line.startswith("#"):
            continue
        qm, xs, sc, codes, packed = [p.strip() for p in line.split("|")]
        yield (int(qm), np.array([float(v) for v in xs.split()], np.float32), int(sc, 16),
               [int(c) for c in codes.split()], None if packed == "-" else [int(b, 16) for b in packed.split()])


@pytest.mark.parametrize("case", list(_cases()), ids=lambda c: f"q{c[0]}-{c[1][:2]}")
def test_worked_examples(oq, case):
    qm, x, scale_bits, codes, packed = case
    got_codes, got_scale = oq.quantize_group(x, qm)
    assert got_scale == scale_bits
    assert got_codes.tolist() == codes
    if packed is not None:
        assert oq.pack_int4(got_codes).tolist() == packed


def _exact_nearest_even(x: float, s: float, qm: int) -> int:
    """argmin over integer codes c in [-qm, qm] of |x - c*s|, exact rationals,
    ties to the even code: the definition of rounding to the grid."""
    X, S = Fraction(x), Fraction(s)
    best = None
    for c in range(-qm, qm + 1):
        d = abs(X - c * S)
        if best is None or d < best[0] or (d == best[0] and c % 2 == 0):
            best = (d, c)
    return best[1]


@pytest.mark.parametrize("qm", [127, 7])
def test_codes_are_nearest_grid_points(oq, qm):
    """Each code is the exact nearest multiple of the stored scale (ties to even),
    except where the fp32 quotient x/s rounds across a half-integer, which the
    reading fixes in fp32; such cases must lie within 2^-20 of a tie."""
    rng = np.random.default_rng(7)
    n_mismatch = 0
    for trial in range(300 if qm < 100 else 40):
        x = rng.standard_normal(32).astype(np.float32) * np.float32(rng.choice([1e-3, 1.0, 50.0]))
        codes, sb = oq.quantize_group(x, qm)
        s = float(oq.f16_to_f64(np.array([sb], np.uint16))[0])
        for xi, ci in zip(x.tolist(), codes.tolist()):
            want = _exact_nearest_even(xi, s, qm)
            if want != ci:
                n_mismatch += 1
                r = Fraction(xi) / Fraction(s)
                frac = abs(r - (r.numerator // r.denominator)) - Fraction(1, 2)
                assert abs(frac) < Fraction(1, 1 << 20) * abs(r), (xi, s, ci, want)
    assert n_mismatch <= 2


@pytest.mark.parametrize("bits,qm", [(8, 127), (4, 7)])
def test_codec_invariants(oq, bits, qm):
    rng = np.random.default_rng(11)
    x = rng.standard_normal((500, 128)).astype(np.float32)
    x[::7] *= np.float32(1e-3)
    x[::11, 5] *= np.float32(40.0)
    payload, scales = oq.encode_rows(x, 128, bits)
    for i in range(x.shape[0]):
        if bits == 8:
            codes = payload[i].view(np.int8)
        else:
            codes = oq.unpack_int4(payload[i], 128)
        s = float(oq.f16_to_f64(scales[i])[0])
        # range and symmetry: -qmax-1 never appears
        assert codes.min() >= -qm and codes.max() <= qm
        # the largest-magnitude element lands on +-qmax
        j = int(np.argmax(np.abs(x[i])))
        assert abs(int(codes[j])) == qm
        # round-trip error at most half a step
        err = np.abs(x[i].astype(np.float64) - codes.astype(np.float64) * s)
        assert err.max() <= s / 2 * (1 + 2.0 ** -20)
        # decode_row is code * scale exactly
        dec = oq.decode_row(payload[i], scales[i], 128, 128, bits)
        assert np.array_equal(dec, codes.astype(np.float64) * s)


@pytest.mark.parametrize("bits", [8, 4])
def test_requantize_is_identity(oq, bits):
    """Quantizing the dequantized row again reproduces codes and scale."""
    rng = np.random.default_rng(5)
    x = rng.standard_normal((2000, 64)).astype(np.float32)
    p1, s1 = oq.encode_rows(x, 64, bits)
    xhat = np.stack([oq.decode_row(p1[i], s1[i], 64, 64, bits) for i in range(len(x))]).astype(np.float32)
    p2, s2 = oq.encode_rows(xhat, 64, bits)
    assert np.array_equal(p1, p2) and np.array_equal(s1, s2)


def test_relative_error_matches_page_bands(oq):
    bands = {}
    for line in (GOLD / "accuracy_bands.txt").read_text().splitlines():
        if line.strip() and not line.startswith("#"):
            b, lo, hi = line.split()
            bands[int(b)] = (float(lo), float(hi))
    rng = np.random.default_rng(3)
    x = rng.standard_normal((4000, 128)).astype(np.float32)
    for bits, (lo, hi) in bands.items():
        p, s = oq.encode_rows(x, 128, bits)
        xhat = np.stack([oq.decode_row(p[i], s[i], 128, 128, bits) for i in range(len(x))])
        rel = np.linalg.norm(xhat - x) / np.linalg.norm(x) * 100
        assert lo <= rel <= hi, (bits, rel)


def test_pack_unpack_all_pairs(oq):
    codes = np.array([(a, b) for a in range(-8, 8) for b in range(-8, 8)], np.int8).ravel()
    packed = oq.pack_int4(codes)
    assert packed.size == 256 and sorted(packed.tolist()) == list(range(256))
    assert np.array_equal(oq.unpack_int4(packed, codes.size), codes)
    # even element in the low nibble
    assert oq.pack_int4(np.array([1, 0], np.int8)).tolist() == [0x01]
    assert oq.pack_int4(np.array([0, 1], np.int8)).tolist() == [0x10]
    assert oq.pack_int4(np.array([-1, 0], np.int8)).tolist() == [0x0F]


def test_group_size_splits_scales(oq):
    """Smaller groups carry their own scales: a row with one large group and
    one small group keeps resolution in the small one."""
    x = np.concatenate([np.full(32, 100.0), np.linspace(-1, 1, 32)]).astype(np.float32)
    p, s = oq.encode_row(x, 32, 8)
    assert s.size == 2
    dec = oq.decode_row(p, s, 64, 32, 8)
    assert np.abs(dec[32:] - x[32:]).max() <= float(oq.f16_to_f64(s[1:2])[0]) / 2 * (1 + 1e-6)
    p1, s1 = oq.encode_row(x, 64, 8)
    assert s1.size == 1
    dec1 = oq.decode_row(p1, s1, 64, 64, 8)
    assert np.abs(dec1[32:] - x[32:]).max() > np.abs(dec[32:] - x[32:]).max()


def test_dense_rows(oq):
    x = np.array([1.0, -2.5, 3.14159, 65519.0, 1e-8], np.float32)
    p, s = oq.encode_row(x, 1, 32)
    assert np.array_equal(oq.decode_row(p, s, 5, 1, 32), x.astype(np.float64))
    p, s = oq.encode_row(x, 1, 16)
    assert np.array_equal(oq.decode_row(p, s, 5, 1, 16), x.astype(np.float16).astype(np.float64))
