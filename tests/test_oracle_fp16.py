"""Pins for the oracle's IEEE binary16 codec.

The pages name FP16 K/V rows and FP16 scales (TinyLoop "KV Cache 模式",
five-modes table) but fix no rounding; the reading is IEEE-754
round-to-nearest-even with subnormals.  numpy's float32 -> float16 cast is
that conversion, so it pins the oracle's hand-written encoder exhaustively.
"""
import os

import numpy as np
import pytest


def test_f16_decode_all_patterns(oq):
    h = np.arange(1 << 16, dtype=np.uint16)
    ours = oq.f16_to_f64(h)
    ref = h.view(np.float16).astype(np.float64)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan)
    assert np.array_equal(ours[~nan], ref[~nan])
    # signed zeros keep their sign
    assert np.array_equal(np.signbit(ours[~nan]), np.signbit(ref[~nan]))


def _check_patterns(oq, u):
    x = u.view(np.float32)
    ours = oq.f16_from_f32(x)
    with np.errstate(over="ignore", invalid="ignore"):
        ref = x.astype(np.float16).view(np.uint16)
    ref_nan = ((ref & 0x7C00) == 0x7C00) & ((ref & 0x03FF) != 0)
    our_nan = ((ours & 0x7C00) == 0x7C00) & ((ours & 0x03FF) != 0)
    assert np.array_equal(our_nan, ref_nan)
    ok = ~ref_nan
    bad = np.flatnonzero(ours[ok] != ref[ok])
    assert bad.size == 0, (x[ok][bad[:4]], ours[ok][bad[:4]], ref[ok][bad[:4]])


def test_f16_encode_rounding_neighbourhoods(oq):
    """Every sign, exponent and top-10 fraction bits, with the low 13 bits
    (the ones rounding drops) at and around the tie points."""
    low = np.array([0, 1, 2, 0x0FFE, 0x0FFF, 0x1000, 0x1001, 0x1002, 0x1FFE, 0x1FFF], np.uint32)
    top = np.arange(1 << 19, dtype=np.uint32) << np.uint32(13)      # sign, exponent, 10 bits
    _check_patterns(oq, (top[:, None] | low[None, :]).ravel())
    # subnormal-result range: exponents 102..113 drop more than 13 bits
    e = np.arange(102, 114, dtype=np.uint32)
    m = np.arange(1 << 23, dtype=np.uint32)[::3]
    _check_patterns(oq, ((e[:, None] << np.uint32(23)) | m[None, :]).ravel())


def test_f16_encode_strided_sample(oq):
    _check_patterns(oq, (np.arange(0, 1 << 32, 4099, dtype=np.uint64)).astype(np.uint32))


@pytest.mark.slow
@pytest.mark.skipif(not os.environ.get("KVQ_EXHAUSTIVE_FP16"), reason="set KVQ_EXHAUSTIVE_FP16=1 (about 6 minutes)")
def test_f16_encode_exhaustive(oq):
    """All 2^32 float32 bit patterns against numpy's cast (any NaN == any NaN)."""
    step = 1 << 26
    for hi in range(0, 1 << 32, step):
        _check_patterns(oq, np.arange(hi, hi + step, dtype=np.uint64).astype(np.uint32))


def test_f16_encode_boundaries(oq):
    cases = {
        65504.0: 0x7BFF,          # largest finite
        65519.99: 0x7BFF,         # below the rounding midpoint to 2^16
        65520.0: 0x7C00,          # midpoint, ties to even -> inf
        2.0 ** -24: 0x0001,       # smallest subnormal
        2.0 ** -25: 0x0000,       # half of it: tie to even -> 0
        1.5 * 2.0 ** -25: 0x0001,
        2.0 ** -14: 0x0400,       # smallest normal
        1.0 + 2.0 ** -11: 0x3C00,  # tie between 1 and 1+2^-10 -> even (1)
        1.0 + 3 * 2.0 ** -11: 0x3C02,
        -0.0: 0x8000,
    }
    for v, want in cases.items():
        assert int(oq.f16_from_f32(np.array([v], np.float32))[0]) == want, (v, hex(want))


def test_scale_saturates(oq):
    x = np.array([65504.0, 65520.0, 1e9, np.inf, 1.0], np.float32)
    got = oq.f16_scale_from_f32(x)
    assert list(map(int, got)) == [0x7BFF, 0x7BFF, 0x7BFF, 0x7BFF, 0x3C00]
