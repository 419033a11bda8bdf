"""Pins for the bytes-per-token accounting against the numbers the pages print."""
from pathlib import Path

import pytest

GOLD = {}
for line in (Path(__file__).parent / "golden" / "bytes_per_token.txt").read_text().splitlines():
    if line.strip() and not line.startswith("#"):
        k, v = line.split()
        GOLD[k] = float(v)

MIB = 1024 * 1024


def test_tinyloop_formula(oq):
    # TinyLoop memory-formula table: D = 2048 = 16 heads x 128.
    assert oq.bytes_per_token(16, 16, 16, 128, 128) == GOLD["tinyloop_fp16_kv_bytes_per_token"]
    assert oq.bytes_per_token(8, 8, 16, 128, 128) == GOLD["tinyloop_int8_kv_bytes_per_token"]


def test_tinyloop_footprint(oq):
    # footprint table: bytes/token x n_layers (34) x max_seq_len (1024)
    fp16 = oq.bytes_per_token(16, 16, 16, 128, 128) * 34 * 1024 / MIB
    int8 = oq.bytes_per_token(8, 8, 16, 128, 128) * 34 * 1024 / MIB
    assert fp16 == GOLD["tinyloop_fp16_kv_total_mib"]
    assert round(int8) == GOLD["tinyloop_int8_kv_total_mib_printed"]
    assert round(100 * (1 - int8 / fp16)) == GOLD["tinyloop_saving_percent_printed"]


def test_kvsplit_ratios(oq):
    """KVSplit 8K table: K8V8 / K8V4 / K4V4 over FP16 are exactly 17/32,
    13/32 and 9/32, i.e. one 2-byte scale per 32 codes."""
    fp16 = oq.bytes_per_token(16, 16, 8, 128, 32)
    for mode, (kb, vb) in {"k8v8": (8, 8), "k8v4": (8, 4), "k4v4": (4, 4)}.items():
        ours = oq.bytes_per_token(kb, vb, 8, 128, 32) / fp16
        page = GOLD[f"kvsplit_{mode}_mb"] / GOLD["kvsplit_fp16_mb"]
        assert ours == pytest.approx(page, abs=1e-12), mode
    # one scale per 128-value head would not reproduce the page
    assert oq.bytes_per_token(8, 8, 8, 128, 128) / fp16 != pytest.approx(93.5 / 176, abs=1e-3)


def test_ondevice_k4v8_codes_only(oq):
    """On-device page: 224 MB -> 84 MB for INT4 keys + INT8 values; the ratio
    3/8 is the code payload alone (scale bytes not counted on the page)."""
    ratio = GOLD["ondevice_k4v8_mb"] / GOLD["ondevice_fp16_mb"]
    D = 3072  # any width: the payload ratio does not depend on it
    payload = D * (4 + 8) / 8
    assert payload / (D * (16 + 16) / 8) == pytest.approx(ratio, abs=1e-12)
    # with one scale per head the full formula lies a little above the page's ratio
    full = oq.bytes_per_token(4, 8, 24, 128, 128) / oq.bytes_per_token(16, 16, 24, 128, 128)
    assert ratio < full < ratio * 1.05


def test_mniml_about_four_x(oq):
    """mni-ml page: INT8 is 1 byte per element vs 4 for FP32, 3.78x after
    scale metadata.  Per-row fp16 scales give 4g/(g+2), just under 4."""
    page = GOLD["mniml_fp32_mb"] / GOLD["mniml_int8_mb"]
    assert 3.7 < page < 4.0
    ours = oq.bytes_per_token(32, 32, 8, 64, 512) / oq.bytes_per_token(8, 8, 8, 64, 512)
    assert ours == pytest.approx(4 * 512 / 514)
    assert page < ours < 4.0


@pytest.mark.parametrize("args", [(3, 8, 8, 128, 128), (8, 8, 8, 128, 48), (8, 8, 0, 128, 128),
                                  (4, 4, 1, 3, 1), (8, 8, 8, 128, 0)])
def test_invalid_returns_zero(oq, args):
    assert oq.bytes_per_token(*args) == 0
