"""Host-side checks of libkvq.so that need no GPU: the library loads, exports
every entry point kvq.h declares, and rejects every invalid argument before
launching anything.  No compute call is made here."""
import ctypes
import re
from pathlib import Path

import numpy as np
import pytest

ROOT = Path(__file__).resolve().parents[1]


@pytest.fixture(scope="module")
def kvq():
    import decode_attention_quantized_kvq_amd as k
    if not k.LIB_PATH.exists():
        pytest.fail("libkvq.so is not built (python -m decode_attention_quantized_kvq_amd.build)")
    k.lib()
    return k


def header_functions():
    text = (ROOT / "include" / "kvq.h").read_text()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(kvq_\w+)\s*\(", text)))


def test_exports_every_declared_symbol(kvq):
    names = header_functions()
    assert len(names) >= 10
    lib = ctypes.CDLL(str(kvq.LIB_PATH))
    for n in names:
        assert hasattr(lib, n), n
    assert sorted(kvq.EXPORTED) == names


def test_status_strings(kvq):
    for code in range(0, -10, -1):
        s = kvq.kvq_status_str(code)
        assert s and s != "unknown status"
    assert kvq.kvq_status_str(-99) == "unknown status"


@pytest.mark.parametrize("args", [
    (8, 8, 16, 128, 128), (16, 16, 16, 128, 128), (8, 4, 8, 128, 128), (4, 4, 8, 128, 128),
    (4, 8, 8, 128, 32), (8, 8, 8, 64, 512), (32, 32, 8, 64, 64), (4, 4, 8, 128, 32),
    (3, 8, 8, 128, 128), (8, 8, 8, 128, 48), (8, 8, 0, 128, 128), (8, 8, 8, 128, 0),
])
def test_bytes_per_token_matches_oracle(kvq, oq, args):
    assert kvq.kvq_bytes_per_token(*args) == oq.bytes_per_token(*args)


def test_bytes_per_token_page_values(kvq):
    # TinyLoop memory-formula table (D = 2048, 16 heads)
    assert kvq.kvq_bytes_per_token(8, 8, 16, 128, 128) == 4160
    assert kvq.kvq_bytes_per_token(16, 16, 16, 128, 128) == 8192


def _desc(kvq, **kw):
    base = dict(batch=2, n_kv_heads=2, head_dim=128, capacity=100, k_bits=8, v_bits=8, group_size=128,
                n_anchor=0, window=0)
    base.update(kw)
    d = kvq.kvq_cache(**base)
    d.k_codes = d.v_codes = 0x10000
    d.k_scales = d.v_scales = 0x20000
    return d


def test_cache_sizes(kvq):
    d = _desc(kvq, batch=3, n_kv_heads=8, head_dim=128, capacity=1600, k_bits=4, v_bits=8, group_size=32)
    kc, vc, ks, vs = kvq.kvq_cache_sizes(d)
    rows = 3 * 8 * 1600
    assert (kc, vc, ks, vs) == (rows * 64, rows * 128, rows * 4 * 2, rows * 4 * 2)
    # integer keys pad each (sequence, head) to whole 64-slot tiles, integer values to 4 slots
    d = _desc(kvq, batch=2, n_kv_heads=3, head_dim=64, capacity=1001, k_bits=8, v_bits=4, group_size=64)
    kc, vc, _, _ = kvq.kvq_cache_sizes(d)
    assert kc == 2 * 3 * 1024 * 64 and vc == 2 * 3 * 1004 * 32
    d = _desc(kvq, n_kv_heads=4, head_dim=64, group_size=256)           # one scale per position
    assert kvq.kvq_cache_sizes(d)[2] == 2 * 100 * 2
    d = _desc(kvq, k_bits=16, v_bits=16)
    assert kvq.kvq_cache_sizes(d)[2:] == (0, 0)


@pytest.mark.parametrize("kw,code", [
    (dict(batch=0), -3), (dict(n_kv_heads=0), -3), (dict(capacity=0), -3), (dict(head_dim=96), -3),
    (dict(k_bits=16, v_bits=8), -2), (dict(k_bits=2), -2), (dict(k_bits=32, v_bits=16), -2),
    (dict(group_size=48), -4), (dict(group_size=16), -4), (dict(group_size=0), -4),
    (dict(n_anchor=4), -5), (dict(window=50), -5), (dict(n_anchor=-1, window=101), -5),
    (dict(batch=40000, n_kv_heads=2), -3),
])
def test_geometry_errors(kvq, kw, code):
    d = _desc(kvq, **kw)
    with pytest.raises(kvq.KvqError) as e:
        kvq.kvq_cache_sizes(d)
    assert e.value.status == code
    assert kvq.kvq_last_error()


def test_paged_cache_sizes(kvq):
    """Paged storage: each buffer is a pool of n_pages pages laid out as
    page_size-slot sequences of every KV head."""
    d = _desc(kvq, batch=3, n_kv_heads=8, head_dim=128, capacity=1024, k_bits=4, v_bits=8, group_size=32,
              page_size=256, n_pages=13)
    d.block_table = 0x50000
    kc, vc, ks, vs = kvq.kvq_cache_sizes(d)
    rows = 13 * 8 * 256
    assert (kc, vc, ks, vs) == (rows * 64, rows * 128, rows * 4 * 2, rows * 4 * 2)
    d = _desc(kvq, n_kv_heads=4, head_dim=64, capacity=128, group_size=256, page_size=64, n_pages=5)
    d.block_table = 0x50000
    assert kvq.kvq_cache_sizes(d)[2] == 5 * 64 * 2           # one scale per slot of each page
    d = _desc(kvq, k_bits=16, v_bits=16, capacity=4096, page_size=4096, n_pages=1)
    d.block_table = 0x50000
    assert kvq.kvq_cache_sizes(d) == (1 * 2 * 4096 * 256, 1 * 2 * 4096 * 256, 0, 0)


@pytest.mark.parametrize("kw,code", [
    (dict(page_size=100, capacity=200), -3), (dict(page_size=32, capacity=64), -3),
    (dict(page_size=8192, capacity=8192), -3), (dict(page_size=-64), -3),
    (dict(page_size=64, capacity=100), -3), (dict(page_size=64, capacity=128, n_pages=0), -3),
    (dict(page_size=4096, capacity=4096, n_pages=300000), -3),
])
def test_paged_geometry_errors(kvq, kw, code):
    d = _desc(kvq, **kw)
    d.block_table = 0x50000
    with pytest.raises(kvq.KvqError) as e:
        kvq.kvq_cache_sizes(d)
    assert e.value.status == code
    assert kvq.kvq_last_error()


def test_paged_pointer_errors(kvq):
    """A paged cache needs a 4-byte aligned block table; contiguous storage
    ignores it."""
    ok = 0x30000
    d = _desc(kvq, capacity=128, page_size=64, n_pages=4)
    with pytest.raises(kvq.KvqError) as e:                    # no block table
        kvq.kvq_append(d, ok, ok, 1, ok, 0)
    assert e.value.status == -1
    d.block_table = 0x50002
    with pytest.raises(kvq.KvqError) as e:
        kvq.kvq_append(d, ok, ok, 1, ok, 0)
    assert e.value.status == -7
    ws = kvq.kvq_workspace_bytes(d, 8, 128, 0)
    with pytest.raises(kvq.KvqError) as e:
        kvq.kvq_decode_attn(d, ok, 8, ok, 128, 0.0, 0, ok, ok, ws, 0)
    assert e.value.status == -7
    c = _desc(kvq)
    c.n_pages, c.block_table = 0, None                        # page_size 0: both ignored
    assert kvq.kvq_cache_sizes(c)[0] == 2 * 2 * 128 * 128


def test_append_argument_errors(kvq):
    d = _desc(kvq)
    ok = 0x30000
    cases = [
        (dict(n_new=-1), -3),
        (dict(k_new=None), -1),
        (dict(start_pos=None), -1),
        (dict(k_new=ok + 4), -7),
        (dict(start_pos=ok + 2), -7),
    ]
    for over, code in cases:
        a = dict(k_new=ok, v_new=ok, n_new=3, start_pos=ok)
        a.update(over)
        with pytest.raises(kvq.KvqError) as e:
            kvq.kvq_append(d, a["k_new"], a["v_new"], a["n_new"], a["start_pos"], 0)
        assert e.value.status == code, over
    # n_new == 0 is a no-op that launches nothing
    kvq.kvq_append(d, None, None, 0, None, 0)
    # misaligned or missing cache buffers
    d2 = _desc(kvq)
    d2.k_codes = 0x10008
    with pytest.raises(kvq.KvqError) as e:
        kvq.kvq_append(d2, ok, ok, 1, ok, 0)
    assert e.value.status == -7
    d3 = _desc(kvq)
    d3.k_scales = None
    with pytest.raises(kvq.KvqError) as e:
        kvq.kvq_append(d3, ok, ok, 1, ok, 0)
    assert e.value.status == -1


def test_decode_argument_errors(kvq):
    d = _desc(kvq)
    ws_need = kvq.kvq_workspace_bytes(d, 8, 100, 0)
    ok = 0x40000
    base = dict(q=ok, n_q_heads=8, seq_len=ok, max_seq_len=100, scale=0.0, chunk=0, out=ok, ws=ok, ws_bytes=ws_need)
    cases = [
        (dict(n_q_heads=6), -3), (dict(n_q_heads=2 * 3), -3), (dict(n_q_heads=32), -3),
        (dict(q=None), -1), (dict(seq_len=None), -1), (dict(ws=None), -1), (dict(out=None), -1),
        (dict(q=ok + 8), -7), (dict(ws=ok + 128), -7), (dict(out=ok + 4), -7), (dict(seq_len=ok + 1), -7),
        (dict(ws_bytes=ws_need - 1), -6),
        (dict(max_seq_len=0), -9), (dict(chunk=100), -9), (dict(chunk=32), -9), (dict(chunk=16384), -9),
        (dict(scale=-1.0), -9), (dict(scale=float("nan")), -9), (dict(scale=float("inf")), -9),
    ]
    for over, code in cases:
        a = dict(base)
        a.update(over)
        with pytest.raises(kvq.KvqError) as e:
            kvq.kvq_decode_attn(d, a["q"], a["n_q_heads"], a["seq_len"], a["max_seq_len"], a["scale"], a["chunk"],
                                a["out"], a["ws"], a["ws_bytes"], 0)
        assert e.value.status == code, over


def test_decode_step_argument_errors(kvq):
    """The fused step checks the append's and the decode's arguments alike,
    before it enqueues anything."""
    d = _desc(kvq)
    ws_need = kvq.kvq_workspace_bytes(d, 8, 100, 0)
    ok = 0x40000
    base = dict(k_new=ok, v_new=ok, n_new=1, start_pos=ok, q=ok, n_q_heads=8, seq_len=ok, max_seq_len=100,
                scale=0.0, chunk=0, out=ok, ws=ok, ws_bytes=ws_need)
    cases = [
        (dict(n_new=-1), -3), (dict(k_new=None), -1), (dict(start_pos=None), -1), (dict(v_new=ok + 4), -7),
        (dict(start_pos=ok + 2), -7),
        (dict(n_q_heads=6), -3), (dict(q=None), -1), (dict(seq_len=None), -1), (dict(ws=None), -1),
        (dict(out=None), -1), (dict(q=ok + 8), -7), (dict(ws=ok + 128), -7), (dict(out=ok + 4), -7),
        (dict(ws_bytes=ws_need - 1), -6), (dict(max_seq_len=0), -9), (dict(chunk=100), -9),
        (dict(scale=float("nan")), -9),
        # the decode's checks also hold when there is nothing to append
        (dict(n_new=0, q=None), -1), (dict(n_new=0, ws_bytes=ws_need - 1), -6),
    ]
    for over, code in cases:
        a = dict(base)
        a.update(over)
        with pytest.raises(kvq.KvqError) as e:
            kvq.kvq_decode_step(d, a["k_new"], a["v_new"], a["n_new"], a["start_pos"], a["q"], a["n_q_heads"],
                                a["seq_len"], a["max_seq_len"], a["scale"], a["chunk"], a["out"], a["ws"],
                                a["ws_bytes"], 0)
        assert e.value.status == code, over


def test_prepared_halves_argument_errors(kvq):
    d = _desc(kvq)
    ws = kvq.kvq_workspace_bytes(d, 8, 100, 0)
    ok = 0x40000
    with pytest.raises(kvq.KvqError) as e:
        kvq.kvq_prepare_query(d, None, 8, 100, 0.0, 0, ok, ws, 0)
    assert e.value.status == -1
    with pytest.raises(kvq.KvqError) as e:
        kvq.kvq_decode_partials_prepared(d, 8, None, 100, 0, ok, ws, 0)
    assert e.value.status == -1
    with pytest.raises(kvq.KvqError) as e:
        kvq.kvq_decode_partials_prepared(d, 8, ok, 100, 0, ok, ws - 1, 0)
    assert e.value.status == -6
    # 16/32-bit caches have no separate query preparation
    f = _desc(kvq, k_bits=16, v_bits=16)
    wf = kvq.kvq_workspace_bytes(f, 8, 100, 0)
    for call in (lambda: kvq.kvq_prepare_query(f, ok, 8, 100, 0.0, 0, ok, wf, 0),
                 lambda: kvq.kvq_decode_partials_prepared(f, 8, ok, 100, 0, ok, wf, 0)):
        with pytest.raises(kvq.KvqError) as e:
            call()
        assert e.value.status == -2


def test_read_probe_argument_errors(kvq):
    ok = 0x40000
    for args, code in [((None, 32768, ok, 64), -1), ((ok, 32768, None, 64), -1), ((ok + 8, 32768, ok, 64), -7),
                       ((ok, 32768, ok + 2, 64), -7), ((ok, 1000, ok, 64), -9), ((ok, 0, ok, 64), -9),
                       ((ok, 32768, ok, 3), -9)]:
        with pytest.raises(kvq.KvqError) as e:
            kvq.kvq_read_probe(*args, 0)
        assert e.value.status == code, args


def test_combine_argument_errors(kvq):
    need = 0
    with pytest.raises(kvq.KvqError) as e:
        kvq.kvq_combine(0, 8, 128, 4, 0x40000, 1 << 20, 0x50000, 0)
    assert e.value.status == -3
    with pytest.raises(kvq.KvqError) as e:
        kvq.kvq_combine(1, 8, 96, 4, 0x40000, 1 << 20, 0x50000, 0)
    assert e.value.status == -3
    with pytest.raises(kvq.KvqError) as e:
        kvq.kvq_combine(1, 8, 128, 4, 0x40000, 100, 0x50000, 0)
    assert e.value.status == -6
    with pytest.raises(kvq.KvqError) as e:
        kvq.kvq_combine(1, 8, 128, 4, 0x40010, 1 << 20, 0x50000, 0)
    assert e.value.status == -7


def test_workspace_and_chunks(kvq):
    # 32 sequences x 8 KV heads x 32K slots, 4:1 GQA, int4 K and V
    d = _desc(kvq, batch=32, n_kv_heads=8, capacity=32768, k_bits=4, v_bits=4)
    ch = kvq.kvq_chunk_tokens(d, 32, 32768)
    assert ch % 64 == 0 and 64 <= ch <= 4096
    n_chunks = kvq.kvq_chunk_count(d, 32, 32768, 0)
    assert n_chunks == -(-32768 // ch)
    assert 32 * 8 * n_chunks >= 2048                     # 8 workgroups per CU over 256 CUs
    P = 32 * 32
    partials = ((P * n_chunks * 8 + 255) // 256) * 256 + P * n_chunks * 128 * 4
    # int4 keys: the query's fixed-point digits (4 Horner digits and the extra low
    # one, per value; then two sums per scale group and head for the zero-point
    # codec; each unit's block padded to 256 bytes) and scales follow the partials,
    # then one extra-digit flag per (sequence, KV head) and the ticket counters'
    # zone (room for two per (sequence, KV head)); four heads at head_dim 128
    # add the matrix-core operand, one byte per digit (low, high, extra), head
    # and channel
    words = -(-(16 * 5 * 4 + 2 * 4 * 4 + 3 * 4 * 128 // 4) // 64) * 64
    digits = 32 * 8 * words * 4 + P * 4
    counters = 32 * 8 * 4 + 2 * 32 * 8 * 4
    ws = kvq.kvq_workspace_bytes(d, 32, 32768, 0)
    assert partials + digits + counters <= ws <= partials + digits + counters + 768
    ws256 = kvq.kvq_workspace_bytes(d, 32, 32768, 256)
    assert ws256 >= ((P * 128 * 8 + 255) // 256) * 256 + P * 128 * 512
    # 8/4-bit caches take chunks in multiples of 256 slots
    with pytest.raises(kvq.KvqError) as e:
        kvq.kvq_workspace_bytes(d, 32, 32768, 64)
    assert e.value.status == -9
    # float caches need the partials, then the zone where an 8/4-bit cache of
    # as many (sequence, KV head) pairs sharing the workspace keeps its ticket
    # counters (256 bytes for 4 pairs, 2 counters each), left untouched
    f = _desc(kvq, batch=2, n_kv_heads=2, capacity=1000, k_bits=16, v_bits=16)
    nc = -(-1000 // kvq.kvq_chunk_tokens(f, 8, 1000))
    fpart = ((16 * nc * 8 + 255) // 256) * 256 + 16 * nc * 128 * 4
    assert kvq.kvq_workspace_bytes(f, 8, 1000, 0) == (fpart + 255) // 256 * 256 + 256
    # max_seq_len beyond capacity sizes by capacity
    assert kvq.kvq_workspace_bytes(d, 32, 10 ** 9, 1024) == kvq.kvq_workspace_bytes(d, 32, 32768, 1024)
    # short contexts use the smallest chunk: 512 slots for integer caches, 64 for float ones
    small = _desc(kvq, batch=1, n_kv_heads=4, head_dim=64, capacity=257, group_size=64)
    assert kvq.kvq_chunk_tokens(small, 4, 257) == 512
    small_f = _desc(kvq, batch=1, n_kv_heads=4, head_dim=64, capacity=257, k_bits=16, v_bits=16)
    assert kvq.kvq_chunk_tokens(small_f, 4, 257) == 64
    # integer caches: the chunk is not bounded by LDS; the largest that gives
    # >= 1024 workgroups: 2048 at 32K for 256, 128 and 64 units, 1024 at 8K for
    # 128 units; contexts of at most 2048 slots that this would split in more
    # than two chunks take two at most (the one-launch decode step): 1024 for
    # a 1600-slot window over 256 units, 512 for 1K contexts
    assert kvq.kvq_chunk_tokens(d, 32, 32768) == 2048
    d8 = _desc(kvq, batch=16, n_kv_heads=8, capacity=32768, k_bits=8, v_bits=4)
    assert kvq.kvq_chunk_tokens(d8, 32, 32768) == 2048
    d4 = _desc(kvq, batch=8, n_kv_heads=8, capacity=32768, k_bits=8, v_bits=4)
    assert kvq.kvq_chunk_tokens(d4, 32, 32768) == 2048
    d8k = _desc(kvq, batch=16, n_kv_heads=8, capacity=8192, k_bits=8, v_bits=4)
    assert kvq.kvq_chunk_tokens(d8k, 32, 8192) == 1024
    win = _desc(kvq, batch=32, n_kv_heads=8, capacity=1600, k_bits=4, v_bits=4, n_anchor=64, window=1536)
    assert kvq.kvq_chunk_tokens(win, 32, 32768) == 1024
    assert kvq.kvq_chunk_count(win, 32, 32768) == 2
    tl = _desc(kvq, batch=8, n_kv_heads=16, capacity=1024)
    assert kvq.kvq_chunk_tokens(tl, 16, 1024) == 512
    assert kvq.kvq_chunk_count(tl, 16, 1024) == 2
    assert kvq.kvq_chunk_tokens(tl, 16, 600) == 512
    assert kvq.kvq_chunk_tokens(tl, 16, 512) == 512
    mid = _desc(kvq, batch=75, n_kv_heads=8, capacity=1024)     # 1200 workgroups of 512 slots fill the chip
    assert kvq.kvq_chunk_tokens(mid, 8, 1024) == 512
    big = _desc(kvq, batch=256, n_kv_heads=8, capacity=2048)    # 2048 workgroups of 2048 slots
    assert kvq.kvq_chunk_tokens(big, 8, 2048) == 2048
    # 32-value scale groups at G = 4 (57 KB of LDS): the same choice
    g32 = _desc(kvq, batch=32, n_kv_heads=8, capacity=32768, k_bits=4, v_bits=4, group_size=32)
    assert kvq.kvq_chunk_tokens(g32, 32, 32768) == 2048
    # float caches: at most 1024 slots (32K, 256 units), >= 2048 workgroups (8K, 128 units: 512)
    f32k = _desc(kvq, batch=32, n_kv_heads=8, capacity=32768, k_bits=16, v_bits=16)
    assert kvq.kvq_chunk_tokens(f32k, 32, 32768) == 1024
    f8k = _desc(kvq, batch=16, n_kv_heads=8, capacity=8192, k_bits=16, v_bits=16)
    assert kvq.kvq_chunk_tokens(f8k, 32, 8192) == 512


def test_chunk_count(kvq):
    d = _desc(kvq, batch=32, n_kv_heads=8, capacity=32768, k_bits=4, v_bits=4)
    assert kvq.kvq_chunk_count(d, 32, 32768) == 16
    assert kvq.kvq_chunk_count(d, 32, 32768, 1024) == 32
    assert kvq.kvq_chunk_count(d, 32, 30001, 1024) == 30
    assert kvq.kvq_chunk_count(d, 32, 10 ** 9, 4096) == 8          # L is capped by the capacity
    rng = np.random.default_rng(5)
    for _ in range(200):
        B, H = int(rng.integers(1, 65)), int(rng.choice([1, 2, 4, 8]))
        L = int(rng.integers(1, 65536))
        dd = _desc(kvq, batch=B, n_kv_heads=H, capacity=L, k_bits=int(rng.choice([4, 8, 16])), v_bits=4)
        if dd.k_bits == 16:
            dd.v_bits = 16
        ch = kvq.kvq_chunk_tokens(dd, H * 4, L)
        assert kvq.kvq_chunk_count(dd, H * 4, L) == -(-L // ch), (B, H, L, ch)
    with pytest.raises(kvq.KvqError):
        kvq.kvq_chunk_count(d, 32, 0)


def test_binding_has_no_fallback(kvq, monkeypatch, tmp_path):
    """With the library missing, the binding raises instead of computing."""
    import importlib
    mod = importlib.import_module("decode_attention_quantized_kvq_amd")
    monkeypatch.setattr(mod, "_lib", None)
    monkeypatch.setattr(mod, "LIB_PATH", tmp_path / "missing.so")
    with pytest.raises(RuntimeError):
        mod.kvq_bytes_per_token(8, 8, 16, 128, 128)


def test_product_does_not_touch_oracle():
    """The package and its sources never import or link the oracle."""
    pkg = ROOT / "decode_attention_quantized_kvq_amd"
    for f in list(pkg.rglob("*.py")) + list(pkg.rglob("*.hip")) + list(pkg.rglob("*.hpp")):
        text = f.read_text()
        assert "oracle" not in text.lower() or f.name == "__init__.py" and "import oracle" not in text, f
        assert "kvq_oracle" not in text and "import oracle" not in text and "from oracle" not in text, f


def test_static_step_rejects_oversize(kvq):
    """kvq_decode_step_static refuses a step whose workspace exceeds its static
    array, on the host, before any device call (the descriptor's buffers are
    never read)."""
    d = _desc(kvq, batch=64, n_kv_heads=8, capacity=131072, k_bits=16, v_bits=16)
    need = kvq.kvq_workspace_bytes(d, 32, 131072, 64)
    assert need > kvq.KVQ_STATIC_SCRATCH_BYTES
    with pytest.raises(kvq.KvqError) as e:
        kvq.kvq_decode_step_static(d, None, None, 1, None, None, 32, None, 131072, 0.0, 64, None, stream=0)
    assert e.value.status == kvq.KVQ_ERR_WORKSPACE
    assert "static scratch" in kvq.kvq_last_error()
    # the array's last 512 KiB are the ticket counters' zone: a step whose
    # other data would reach into it is refused although its whole need fits
    zone = 512 * 1024
    f = _desc(kvq, batch=32, n_kv_heads=8, capacity=63 * 64, k_bits=16, v_bits=16)
    need = kvq.kvq_workspace_bytes(f, 32, 63 * 64, 64)
    cnt = 2 * 32 * 8 * 4
    assert kvq.KVQ_STATIC_SCRATCH_BYTES - zone < need - cnt and need <= kvq.KVQ_STATIC_SCRATCH_BYTES
    with pytest.raises(kvq.KvqError) as e:
        kvq.kvq_decode_step_static(f, None, None, 1, None, None, 32, None, 63 * 64, 0.0, 64, None, stream=0)
    assert e.value.status == kvq.KVQ_ERR_WORKSPACE
    # (the zone holds two counters for each of the most (sequence, KV head)
    # pairs a cache may have: 65535 x 8 bytes)
    assert 65535 * 8 <= zone


def test_zero_point_rules(kvq):
    """The zero-point codec: 8/4-bit caches, contiguous or paged; its scale
    buffers hold 32-bit words (fp16 scale | zero point), twice the symmetric
    size, and must be 4-byte aligned."""
    d = _desc(kvq, batch=2, n_kv_heads=2, capacity=100, k_bits=4, v_bits=8, group_size=32)
    sym = kvq.kvq_cache_sizes(d)
    d.zero_point = 1
    zp = kvq.kvq_cache_sizes(d)
    assert zp[:2] == sym[:2] and zp[2] == 2 * sym[2] and zp[3] == 2 * sym[3]
    d.zero_point = 2
    with pytest.raises(kvq.KvqError) as e:
        kvq.kvq_cache_sizes(d)
    assert e.value.status == kvq.KVQ_ERR_ARG
    f = _desc(kvq, k_bits=16, v_bits=16)
    f.zero_point = 1
    with pytest.raises(kvq.KvqError) as e:
        kvq.kvq_cache_sizes(f)
    assert e.value.status == kvq.KVQ_ERR_BITS
    pg = _desc(kvq, capacity=128, k_bits=8, v_bits=4)
    pg.page_size, pg.n_pages, pg.block_table = 64, 5, 0x30000
    psym = kvq.kvq_cache_sizes(pg)
    pg.zero_point = 1
    pz = kvq.kvq_cache_sizes(pg)
    assert pz[:2] == psym[:2] and pz[2] == 2 * psym[2] == 5 * 2 * 64 * 4 and pz[3] == 2 * psym[3]
    ok = 0x30000
    c = _desc(kvq, k_bits=8, v_bits=8)
    c.zero_point = 1
    c.k_codes, c.v_codes, c.k_scales, c.v_scales = ok, ok, ok, ok + 2     # 2-byte aligned scale words
    with pytest.raises(kvq.KvqError) as e:
        kvq.kvq_append(c, ok, ok, 1, ok, 0)
    assert e.value.status == kvq.KVQ_ERR_ALIGN and "4-byte aligned" in kvq.kvq_last_error()


def test_header_is_c_and_links_from_c(kvq, tmp_path):
    """kvq.h compiles as strict C99 and a C program linked against libkvq.so
    calls the host-only entry points (no GPU work): TinyLoop's 4160 / 8192
    bytes per token, a cache's buffer sizes, the chunk rule, an error string."""
    import shutil
    import subprocess
    cc = shutil.which("gcc") or shutil.which("cc")
    if cc is None:
        pytest.skip("no C compiler")
    src = tmp_path / "abi.c"
    src.write_text(r"""
#include <stdio.h>
#include <string.h>
#include "kvq.h"
int main(void)
{
    kvq_cache c;
    size_t kc = 0, vc = 0, ks = 0, vs = 0;
    memset(&c, 0, sizeof c);
    c.batch = 2; c.n_kv_heads = 8; c.head_dim = 128; c.capacity = 1000;
    c.k_bits = 4; c.v_bits = 4; c.group_size = 128;
    if (kvq_cache_sizes(&c, &kc, &vc, &ks, &vs) != KVQ_OK) return 1;
    printf("%zu %zu\n", kvq_bytes_per_token(8, 8, 16, 128, 128), kvq_bytes_per_token(16, 16, 16, 128, 128));
    printf("%zu %zu %zu %zu\n", kc, vc, ks, vs);
    printf("%d %d\n", kvq_chunk_tokens(&c, 32, 1000), kvq_chunk_count(&c, 32, 1000, 0));
    c.head_dim = 96;
    printf("%d %s\n", kvq_cache_sizes(&c, NULL, NULL, NULL, NULL), kvq_status_str(KVQ_ERR_SHAPE));
    return 0;
}
""")
    exe = tmp_path / "abi"
    libdir = kvq.LIB_PATH.parent
    subprocess.run([cc, "-std=c99", "-Wall", "-Wextra", "-Werror", "-pedantic", f"-I{ROOT / 'include'}", str(src),
                    f"-L{libdir}", "-lkvq", f"-Wl,-rpath,{libdir}", "-o", str(exe)], check=True)
    out = subprocess.run([str(exe)], check=True, capture_output=True, text=True).stdout.split("\n")
    assert out[0].split() == ["4160", "8192"]
    cap64, cap4 = 1024, 1000
    assert [int(x) for x in out[1].split()] == [2 * 8 * cap64 * 64, 2 * 8 * cap4 * 64, 2 * 8 * 1000 * 2,
                                               2 * 8 * 1000 * 2]
    ch, n = (int(x) for x in out[2].split())
    assert ch == kvq.kvq_chunk_tokens(kvq.kvq_cache(2, 8, 128, 1000, 4, 4, 128, 0, 0), 32, 1000)
    assert n == (1000 + ch - 1) // ch
    st, msg = out[3].split(" ", 1)
    assert int(st) == kvq.KVQ_ERR_SHAPE and msg == kvq.kvq_status_str(kvq.KVQ_ERR_SHAPE)


def test_split_head_workspace(kvq):
    """Eight query heads per KV head with scale groups inside the head run as
    two workgroup heads of four: the query digits, scales, flags and ticket
    counters are laid out per (sequence, workgroup head), each block holding
    four heads' digits; one scale per head keeps one unit of eight."""
    a256 = lambda x: (x + 255) // 256 * 256

    def stride(G):                                   # int32 words of one unit's digits (int4 keys, HD 128)
        mf = 3 * G * 128 // 4 if G in (4, 8) else 0  # the matrix-core operand of four or eight heads
        return -(-(5 * 16 * G + 2 * 4 * G + mf) // 64) * 64

    def expect(B, Hkv, Hq, C, units, G):
        P = B * Hq
        off = a256(P * C * 8) + P * C * 128 * 4
        off = a256(off) + units * (C if C <= 2 else 1) * stride(G) * 4
        off = a256(off) + P * 4
        off = a256(off) + units * 4
        return a256(off) + a256(8 * B * Hkv)

    for group, split in ((32, True), (64, True), (128, False)):
        d = _desc(kvq, batch=4, n_kv_heads=8, capacity=32768, k_bits=4, v_bits=4, group_size=group)
        C = kvq.kvq_chunk_count(d, 64, 32768, 2048)
        assert C == 16
        want = expect(4, 8, 64, C, 4 * 8 * (2 if split else 1), 4 if split else 8)
        assert kvq.kvq_workspace_bytes(d, 64, 32768, 2048) == want, group


def test_split_head_limit(kvq):
    """G = 8 with scale groups runs two workgroup heads per KV head, so the
    split kernel's grid allows at most 32767 KV heads there (65535 otherwise)."""
    big = _desc(kvq, batch=1, n_kv_heads=40000, head_dim=128, capacity=256, k_bits=4, v_bits=4, group_size=32)
    assert kvq.kvq_chunk_count(big, 4 * 40000, 256, 0) == 1     # G = 4: one head per workgroup
    with pytest.raises(kvq.KvqError) as e:
        kvq.kvq_chunk_count(big, 8 * 40000, 256, 0)
    assert e.value.status == kvq.KVQ_ERR_SHAPE
    per_head = _desc(kvq, batch=1, n_kv_heads=40000, head_dim=128, capacity=256, k_bits=4, v_bits=4)
    assert kvq.kvq_chunk_count(per_head, 8 * 40000, 256, 0) == 1   # one scale per head: no split
