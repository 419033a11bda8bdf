"""CPU oracle for the quantized-KV decode path (ctypes wrapper over kvq_oracle.c).

TEST INFRASTRUCTURE ONLY.  The product library never imports, links or runs
anything in this package; only the tests, the smoke check and the bench's
CPU-baseline leg do.  The arithmetic lives in ``kvq_oracle.c`` (float64, one
loop per definition); this module only builds the shared object and moves
numpy arrays across the boundary.

Functions (each cites the page passage its C counterpart follows):

* ``f16_from_f32`` / ``f16_scale_from_f32`` / ``f16_to_f64``: IEEE binary16,
  nearest-even.  The pages name FP16 scales and an FP16 KV mode (TinyLoop
  "KV Cache 模式", five-modes table) without fixing a rounding; nearest-even is
  the reading taken.
* ``encode_row`` / ``decode_row``: symmetric per-group quantization with one
  fp16 scale per group and nibble packing (TinyLoop five-modes table, INT8 KV
  and INT4-h rows; KVSplit key/value bit widths).
* ``quantize_group_asym`` / ``encode_rows_asym`` / ``decode_row_asym``: the
  asymmetric codec, one fp16 scale and one integer zero point per group (the
  mni-ml page names scale/zero-point metadata; the min/max affine form with
  the range widened to contain zero is the reading taken).
* ``bytes_per_token``: TinyLoop memory-formula table; ``bytes_per_token_zp``
  the same with the asymmetric codec's metadata as this library stores it.
* ``slot_of`` / ``attended_positions``: on-device page, sliding-window
  eviction (64 anchors + 1536 recent).
* ``attend``: softmax attention of one query over the cached rows (mni-ml
  page, "how the KV cache creates speed"; aihot.vn: Q only at the current
  position).
* ``decode_step``: one decode step of one sequence from raw float32 rows.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from pathlib import Path

import numpy as np

_HERE = Path(__file__).resolve().parent
_SRC = _HERE / "kvq_oracle.c"
_LIB_PATH = _HERE / "libkvq_oracle.so"

# -ffp-contract=off: no fused multiply-add may change a rounding the oracle
# states; -fno-fast-math keeps IEEE division, rint and exp.
_CFLAGS = ["-O2", "-std=c11", "-fPIC", "-shared", "-ffp-contract=off", "-fno-fast-math"]


def build(force: bool = True) -> Path:
    """Compile kvq_oracle.c into libkvq_oracle.so with gcc."""
    if force or not _LIB_PATH.exists() or _LIB_PATH.stat().st_mtime < _SRC.stat().st_mtime:
        tmp = _LIB_PATH.with_suffix(".so.tmp")
        subprocess.run(["gcc", *_CFLAGS, str(_SRC), "-o", str(tmp), "-lm"], check=True)
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


_lib = None


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        if not _LIB_PATH.exists():
            build(force=False)
        L = ctypes.CDLL(str(_LIB_PATH))
        c_f = ctypes.c_float
        c_i = ctypes.c_int
        c_l = ctypes.c_long
        P = ctypes.c_void_p
        L.oq_f16_to_f64.argtypes = [ctypes.c_uint16]
        L.oq_f16_to_f64.restype = ctypes.c_double
        L.oq_f16_from_f32.argtypes = [c_f]
        L.oq_f16_from_f32.restype = ctypes.c_uint16
        L.oq_f16_scale_from_f32.argtypes = [c_f]
        L.oq_f16_scale_from_f32.restype = ctypes.c_uint16
        L.oq_qmax.argtypes = [c_i]
        L.oq_qmax.restype = c_i
        L.oq_quantize_group.argtypes = [P, c_i, c_i, P, P]
        L.oq_quantize_group.restype = None
        L.oq_pack_int4.argtypes = [P, c_i, P]
        L.oq_unpack_int4.argtypes = [P, c_i, P]
        L.oq_encode_row.argtypes = [P, c_i, c_i, c_i, P, P]
        L.oq_encode_row.restype = c_i
        L.oq_decode_row.argtypes = [P, P, c_i, c_i, c_i, P]
        L.oq_decode_row.restype = c_i
        L.oq_bytes_per_token.argtypes = [c_i, c_i, c_i, c_i, c_i]
        L.oq_bytes_per_token.restype = ctypes.c_size_t
        L.oq_slot_of.argtypes = [c_l, c_i, c_i]
        L.oq_slot_of.restype = c_l
        L.oq_attended_positions.argtypes = [c_l, c_i, c_i, P]
        L.oq_attended_positions.restype = c_l
        L.oq_attend.argtypes = [P, P, P, c_l, c_i, ctypes.c_double, P]
        L.oq_attend.restype = None
        L.oq_decode_step.argtypes = [c_i, c_i, c_i, c_i, c_i, c_i, c_i, P, P, c_l, P, c_i, c_i, c_i,
                                     ctypes.c_double, P]
        L.oq_decode_step.restype = c_i
        L.oq_levels.argtypes = [c_i]
        L.oq_levels.restype = c_i
        L.oq_quantize_group_asym.argtypes = [P, c_i, c_i, P, P, P]
        L.oq_quantize_group_asym.restype = None
        L.oq_encode_row_asym.argtypes = [P, c_i, c_i, c_i, P, P, P]
        L.oq_encode_row_asym.restype = c_i
        L.oq_decode_row_asym.argtypes = [P, P, P, c_i, c_i, c_i, P]
        L.oq_decode_row_asym.restype = c_i
        L.oq_bytes_per_token_zp.argtypes = [c_i, c_i, c_i, c_i, c_i, c_i]
        L.oq_bytes_per_token_zp.restype = ctypes.c_size_t
        L.oq_decode_step_zp.argtypes = [c_i, c_i, c_i, c_i, c_i, c_i, c_i, c_i, P, P, c_l, P, c_i, c_i, c_i,
                                        ctypes.c_double, P]
        L.oq_decode_step_zp.restype = c_i
        L.oq_f16_from_f32_n.argtypes = [P, ctypes.c_size_t, P]
        L.oq_f16_from_f32_n.restype = None
        L.oq_f16_to_f64_n.argtypes = [P, ctypes.c_size_t, P]
        L.oq_f16_to_f64_n.restype = None
        _lib = L
    return _lib


def _ptr(a: np.ndarray) -> int:
    assert a.flags["C_CONTIGUOUS"]
    return a.ctypes.data


# ---------------------------------------------------------------- fp16
def f16_from_f32(x) -> np.ndarray:
    """binary16 bit patterns (uint16) of float32 values, nearest-even."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    out = np.empty(x.shape, dtype=np.uint16)
    lib().oq_f16_from_f32_n(_ptr(x), x.size, _ptr(out))
    return out


def f16_scale_from_f32(x) -> np.ndarray:
    x = np.ascontiguousarray(x, dtype=np.float32)
    f = lib().oq_f16_scale_from_f32
    return np.array([f(float(v)) for v in x.ravel()], dtype=np.uint16).reshape(x.shape)


def f16_to_f64(h) -> np.ndarray:
    h = np.ascontiguousarray(h, dtype=np.uint16)
    out = np.empty(h.shape, dtype=np.float64)
    lib().oq_f16_to_f64_n(_ptr(h), h.size, _ptr(out))
    return out


# ---------------------------------------------------------------- codec
def qmax(bits: int) -> int:
    return int(lib().oq_qmax(bits))


def quantize_group(x, qm: int) -> tuple[np.ndarray, int]:
    """(codes int8[g], scale bit pattern) of one group at qmax = qm."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    codes = np.zeros(x.size, dtype=np.int8)
    sb = np.zeros(1, dtype=np.uint16)
    lib().oq_quantize_group(_ptr(x), x.size, qm, _ptr(codes), _ptr(sb))
    return codes, int(sb[0])


def pack_int4(codes) -> np.ndarray:
    c = np.ascontiguousarray(codes, dtype=np.int8)
    out = np.zeros(c.size // 2, dtype=np.uint8)
    lib().oq_pack_int4(_ptr(c), c.size, _ptr(out))
    return out


def unpack_int4(packed, n: int) -> np.ndarray:
    p = np.ascontiguousarray(packed, dtype=np.uint8)
    out = np.zeros(n, dtype=np.int8)
    lib().oq_unpack_int4(_ptr(p), n, _ptr(out))
    return out


def encode_row(x, g: int, bits: int) -> tuple[np.ndarray, np.ndarray]:
    """Stored form of one row: (payload uint8[n*bits/8], scales uint16[n/g] or empty)."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    n = x.size
    payload = np.zeros(n * bits // 8, dtype=np.uint8)
    nsc = n // g if (bits < 16 and g > 0) else 0
    scales = np.zeros(max(nsc, 1), dtype=np.uint16)
    rc = lib().oq_encode_row(_ptr(x), n, g, bits, _ptr(payload), _ptr(scales))
    if rc != 0:
        raise ValueError(f"encode_row: bad arguments n={n} g={g} bits={bits}")
    return payload, scales[:nsc]


def encode_rows(x, g: int, bits: int) -> tuple[np.ndarray, np.ndarray]:
    """encode_row over the last axis of x (any leading shape)."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    lead = x.shape[:-1]
    n = x.shape[-1]
    flat = x.reshape(-1, n)
    nsc = n // g if bits < 16 else 0
    P = np.zeros((flat.shape[0], n * bits // 8), dtype=np.uint8)
    S = np.zeros((flat.shape[0], max(nsc, 1)), dtype=np.uint16)
    f = lib().oq_encode_row
    for i in range(flat.shape[0]):
        rc = f(_ptr(flat[i]), n, g, bits, P[i].ctypes.data, S[i].ctypes.data)
        if rc != 0:
            raise ValueError("encode_rows: bad arguments")
    return P.reshape(*lead, n * bits // 8), S[:, :nsc].reshape(*lead, nsc)


def decode_row(payload, scales, n: int, g: int, bits: int) -> np.ndarray:
    p = np.ascontiguousarray(payload, dtype=np.uint8)
    s = np.ascontiguousarray(scales if scales is not None and np.size(scales) else np.zeros(1), dtype=np.uint16)
    out = np.zeros(n, dtype=np.float64)
    rc = lib().oq_decode_row(_ptr(p), _ptr(s), n, g, bits, _ptr(out))
    if rc != 0:
        raise ValueError("decode_row: bad arguments")
    return out


def levels(bits: int) -> int:
    return int(lib().oq_levels(bits))


def quantize_group_asym(x, L: int) -> tuple[np.ndarray, int, int]:
    """(codes uint8[g] in [0, L], scale bit pattern, zero point) of one group."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    codes = np.zeros(x.size, dtype=np.uint8)
    sb = np.zeros(1, dtype=np.uint16)
    zp = np.zeros(1, dtype=np.uint8)
    lib().oq_quantize_group_asym(_ptr(x), x.size, L, _ptr(codes), _ptr(sb), _ptr(zp))
    return codes, int(sb[0]), int(zp[0])


def encode_rows_asym(x, g: int, bits: int) -> tuple[np.ndarray, np.ndarray, np.ndarray]:
    """The asymmetric codec over the last axis of x (any leading shape):
    (payload uint8[..., n*bits/8], scales uint16[..., n/g], zeros uint8[..., n/g])."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    lead, n = x.shape[:-1], x.shape[-1]
    flat = x.reshape(-1, n)
    P = np.zeros((flat.shape[0], n * bits // 8), dtype=np.uint8)
    S = np.zeros((flat.shape[0], n // g), dtype=np.uint16)
    Z = np.zeros((flat.shape[0], n // g), dtype=np.uint8)
    f = lib().oq_encode_row_asym
    for i in range(flat.shape[0]):
        if f(_ptr(flat[i]), n, g, bits, P[i].ctypes.data, S[i].ctypes.data, Z[i].ctypes.data) != 0:
            raise ValueError("encode_rows_asym: bad arguments")
    return P.reshape(*lead, -1), S.reshape(*lead, -1), Z.reshape(*lead, -1)


def decode_row_asym(payload, scales, zeros, n: int, g: int, bits: int) -> np.ndarray:
    p = np.ascontiguousarray(payload, dtype=np.uint8)
    s = np.ascontiguousarray(scales, dtype=np.uint16)
    z = np.ascontiguousarray(zeros, dtype=np.uint8)
    out = np.zeros(n, dtype=np.float64)
    if lib().oq_decode_row_asym(_ptr(p), _ptr(s), _ptr(z), n, g, bits, _ptr(out)) != 0:
        raise ValueError("decode_row_asym: bad arguments")
    return out


# ---------------------------------------------------------------- accounting / window
def bytes_per_token(k_bits: int, v_bits: int, n_kv_heads: int, head_dim: int, group_size: int) -> int:
    return int(lib().oq_bytes_per_token(k_bits, v_bits, n_kv_heads, head_dim, group_size))


def bytes_per_token_zp(k_bits: int, v_bits: int, n_kv_heads: int, head_dim: int, group_size: int,
                       asym: int) -> int:
    return int(lib().oq_bytes_per_token_zp(k_bits, v_bits, n_kv_heads, head_dim, group_size, asym))


def slot_of(pos: int, n_anchor: int, window: int) -> int:
    return int(lib().oq_slot_of(pos, n_anchor, window))


def attended_positions(t: int, n_anchor: int, window: int) -> np.ndarray:
    out = np.zeros(t + 1, dtype=np.int64)
    n = lib().oq_attended_positions(t, n_anchor, window, _ptr(out))
    return out[:n].copy()


# ---------------------------------------------------------------- attention
def attend(q, K, V, scale: float) -> np.ndarray:
    q = np.ascontiguousarray(q, dtype=np.float64)
    K = np.ascontiguousarray(K, dtype=np.float64)
    V = np.ascontiguousarray(V, dtype=np.float64)
    n, hd = K.shape
    out = np.zeros(hd, dtype=np.float64)
    lib().oq_attend(_ptr(q), _ptr(K), _ptr(V), n, hd, float(scale), _ptr(out))
    return out


def decode_step(k_bits: int, v_bits: int, group_size: int, n_anchor: int, window: int,
                k_src, v_src, q, softmax_scale: float, hq_begin: int = 0, hq_end: int | None = None,
                asym: bool = False) -> np.ndarray:
    """One decode step of one sequence.

    k_src, v_src: float32 [n_kv_heads][n_pos][head_dim]; q: float32 [n_q_heads][head_dim].
    asym: the 8/4-bit sides use the asymmetric (zero-point) codec.
    Returns float64 [hq_end-hq_begin][head_dim].
    """
    k_src = np.ascontiguousarray(k_src, dtype=np.float32)
    v_src = np.ascontiguousarray(v_src, dtype=np.float32)
    q = np.ascontiguousarray(q, dtype=np.float32)
    hkv, n_pos, hd = k_src.shape
    hq = q.shape[0]
    if hq_end is None:
        hq_end = hq
    out = np.zeros((hq_end - hq_begin, hd), dtype=np.float64)
    rc = lib().oq_decode_step_zp(k_bits, v_bits, group_size, 1 if asym else 0, hkv, hd, n_anchor, window,
                                 _ptr(k_src), _ptr(v_src), n_pos, _ptr(q), hq, hq_begin, hq_end,
                                 float(softmax_scale), _ptr(out))
    if rc != 0:
        raise ValueError("decode_step: bad arguments")
    return out
