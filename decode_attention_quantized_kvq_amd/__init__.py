"""Python binding of libkvq.so: the quantized-KV append and decode-attention C ABI.

Every function here has the name and arguments of its C entry point in
``include/kvq.h`` and only marshals arguments (torch tensors -> device
pointers, status codes -> exceptions); every step of the computation runs in
the library's HIP kernels.  There is no fallback: if ``libkvq.so`` has not
been built, importing the functions raises.

PyTorch is used for device memory and streams only (``alloc_cache`` below
allocates the cache buffers as torch tensors).
"""
from __future__ import annotations

import ctypes
import math
from dataclasses import dataclass, field
from pathlib import Path
from typing import Any

_PKG = Path(__file__).resolve().parent
LIB_PATH = _PKG / "libkvq.so"

KVQ_OK = 0
KVQ_ERR_NULL = -1
KVQ_ERR_BITS = -2
KVQ_ERR_SHAPE = -3
KVQ_ERR_GROUP = -4
KVQ_ERR_WINDOW = -5
KVQ_ERR_WORKSPACE = -6
KVQ_ERR_ALIGN = -7
KVQ_ERR_HIP = -8
KVQ_ERR_ARG = -9

EXPORTED = (
    "kvq_bytes_per_token", "kvq_cache_sizes", "kvq_append", "kvq_chunk_tokens", "kvq_chunk_count",
    "kvq_workspace_bytes",
    "kvq_decode_partials", "kvq_prepare_query", "kvq_decode_partials_prepared", "kvq_combine", "kvq_decode_attn",
    "kvq_decode_step", "kvq_decode_step_static", "kvq_read_probe", "kvq_status_str", "kvq_last_error",
)
KVQ_STATIC_SCRATCH_BYTES = 32 << 20


class KvqError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"kvq error {status}: {message}")
        self.status = status


class kvq_cache(ctypes.Structure):
    """Mirror of the C struct kvq_cache (see include/kvq.h)."""
    _fields_ = [
        ("batch", ctypes.c_int32),
        ("n_kv_heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
        ("capacity", ctypes.c_int32),
        ("k_bits", ctypes.c_int32),
        ("v_bits", ctypes.c_int32),
        ("group_size", ctypes.c_int32),
        ("n_anchor", ctypes.c_int32),
        ("window", ctypes.c_int32),
        ("k_codes", ctypes.c_void_p),
        ("v_codes", ctypes.c_void_p),
        ("k_scales", ctypes.c_void_p),
        ("v_scales", ctypes.c_void_p),
        ("page_size", ctypes.c_int32),
        ("n_pages", ctypes.c_int32),
        ("block_table", ctypes.c_void_p),
        ("zero_point", ctypes.c_int32),
    ]


_lib = None


def lib() -> ctypes.CDLL:
    """Load libkvq.so (built in-tree); raise if it is missing."""
    global _lib
    if _lib is None:
        if not LIB_PATH.exists():
            raise RuntimeError(f"{LIB_PATH} is not built: run `python -m decode_attention_quantized_kvq_amd.build`")
        L = ctypes.CDLL(str(LIB_PATH))
        P = ctypes.c_void_p
        I = ctypes.c_int
        S = ctypes.c_size_t
        C = ctypes.POINTER(kvq_cache)
        L.kvq_bytes_per_token.argtypes = [I, I, I, I, I]
        L.kvq_bytes_per_token.restype = S
        L.kvq_cache_sizes.argtypes = [C, ctypes.POINTER(S), ctypes.POINTER(S), ctypes.POINTER(S), ctypes.POINTER(S)]
        L.kvq_cache_sizes.restype = I
        L.kvq_append.argtypes = [C, P, P, I, P, P]
        L.kvq_append.restype = I
        L.kvq_chunk_tokens.argtypes = [C, I, I]
        L.kvq_chunk_tokens.restype = I
        L.kvq_chunk_count.argtypes = [C, I, I, I]
        L.kvq_chunk_count.restype = I
        L.kvq_workspace_bytes.argtypes = [C, I, I, I]
        L.kvq_workspace_bytes.restype = S
        L.kvq_decode_partials.argtypes = [C, P, I, P, I, ctypes.c_float, I, P, S, P]
        L.kvq_decode_partials.restype = I
        L.kvq_prepare_query.argtypes = [C, P, I, I, ctypes.c_float, I, P, S, P]
        L.kvq_prepare_query.restype = I
        L.kvq_decode_partials_prepared.argtypes = [C, I, P, I, I, P, S, P]
        L.kvq_decode_partials_prepared.restype = I
        L.kvq_combine.argtypes = [I, I, I, I, P, S, P, P]
        L.kvq_combine.restype = I
        L.kvq_decode_attn.argtypes = [C, P, I, P, I, ctypes.c_float, I, P, P, S, P]
        L.kvq_decode_attn.restype = I
        L.kvq_decode_step.argtypes = [C, P, P, I, P, P, I, P, I, ctypes.c_float, I, P, P, S, P]
        L.kvq_decode_step.restype = I
        L.kvq_decode_step_static.argtypes = [C, P, P, I, P, P, I, P, I, ctypes.c_float, I, P, P]
        L.kvq_decode_step_static.restype = I
        L.kvq_read_probe.argtypes = [P, S, P, S, P]
        L.kvq_read_probe.restype = I
        L.kvq_status_str.argtypes = [I]
        L.kvq_status_str.restype = ctypes.c_char_p
        L.kvq_last_error.argtypes = []
        L.kvq_last_error.restype = ctypes.c_char_p
        _lib = L
    return _lib


# ---------------------------------------------------------------- marshalling
def _ptr(x) -> int | None:
    """Device pointer of a torch tensor, or an int / None passed through."""
    if x is None:
        return None
    if isinstance(x, int):
        return x
    return x.data_ptr()


def _stream(stream) -> int | None:
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream if torch.cuda.is_available() else None
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _check(status: int) -> int:
    if status < 0:
        raise KvqError(status, f"{kvq_status_str(status)}: {kvq_last_error()}")
    return status


def _desc(cache) -> kvq_cache:
    return cache.desc if isinstance(cache, Cache) else cache


# ---------------------------------------------------------------- the C ABI
def kvq_bytes_per_token(k_bits: int, v_bits: int, n_kv_heads: int, head_dim: int, group_size: int) -> int:
    return int(lib().kvq_bytes_per_token(k_bits, v_bits, n_kv_heads, head_dim, group_size))


def kvq_cache_sizes(cache) -> tuple[int, int, int, int]:
    out = [ctypes.c_size_t(0) for _ in range(4)]
    _check(lib().kvq_cache_sizes(ctypes.byref(_desc(cache)), *[ctypes.byref(o) for o in out]))
    return tuple(int(o.value) for o in out)


def kvq_append(cache, k_new, v_new, n_new: int, start_pos, stream=None) -> None:
    _check(lib().kvq_append(ctypes.byref(_desc(cache)), _ptr(k_new), _ptr(v_new), int(n_new), _ptr(start_pos),
                            _stream(stream)))


def kvq_chunk_tokens(cache, n_q_heads: int, max_seq_len: int) -> int:
    return _check(lib().kvq_chunk_tokens(ctypes.byref(_desc(cache)), n_q_heads, max_seq_len))


def kvq_chunk_count(cache, n_q_heads: int, max_seq_len: int, chunk_tokens: int = 0) -> int:
    return _check(lib().kvq_chunk_count(ctypes.byref(_desc(cache)), n_q_heads, max_seq_len, chunk_tokens))


def kvq_workspace_bytes(cache, n_q_heads: int, max_seq_len: int, chunk_tokens: int = 0) -> int:
    n = int(lib().kvq_workspace_bytes(ctypes.byref(_desc(cache)), n_q_heads, max_seq_len, chunk_tokens))
    if n == 0:
        raise KvqError(KVQ_ERR_ARG, kvq_last_error())
    return n


def kvq_decode_partials(cache, q, n_q_heads: int, seq_len, max_seq_len: int, softmax_scale: float,
                        chunk_tokens: int, workspace, workspace_bytes: int, stream=None) -> None:
    _check(lib().kvq_decode_partials(ctypes.byref(_desc(cache)), _ptr(q), n_q_heads, _ptr(seq_len), max_seq_len,
                                     float(softmax_scale), chunk_tokens, _ptr(workspace), int(workspace_bytes),
                                     _stream(stream)))


def kvq_prepare_query(cache, q, n_q_heads: int, max_seq_len: int, softmax_scale: float, chunk_tokens: int,
                      workspace, workspace_bytes: int, stream=None) -> None:
    _check(lib().kvq_prepare_query(ctypes.byref(_desc(cache)), _ptr(q), n_q_heads, max_seq_len, float(softmax_scale),
                                   chunk_tokens, _ptr(workspace), int(workspace_bytes), _stream(stream)))


def kvq_decode_partials_prepared(cache, n_q_heads: int, seq_len, max_seq_len: int, chunk_tokens: int, workspace,
                                 workspace_bytes: int, stream=None) -> None:
    _check(lib().kvq_decode_partials_prepared(ctypes.byref(_desc(cache)), n_q_heads, _ptr(seq_len), max_seq_len,
                                              chunk_tokens, _ptr(workspace), int(workspace_bytes), _stream(stream)))


def kvq_combine(batch: int, n_q_heads: int, head_dim: int, n_chunks: int, workspace, workspace_bytes: int, out,
                stream=None) -> None:
    _check(lib().kvq_combine(batch, n_q_heads, head_dim, n_chunks, _ptr(workspace), int(workspace_bytes), _ptr(out),
                             _stream(stream)))


def kvq_decode_attn(cache, q, n_q_heads: int, seq_len, max_seq_len: int, softmax_scale: float, chunk_tokens: int,
                    out, workspace, workspace_bytes: int, stream=None) -> None:
    _check(lib().kvq_decode_attn(ctypes.byref(_desc(cache)), _ptr(q), n_q_heads, _ptr(seq_len), max_seq_len,
                                 float(softmax_scale), chunk_tokens, _ptr(out), _ptr(workspace), int(workspace_bytes),
                                 _stream(stream)))


def kvq_decode_step(cache, k_new, v_new, n_new: int, start_pos, q, n_q_heads: int, seq_len, max_seq_len: int,
                    softmax_scale: float, chunk_tokens: int, out, workspace, workspace_bytes: int,
                    stream=None) -> None:
    _check(lib().kvq_decode_step(ctypes.byref(_desc(cache)), _ptr(k_new), _ptr(v_new), int(n_new), _ptr(start_pos),
                                 _ptr(q), n_q_heads, _ptr(seq_len), max_seq_len, float(softmax_scale), chunk_tokens,
                                 _ptr(out), _ptr(workspace), int(workspace_bytes), _stream(stream)))


def kvq_decode_step_static(cache, k_new, v_new, n_new: int, start_pos, q, n_q_heads: int, seq_len,
                           max_seq_len: int, softmax_scale: float, chunk_tokens: int, out, stream=None) -> None:
    _check(lib().kvq_decode_step_static(ctypes.byref(_desc(cache)), _ptr(k_new), _ptr(v_new), int(n_new),
                                        _ptr(start_pos), _ptr(q), n_q_heads, _ptr(seq_len), max_seq_len,
                                        float(softmax_scale), chunk_tokens, _ptr(out), _stream(stream)))


def kvq_read_probe(buf, nbytes: int, sink, sink_bytes: int, stream=None) -> None:
    _check(lib().kvq_read_probe(_ptr(buf), int(nbytes), _ptr(sink), int(sink_bytes), _stream(stream)))


def kvq_status_str(status: int) -> str:
    return lib().kvq_status_str(status).decode()


def kvq_last_error() -> str:
    return lib().kvq_last_error().decode()


# ---------------------------------------------------------------- device memory
@dataclass
class Cache:
    """A kvq_cache descriptor plus the torch tensors that own its buffers."""
    desc: kvq_cache
    k_codes: Any
    v_codes: Any
    k_scales: Any = None
    v_scales: Any = None
    keep: list = field(default_factory=list)

    @property
    def batch(self) -> int:
        return self.desc.batch

    def sequence(self, b: int) -> "Cache":
        """Descriptor of sequence b alone (batch 1), sharing the buffers.  A
        paged cache keeps its pools and points at row b of the block table."""
        d = kvq_cache.from_buffer_copy(self.desc)
        d.batch = 1
        if d.page_size:
            d.block_table = self.desc.block_table + 4 * b * (d.capacity // d.page_size)
            return Cache(d, self.k_codes, self.v_codes, self.k_scales, self.v_scales, keep=[self])
        per_seq = lambda t: None if t is None else t.view(self.desc.batch, -1)[b]
        kc, vc, ks, vs = (per_seq(t) for t in (self.k_codes, self.v_codes, self.k_scales, self.v_scales))
        d.k_codes, d.v_codes = kc.data_ptr(), vc.data_ptr()
        d.k_scales = ks.data_ptr() if ks is not None else None
        d.v_scales = vs.data_ptr() if vs is not None else None
        return Cache(d, kc, vc, ks, vs, keep=[self])


def alloc_cache(batch: int, n_kv_heads: int, head_dim: int, capacity: int, k_bits: int, v_bits: int,
                group_size: int = 0, n_anchor: int = 0, window: int = 0, device="cuda",
                page_size: int = 0, n_pages: int = 0, block_table=None, zero_point: int = 0) -> Cache:
    """Allocate the four cache buffers with torch (zero-filled) and describe them.

    group_size 0 means one scale per head (group_size = head_dim).  page_size > 0
    allocates pools of n_pages pages of page_size slots instead of one region per
    sequence; block_table is then an int32 device tensor of batch x
    (capacity / page_size) page indices, kept alive by the returned Cache.
    zero_point 1 selects the zero-point codec (scale buffers of 32-bit words)."""
    import torch
    d = kvq_cache(batch, n_kv_heads, head_dim, capacity, k_bits, v_bits, group_size or head_dim, n_anchor, window,
                  None, None, None, None, page_size, n_pages, None, zero_point)
    keep = []
    if page_size:
        if block_table is None:
            raise ValueError("a paged cache needs a block table")
        if block_table.dtype != torch.int32 or not block_table.is_contiguous():
            raise ValueError("block_table must be a contiguous int32 tensor")
        d.block_table = block_table.data_ptr()
        keep.append(block_table)
    kc, vc, ks, vs = kvq_cache_sizes(d)
    k_codes = torch.zeros(max(kc, 16), dtype=torch.uint8, device=device)
    v_codes = torch.zeros(max(vc, 16), dtype=torch.uint8, device=device)
    k_scales = torch.zeros(ks // 2, dtype=torch.int16, device=device) if ks else None
    v_scales = torch.zeros(vs // 2, dtype=torch.int16, device=device) if vs else None
    d.k_codes, d.v_codes = k_codes.data_ptr(), v_codes.data_ptr()
    d.k_scales = k_scales.data_ptr() if k_scales is not None else None
    d.v_scales = v_scales.data_ptr() if v_scales is not None else None
    return Cache(d, k_codes, v_codes, k_scales, v_scales, keep=keep)


def default_scale(head_dim: int) -> float:
    return 1.0 / math.sqrt(head_dim)
