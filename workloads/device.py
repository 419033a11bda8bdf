"""Device-side harness helpers: upload the seeded workload draws and append
them to caches through the library's own kvq_append.

No arithmetic of the method lives here; it only moves the arrays that
``workloads`` draws into device memory and calls the C ABI.
"""
from __future__ import annotations

import numpy as np
import torch

import decode_attention_quantized_kvq_amd as kvq

from . import K_STREAM, V_STREAM, Workload, batch_query, rows


def to_device(x: np.ndarray, device="cuda") -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(x)).to(device, non_blocking=False)


def positions(values, device="cuda") -> torch.Tensor:
    return torch.tensor(list(values), dtype=torch.int32, device=device)


def fill(caches: list, w: Workload, layer: int, n_pos: int, piece: int = 8192, device="cuda"):
    """Append positions 0 .. n_pos-1 of every sequence of `layer` to each
    cache in `caches` (same draws for all): one sequence per call, the
    context in calls of at most `piece` positions, and the newest position
    (the decode step's row) in a call of its own.

    Returns the newest rows as device tensors (k, v), each
    [batch][n_kv_heads][1][head_dim]."""
    last_k, last_v = [], []
    for b in range(w.batch):
        seq = [c.sequence(b) for c in caches]
        k = to_device(rows(w, K_STREAM, layer, b, n_pos)[None], device)    # [1][Hkv][n_pos][HD]
        v = to_device(rows(w, V_STREAM, layer, b, n_pos)[None], device)
        segments = [(p0, min(piece, n_pos - 1 - p0)) for p0 in range(0, n_pos - 1, piece)] + [(n_pos - 1, 1)]
        for p0, n in segments:
            kk = k[:, :, p0:p0 + n].contiguous()
            vv = v[:, :, p0:p0 + n].contiguous()
            sp = positions([p0], device)
            for c in seq:
                kvq.kvq_append(c, kk, vv, n, sp)
        last_k.append(kk)
        last_v.append(vv)
        del k, v
    torch.cuda.synchronize()
    return torch.cat(last_k), torch.cat(last_v)


def queries(w: Workload, layer: int, step: int = 0, device="cuda") -> torch.Tensor:
    return to_device(batch_query(w, layer, step), device)


def decode(cache, q: torch.Tensor, n_q_heads: int, seq_len: torch.Tensor, max_seq_len: int,
           softmax_scale: float = 0.0, chunk_tokens: int = 0) -> torch.Tensor:
    """Allocate workspace and output with torch and run kvq_decode_attn."""
    ws_bytes = kvq.kvq_workspace_bytes(cache, n_q_heads, max_seq_len, chunk_tokens)
    ws = torch.empty(ws_bytes // 4 + 64, dtype=torch.float32, device=q.device)
    out = torch.empty_like(q)
    kvq.kvq_decode_attn(cache, q, n_q_heads, seq_len, max_seq_len, softmax_scale, chunk_tokens, out, ws, ws_bytes)
    return out
