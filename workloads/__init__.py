"""Seeded synthetic workloads shared by the tests, the bench and the oracle checks.

This module draws random inputs and describes shapes.  It holds none of the
method's arithmetic (no quantization, no attention): both the HIP path and the
CPU oracle receive exactly the arrays produced here.

Every random array comes from ``numpy.random.default_rng([seed, stream,
layer, b, step])`` (PCG64 seeded through SeedSequence), so any slice can be
regenerated on its own.  Streams: 0 = K rows, 1 = V rows, 2 = queries,
3 = the choice of outlier key channels.  Rows are drawn position-major, so the
first n positions of a sequence do not depend on how many are drawn.

The five workloads stand in for the pages' models (none of their weights or
datasets are used): they take the shapes the pages describe, with N(0, 1)
activations and, where a workload says so, a few key channels scaled up as
outliers.
"""
from __future__ import annotations

from dataclasses import dataclass, field, replace

import numpy as np

K_STREAM, V_STREAM, Q_STREAM, OUTLIER_STREAM = 0, 1, 2, 3


@dataclass(frozen=True)
class Mode:
    """One cache precision: key bits, value bits, elements per fp16 scale.

    bits 32 = float32 rows, 16 = fp16 rows, 8 / 4 = symmetric codes with one
    fp16 scale per ``group`` elements (ignored for 16/32-bit sides).
    ``group = 0`` means one scale per head (group = head_dim); ``group = -1``
    means one scale per position row across all KV heads.  ``zero_point``:
    the asymmetric codec (an fp16 scale and an integer zero point per group).
    """
    name: str
    k_bits: int
    v_bits: int
    group: int = 0
    zero_point: bool = False

    def group_size(self, n_kv_heads: int, head_dim: int) -> int:
        if self.group == 0:
            return head_dim
        if self.group == -1:
            return n_kv_heads * head_dim
        return self.group


FP32 = Mode("fp32", 32, 32)
FP16 = Mode("fp16", 16, 16)
K8V8 = Mode("k8v8", 8, 8)
K8V4 = Mode("k8v4", 8, 4)
K4V4 = Mode("k4v4", 4, 4)
K4V8 = Mode("k4v8", 4, 8)
K8V8_ROW = Mode("k8v8-row", 8, 8, -1)
K4V4_G32 = Mode("k4v4-g32", 4, 4, 32)      # one scale per 32 codes (KVSplit's footprint ratios)
K4V4_ZP = Mode("k4v4-zp", 4, 4, 0, True)   # per-head scale and zero point


@dataclass(frozen=True)
class Workload:
    name: str
    batch: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    n_layers: int
    capacity: int          # slots per (sequence, KV head)
    n_pos: int             # positions written once the step's row is appended
    modes: tuple = ()
    n_anchor: int = 0
    window: int = 0
    outlier_frac: float = 0.0
    outlier_scale: float = 1.0
    seed: int = 1000
    prompt: int = 0        # > 0: a prompt of this many rows, then one row per step
    note: str = ""

    @property
    def group_q(self) -> int:
        return self.n_q_heads // self.n_kv_heads

    def with_(self, **kw) -> "Workload":
        return replace(self, **kw)


# The five workloads.  Shapes follow the pages' descriptions; sizes the
# pages leave open are stated in `note`.
TINY = Workload(
    "tiny", batch=1, n_q_heads=4, n_kv_heads=4, head_dim=64, n_layers=1,
    capacity=257, n_pos=257, modes=(K8V8, FP16), seed=1001,
    note="256 cached tokens + the appended one; per-token-per-head fp16 scales")

MNIML = Workload(
    "mniml", batch=1, n_q_heads=8, n_kv_heads=8, head_dim=64, n_layers=1,
    capacity=256, n_pos=256, modes=(K8V8_ROW, FP32, K8V8), seed=1002, prompt=4,
    note="4-token prompt then 252 decode steps (append + attend each step); "
         "int8 with one scale per position row vs a float32 cache")

TINYLOOP = Workload(
    "tinyloop", batch=8, n_q_heads=16, n_kv_heads=16, head_dim=128, n_layers=34,
    capacity=1024, n_pos=1024, modes=(K8V8, FP16), seed=1003,
    outlier_frac=0.01, outlier_scale=8.0,
    note="D = 2048 = 16 x 128, 34 layers, max_seq_len 1024; 1% of key channels x8")

K8V4_8K = Workload(
    "k8v4-8k", batch=16, n_q_heads=32, n_kv_heads=8, head_dim=128, n_layers=1,
    capacity=8192, n_pos=8192, modes=(K8V4, FP16, K8V8, K4V4), seed=1004,
    outlier_frac=0.02, outlier_scale=10.0,
    note="GQA 4:1; 2% of key channels x10; values N(0,1)")

K8V4_32K = K8V4_8K.with_(name="k8v4-32k", capacity=32768, n_pos=32768, modes=(K8V4,),
                         note="the 8K workload at 32K context")

K4V4_32K = Workload(
    "k4v4-32k", batch=32, n_q_heads=32, n_kv_heads=8, head_dim=128, n_layers=1,
    capacity=32768, n_pos=32768, modes=(K4V4, FP16), seed=1005,
    note="nibble-packed int4 K and V, full 32K context")

K4V4_WINDOW = K4V4_32K.with_(
    name="k4v4-window", capacity=64 + 1536, n_anchor=64, window=1536, modes=(K4V4,),
    note="64 anchor + 1536 recent tokens of a 32K-token sequence, ring storage")

WORKLOADS = {w.name: w for w in (TINY, MNIML, TINYLOOP, K8V4_8K, K8V4_32K, K4V4_32K, K4V4_WINDOW)}


# ------------------------------------------------------------------ draws
def _rng(w: Workload, stream: int, layer: int, b: int, step: int = 0) -> np.random.Generator:
    return np.random.default_rng([w.seed, stream, layer, b, step])


def outlier_channels(w: Workload) -> np.ndarray:
    """Flat (kv_head * head_dim + channel) indices of the scaled key channels.

    round(frac * n_kv_heads * head_dim) channels, drawn without replacement,
    fixed across positions, sequences and layers."""
    n = int(round(w.outlier_frac * w.n_kv_heads * w.head_dim))
    if n == 0:
        return np.zeros(0, dtype=np.int64)
    rng = np.random.default_rng([w.seed, OUTLIER_STREAM])
    return np.sort(rng.choice(w.n_kv_heads * w.head_dim, size=n, replace=False))


def rows(w: Workload, stream: int, layer: int, b: int, n_pos: int, start: int = 0) -> np.ndarray:
    """float32 [n_kv_heads][n_pos][head_dim]: the K (stream 0) or V (stream 1)
    rows of positions start .. start+n_pos-1 of sequence b in `layer`."""
    rng = _rng(w, stream, layer, b)
    total = start + n_pos
    x = rng.standard_normal((total, w.n_kv_heads, w.head_dim), dtype=np.float32)[start:]
    if stream == K_STREAM and w.outlier_frac > 0:
        flat = x.reshape(n_pos, w.n_kv_heads * w.head_dim)
        flat[:, outlier_channels(w)] *= np.float32(w.outlier_scale)
    return np.ascontiguousarray(x.transpose(1, 0, 2))


def query(w: Workload, layer: int, b: int, step: int = 0) -> np.ndarray:
    """float32 [n_q_heads][head_dim]: the query of sequence b at a decode step."""
    rng = _rng(w, Q_STREAM, layer, b, step)
    return rng.standard_normal((w.n_q_heads, w.head_dim), dtype=np.float32)


def batch_rows(w: Workload, stream: int, layer: int, n_pos: int, start: int = 0) -> np.ndarray:
    """float32 [batch][n_kv_heads][n_pos][head_dim]."""
    return np.stack([rows(w, stream, layer, b, n_pos, start) for b in range(w.batch)])


def batch_query(w: Workload, layer: int, step: int = 0) -> np.ndarray:
    """float32 [batch][n_q_heads][head_dim]."""
    return np.stack([query(w, layer, b, step) for b in range(w.batch)])


def small(w: Workload, **kw) -> Workload:
    """A reduced copy of a workload for oracle-speed parity runs."""
    return w.with_(**kw)
