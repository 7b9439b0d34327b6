"""Seeded synthetic inputs for the quantized-KV attention workloads.

This module only draws random numbers and names workload shapes; it holds
none of the method's arithmetic, so both the GPU path's tests and the oracle
can take their inputs from it.

Values are float32 N(0, 1) from NumPy's PCG64, seeded by
``SeedSequence([seed, workload, layer, tensor, chunk])`` with tensor 0 = q,
1 = K, 2 = V, 3 = outlier-channel choice.  Large tensors are drawn in fixed
chunks of rows (a function of the shape only), so the values do not depend
on the number of threads used to draw them.

The pages measure whole models on llama.cpp runs; these shapes stand in for
those runs: a 16-layer stack of full-attention layers with 24 query heads, 4
KV heads and head_dim 256 (1,664 bytes per token per layer at Q8_0 K + Q4_0
V), contexts of 65,536 / 131,072 / 262,144 tokens, 256-token pages.
"""
from __future__ import annotations

import concurrent.futures as _cf
import math
import os
from dataclasses import dataclass

import numpy as np

Q, K, V, OUTLIER = 0, 1, 2, 3
_CHUNK_VALUES = 1 << 22


def normal(key, shape, threads: int | None = None) -> np.ndarray:
    """float32 N(0,1) array of ``shape`` for the integer tuple ``key``."""
    shape = tuple(int(s) for s in shape)
    out = np.empty(shape, dtype=np.float32)
    if out.size == 0:
        return out
    n0 = shape[0]
    row = out.size // n0
    rows_per_chunk = max(1, _CHUNK_VALUES // max(row, 1))
    flat = out.reshape(n0, row)
    n_chunks = (n0 + rows_per_chunk - 1) // rows_per_chunk

    def fill(c):
        r0 = c * rows_per_chunk
        r1 = min(n0, r0 + rows_per_chunk)
        rng = np.random.default_rng(np.random.SeedSequence(list(key) + [c]))
        rng.standard_normal(out=flat[r0:r1], dtype=np.float32)

    if n_chunks == 1:
        fill(0)
    else:
        threads = threads or min(16, os.cpu_count() or 1)
        with _cf.ThreadPoolExecutor(threads) as ex:
            list(ex.map(fill, range(n_chunks)))
    return out


def outlier_channels(key, n_channels: int, frac: float = 0.01) -> np.ndarray:
    """Sorted distinct channel indices, round(frac * n_channels) of them."""
    count = int(round(frac * n_channels))
    rng = np.random.default_rng(np.random.SeedSequence(list(key) + [OUTLIER]))
    return np.sort(rng.choice(n_channels, size=count, replace=False))


def with_outliers(x: np.ndarray, channels: np.ndarray, factor: float = 20.0) -> np.ndarray:
    """Scale the given channels of the flattened (head, dim) axis of x [..., H, D]."""
    flat = x.reshape(x.shape[:-2] + (x.shape[-2] * x.shape[-1],))
    flat[..., channels] *= np.float32(factor)
    return x


@dataclass(frozen=True)
class Workload:
    """One workload: a cache of ``cached`` tokens, ``n_new`` rows appended at
    position ``cached``, then ``n_q`` queries ending at ``cached + n_new``;
    ``n_seqs`` such sequences per layer (batched decode) when above 1;
    ``host_resident``: the caches live in host memory and stream in;
    ``codec``: how the cache stores K and V."""
    name: str
    wid: int
    layers: int
    n_heads: int
    n_kv: int
    head_dim: int
    cached: int
    n_new: int
    n_q: int
    page_size: int = 256
    outliers: bool = False
    n_seqs: int = 1
    host_resident: bool = False
    codec: int = 0          # 0: K Q8_0 + V Q4_0; 1: K and V INT2 (128-value blocks)

    @property
    def ctx(self) -> int:
        return self.cached + self.n_new

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.head_dim)

    @property
    def n_pages(self) -> int:
        return (self.ctx + self.page_size - 1) // self.page_size


WORKLOADS = {
    # tiny single-layer decode, 2 q heads sharing 1 KV head, D = 64, 512 tokens
    "tiny": Workload("tiny", 1, 1, 2, 1, 64, 511, 1, 1),
    # 16-layer GQA 24/4 x 256 decode at 65,536 tokens
    "decode65k": Workload("decode65k", 2, 16, 24, 4, 256, 65535, 1, 1),
    # same at 262,144 tokens, split over pages and merged
    "decode262k": Workload("decode262k", 3, 16, 24, 4, 256, 262143, 1, 1),
    # speculative verify batch: 4 rows appended after 131,072 tokens, 4 queries
    "verify131k": Workload("verify131k", 4, 16, 24, 4, 256, 131072, 4, 4),
    # chunked prefill: 2,048 rows appended after 260,096 tokens, 1% outliers x20
    "prefill262k": Workload("prefill262k", 5, 1, 24, 4, 256, 260096, 2048, 2048, outliers=True),
    # batched decode: 16 sequences of 16,384 tokens per layer (the KV bytes of
    # decode262k spread over 16 requests)
    "batch16x16k": Workload("batch16x16k", 6, 16, 24, 4, 256, 16383, 1, 1, n_seqs=16),
    # decode262k with every layer's cache in pinned host memory, streamed to
    # the GPU layer by layer while the previous layer's attention runs
    "stream262k": Workload("stream262k", 7, 16, 24, 4, 256, 262144, 0, 1, host_resident=True),
    # decode262k over the 2-bit cache (K and V INT2: 144 bytes per token and
    # KV head instead of 416)
    "int2decode262k": Workload("int2decode262k", 8, 16, 24, 4, 256, 262143, 1, 1, codec=1),
    # batch16x16k over the 2-bit cache
    "int2batch16x16k": Workload("int2batch16x16k", 9, 16, 24, 4, 256, 16383, 1, 1, n_seqs=16, codec=1),
    # prefill262k over the 2-bit cache
    "int2prefill262k": Workload("int2prefill262k", 10, 1, 24, 4, 256, 260096, 2048, 2048, outliers=True, codec=1),
}


def layer_kv(w: Workload, layer: int, seed: int = 0, rows: int | None = None):
    """fp32 K and V rows [ctx][n_kv][D] of one layer (first ``rows`` rows only
    if given; the values do not depend on ``rows``, chunks are fixed)."""
    n = w.ctx if rows is None else rows
    k = normal((seed, w.wid, layer, K), (n, w.n_kv, w.head_dim))
    v = normal((seed, w.wid, layer, V), (n, w.n_kv, w.head_dim))
    if w.outliers:
        with_outliers(k, outlier_channels((seed, w.wid, layer, K), w.n_kv * w.head_dim))
        with_outliers(v, outlier_channels((seed, w.wid, layer, V), w.n_kv * w.head_dim))
    return k, v


def layer_q(w: Workload, layer: int, seed: int = 0) -> np.ndarray:
    q = normal((seed, w.wid, layer, Q), (w.n_q, w.n_heads, w.head_dim))
    if w.outliers:
        with_outliers(q, outlier_channels((seed, w.wid, layer, Q), w.n_heads * w.head_dim))
    return q
