"""CPU oracle for attention over a Q8_0-K / Q4_0-V block-quantized KV cache.

TEST INFRASTRUCTURE ONLY: the test-suite, the smoke check and the CPU-baseline
leg of the benchmark are the only callers.  The GPU library never imports it,
and it imports nothing from the GPU library.  The arithmetic lives in
``kvq_oracle.c`` (plain C, fp32 quantizer, fp64 attention); this module only
marshals numpy arrays.  ``brute.py`` repeats the same definitions with
pure-Python loops for tiny inputs.

Sources (web pages, cited by title and section):
  [RX9070]  "Qwen 27B (IQ4_XS, Q8/Q4 KV) on a 16GB RX 9070 XT at 262k context,
            via adaptive KV streaming" (molayo1419.me)
  [ROCmKV]  "Adaptive KV streaming lands on ROCm: Qwen3.8-27B at full 262k
            context on a 16 GB RX 9070 XT" (richland.au)
  [OSCAR2]  "OSCAR2 KV Cache benchmark" (molayo1419.me)
  [KVGUIDE] "Context window and KV cache" (localaiforum.com guide)

Every function here is pinned by the CPU tests (``tests/test_oracle_*.py``)
to facts other than itself: the pages' worked byte counts, hand-derived
quantization blocks, closed forms of attention (one key, equal scores),
split-and-merge algebra, a numpy/scipy route and pure-Python brute force.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "kvq_oracle.c")
_LIB_PATH = os.path.join(_HERE, "_liboracle_kvq.so")
BLOCK = 32

_lib = None


def build() -> str:
    """Compile the C oracle with gcc (no fast-math, no FMA contraction)."""
    cmd = ["gcc", "-std=c11", "-O2", "-fPIC", "-shared", "-fopenmp", "-ffp-contract=off",
           "-fno-fast-math", "-Wall", "-o", _LIB_PATH + ".tmp", _SRC, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(_LIB_PATH + ".tmp", _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        build()
    lib = ctypes.CDLL(_LIB_PATH)
    P = ctypes.c_void_p
    i32, i64, f64 = ctypes.c_int32, ctypes.c_int64, ctypes.c_double
    lib.orc_f32_to_f16.argtypes = [ctypes.c_float]
    lib.orc_f32_to_f16.restype = ctypes.c_uint16
    lib.orc_f16_to_f32.argtypes = [ctypes.c_uint16]
    lib.orc_f16_to_f32.restype = ctypes.c_float
    for name in ("orc_quantize_q8_0", "orc_quantize_q4_0"):
        getattr(lib, name).argtypes = [P, i64, P, P]
        getattr(lib, name).restype = None
    for name in ("orc_dequant_q8_0", "orc_dequant_q4_0"):
        getattr(lib, name).argtypes = [P, P, i64, P]
        getattr(lib, name).restype = None
    for name in ("orc_kv_bytes_per_token_f16", "orc_kv_bytes_per_token_q8k_q4v"):
        getattr(lib, name).argtypes = [i64, i64, i64]
        getattr(lib, name).restype = i64
    lib.orc_q8_0_block_bytes.restype = i64
    lib.orc_q4_0_block_bytes.restype = i64
    lib.orc_int2_block_bytes.restype = i64
    lib.orc_quantize_int2.argtypes = [P, i64, P, P, P]
    lib.orc_quantize_int2.restype = None
    lib.orc_dequant_int2.argtypes = [P, P, P, i64, P]
    lib.orc_dequant_int2.restype = None
    lib.orc_attention_dense.argtypes = [i32, i32, i32, i32, i32, P, P, P, f64, i32, P, P, P]
    lib.orc_attention_dense.restype = ctypes.c_int
    lib.orc_attention.argtypes = [i32, i32, i32, i32, i32, P, P, P, P, P, f64, i32, P, P, P]
    lib.orc_attention.restype = ctypes.c_int
    lib.orc_attention_partial.argtypes = [i32, i32, i32, i32, i32, P, P, P, P, P, f64,
                                          i64, i64, P, P, P]
    lib.orc_attention_partial.restype = None
    lib.orc_merge.argtypes = [i32, i32, P, P, P, P, P]
    lib.orc_merge.restype = None
    lib.orc_max_threads.restype = ctypes.c_int
    _lib = lib
    return lib


def _ptr(a: np.ndarray):
    assert a.flags["C_CONTIGUOUS"]
    return a.ctypes.data_as(ctypes.c_void_p)


# --------------------------------------------------------------------------
# scalars
# --------------------------------------------------------------------------

def f32_to_f16_bits(x: float) -> int:
    """Nearest binary16 (ties to even), as a 16-bit pattern."""
    return int(_load().orc_f32_to_f16(float(np.float32(x))))


def f16_bits_to_f32(h: int) -> float:
    return float(_load().orc_f16_to_f32(int(h)))


_F16_TABLE = None


def f16_bits_to_f64_array(h: np.ndarray) -> np.ndarray:
    """Exact values of an array of fp16 bit patterns (a table of the C routine)."""
    global _F16_TABLE
    if _F16_TABLE is None:
        lib = _load()
        _F16_TABLE = np.array([lib.orc_f16_to_f32(i) for i in range(65536)], dtype=np.float64)
    flat = np.ascontiguousarray(h, dtype=np.uint16).ravel()
    return _F16_TABLE[flat].reshape(np.shape(h))


# --------------------------------------------------------------------------
# quantizers: x [..., D] with D % 32 == 0, blocks along the last axis
# --------------------------------------------------------------------------

def quantize_q8_0(x: np.ndarray):
    """Q8_0 codes (int8, same shape as x) and fp16 scale bits ([..., D/32])."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    assert x.shape[-1] % BLOCK == 0
    nb = x.size // BLOCK
    codes = np.empty(x.shape, dtype=np.int8)
    scales = np.empty(x.shape[:-1] + (x.shape[-1] // BLOCK,), dtype=np.uint16)
    _load().orc_quantize_q8_0(_ptr(x), nb, _ptr(codes), _ptr(scales))
    return codes, scales


def quantize_q4_0(x: np.ndarray):
    """Q4_0 codes (uint8 0..15, one per value) and fp16 scale bits."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    assert x.shape[-1] % BLOCK == 0
    nb = x.size // BLOCK
    codes = np.empty(x.shape, dtype=np.uint8)
    scales = np.empty(x.shape[:-1] + (x.shape[-1] // BLOCK,), dtype=np.uint16)
    _load().orc_quantize_q4_0(_ptr(x), nb, _ptr(codes), _ptr(scales))
    return codes, scales


BLOCK2 = 128     # values per INT2 block


def quantize_int2(x: np.ndarray):
    """INT2 codes (uint8 0..3, one per value), fp16 scale bits and fp16 zero
    bits ([..., D/128]); blocks of 128 along the last axis."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    assert x.shape[-1] % BLOCK2 == 0
    nb = x.size // BLOCK2
    codes = np.empty(x.shape, dtype=np.uint8)
    scales = np.empty(x.shape[:-1] + (x.shape[-1] // BLOCK2,), dtype=np.uint16)
    zeros = np.empty_like(scales)
    _load().orc_quantize_int2(_ptr(x), nb, _ptr(codes), _ptr(scales), _ptr(zeros))
    return codes, scales, zeros


def dequant_int2(codes: np.ndarray, scales: np.ndarray, zeros: np.ndarray) -> np.ndarray:
    codes = np.ascontiguousarray(codes, dtype=np.uint8)
    scales = np.ascontiguousarray(scales, dtype=np.uint16)
    zeros = np.ascontiguousarray(zeros, dtype=np.uint16)
    out = np.empty(codes.shape, dtype=np.float64)
    _load().orc_dequant_int2(_ptr(codes), _ptr(scales), _ptr(zeros), codes.size // BLOCK2, _ptr(out))
    return out


def dequant_q8_0(codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    codes = np.ascontiguousarray(codes, dtype=np.int8)
    scales = np.ascontiguousarray(scales, dtype=np.uint16)
    out = np.empty(codes.shape, dtype=np.float64)
    _load().orc_dequant_q8_0(_ptr(codes), _ptr(scales), codes.size // BLOCK, _ptr(out))
    return out


def dequant_q4_0(codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    codes = np.ascontiguousarray(codes, dtype=np.uint8)
    scales = np.ascontiguousarray(scales, dtype=np.uint16)
    out = np.empty(codes.shape, dtype=np.float64)
    _load().orc_dequant_q4_0(_ptr(codes), _ptr(scales), codes.size // BLOCK, _ptr(out))
    return out


# --------------------------------------------------------------------------
# byte formulas
# --------------------------------------------------------------------------

def kv_bytes_per_token_f16(layers: int, kv_heads: int, head_dim: int) -> int:
    return int(_load().orc_kv_bytes_per_token_f16(layers, kv_heads, head_dim))


def kv_bytes_per_token_q8k_q4v(layers: int, kv_heads: int, head_dim: int) -> int:
    return int(_load().orc_kv_bytes_per_token_q8k_q4v(layers, kv_heads, head_dim))


def q8_0_block_bytes() -> int:
    return int(_load().orc_q8_0_block_bytes())


def q4_0_block_bytes() -> int:
    return int(_load().orc_q4_0_block_bytes())


def int2_block_bytes() -> int:
    """Bytes per 128 values of the INT2 codec."""
    return int(_load().orc_int2_block_bytes())


# --------------------------------------------------------------------------
# attention
# --------------------------------------------------------------------------

class QuantCache:
    """One layer's quantized cache in the oracle's logical (token-major) layout."""

    def __init__(self, k_codes, k_scales, v_codes, v_scales):
        self.k_codes = np.ascontiguousarray(k_codes, dtype=np.int8)
        self.k_scales = np.ascontiguousarray(k_scales, dtype=np.uint16)
        self.v_codes = np.ascontiguousarray(v_codes, dtype=np.uint8)
        self.v_scales = np.ascontiguousarray(v_scales, dtype=np.uint16)
        self.ctx, self.n_kv, self.D = self.k_codes.shape

    @classmethod
    def from_float(cls, k: np.ndarray, v: np.ndarray) -> "QuantCache":
        """Quantize fp32 k, v [ctx][n_kv][D] (K as Q8_0, V as Q4_0)."""
        kc, ks = quantize_q8_0(k)
        vc, vs = quantize_q4_0(v)
        return cls(kc, ks, vc, vs)

    def k_hat(self) -> np.ndarray:
        return dequant_q8_0(self.k_codes, self.k_scales)

    def v_hat(self) -> np.ndarray:
        return dequant_q4_0(self.v_codes, self.v_scales)


class Int2Cache:
    """One layer's INT2 cache (K and V both INT2), logical token-major layout."""

    def __init__(self, kc, ks, kz, vc, vs, vz):
        self.k = (kc, ks, kz)
        self.v = (vc, vs, vz)
        self.ctx, self.n_kv, self.D = kc.shape

    @classmethod
    def from_float(cls, k: np.ndarray, v: np.ndarray) -> "Int2Cache":
        return cls(*quantize_int2(k), *quantize_int2(v))

    def k_hat(self) -> np.ndarray:
        return dequant_int2(*self.k)

    def v_hat(self) -> np.ndarray:
        return dequant_int2(*self.v)


def hadamard_matrix(n: int) -> np.ndarray:
    """The n x n Hadamard matrix of Sylvester's construction (n a power of
    two): H_1 = [1], H_2m = [[H_m, H_m], [H_m, -H_m]].  Entries +-1, symmetric,
    H H = n I."""
    assert n >= 1 and n & (n - 1) == 0, "n must be a power of two"
    h = np.ones((1, 1))
    while h.shape[0] < n:
        h = np.block([[h, h], [h, -h]])
    return h


def hadamard(x: np.ndarray) -> np.ndarray:
    """The normalized Hadamard rotation of every row (last axis, a power of
    two): y = x H / sqrt(n), fp64.  The rotation the pages bake into a model
    so that the 2-bit cache holds rotated K and V ("OSCAR2 KV Cache
    benchmark", rotation model conversion: a Hadamard rotation per head of
    dimension 256).  H / sqrt(n) is orthogonal and symmetric, so it is its own
    inverse: rotating q and k leaves every score unchanged, and rotating v
    rotates the output, which one more rotation undoes."""
    x = np.asarray(x, dtype=np.float64)
    n = x.shape[-1]
    return x @ hadamard_matrix(n) / np.sqrt(n)


def attention_dense(q: np.ndarray, k_hat: np.ndarray, v_hat: np.ndarray, scale: float, rows=None,
                    ctx: int | None = None):
    """attention() over given dequantized K and V [ctx][n_kv][D] (fp64)."""
    q = np.ascontiguousarray(q, dtype=np.float32)
    k_hat = np.ascontiguousarray(k_hat, dtype=np.float64)
    v_hat = np.ascontiguousarray(v_hat, dtype=np.float64)
    n_q, n_heads, D = q.shape
    full, n_kv, Dk = k_hat.shape
    ctx = full if ctx is None else int(ctx)
    assert D == Dk and v_hat.shape == k_hat.shape and n_heads % n_kv == 0 and 1 <= n_q <= ctx <= full
    lib = _load()
    if rows is None:
        out = np.empty((n_q, n_heads, D), dtype=np.float64)
        lse = np.empty((n_q, n_heads), dtype=np.float64)
        threads = lib.orc_attention_dense(n_q, n_heads, n_kv, D, ctx, _ptr(q), _ptr(k_hat), _ptr(v_hat),
                                          float(scale), 0, None, _ptr(out), _ptr(lse))
        return out, lse, threads
    r = np.ascontiguousarray(np.asarray(rows, dtype=np.int32).reshape(-1, 2))
    out = np.empty((r.shape[0], D), dtype=np.float64)
    lse = np.empty((r.shape[0],), dtype=np.float64)
    lib.orc_attention_dense(n_q, n_heads, n_kv, D, ctx, _ptr(q), _ptr(k_hat), _ptr(v_hat), float(scale),
                            r.shape[0], _ptr(r), _ptr(out), _ptr(lse))
    return out, lse


def attention(q: np.ndarray, cache: QuantCache, scale: float, rows=None, ctx: int | None = None):
    """Exact attention (fp64) of q [n_q][n_heads][D] over the first ``ctx``
    cached tokens (default: all).  Query i sits at position ctx - n_q + i and
    sees keys at positions <= its own.

    rows: optional list of (i, h) pairs; returns (out [n_rows][D], lse [n_rows]).
    Without rows returns (out [n_q][n_heads][D], lse [n_q][n_heads]) and the
    thread count as a third element.
    """
    if isinstance(cache, Int2Cache):
        return attention_dense(q, cache.k_hat(), cache.v_hat(), scale, rows=rows, ctx=ctx)
    q = np.ascontiguousarray(q, dtype=np.float32)
    n_q, n_heads, D = q.shape
    ctx = cache.ctx if ctx is None else int(ctx)
    assert D == cache.D and n_heads % cache.n_kv == 0 and 1 <= n_q <= ctx <= cache.ctx
    lib = _load()
    if rows is None:
        out = np.empty((n_q, n_heads, D), dtype=np.float64)
        lse = np.empty((n_q, n_heads), dtype=np.float64)
        threads = lib.orc_attention(n_q, n_heads, cache.n_kv, D, ctx, _ptr(q), _ptr(cache.k_codes),
                                    _ptr(cache.k_scales), _ptr(cache.v_codes), _ptr(cache.v_scales),
                                    float(scale), 0, None, _ptr(out), _ptr(lse))
        return out, lse, threads
    r = np.ascontiguousarray(np.asarray(rows, dtype=np.int32).reshape(-1, 2))
    out = np.empty((r.shape[0], D), dtype=np.float64)
    lse = np.empty((r.shape[0],), dtype=np.float64)
    lib.orc_attention(n_q, n_heads, cache.n_kv, D, ctx, _ptr(q), _ptr(cache.k_codes),
                      _ptr(cache.k_scales), _ptr(cache.v_codes), _ptr(cache.v_scales),
                      float(scale), r.shape[0], _ptr(r), _ptr(out), _ptr(lse))
    return out, lse


def attention_partial(q: np.ndarray, cache: QuantCache, scale: float, j0: int, j1: int,
                      ctx: int | None = None):
    """Softmax state (m, l, acc) of every row over keys [j0, j1) (causal)."""
    q = np.ascontiguousarray(q, dtype=np.float32)
    n_q, n_heads, D = q.shape
    ctx = cache.ctx if ctx is None else int(ctx)
    m = np.empty((n_q, n_heads), dtype=np.float64)
    l = np.empty((n_q, n_heads), dtype=np.float64)
    acc = np.empty((n_q, n_heads, D), dtype=np.float64)
    _load().orc_attention_partial(n_q, n_heads, cache.n_kv, D, ctx, _ptr(q), _ptr(cache.k_codes),
                                  _ptr(cache.k_scales), _ptr(cache.v_codes), _ptr(cache.v_scales),
                                  float(scale), int(j0), int(j1), _ptr(m), _ptr(l), _ptr(acc))
    return m, l, acc


def merge(m: np.ndarray, l: np.ndarray, acc: np.ndarray):
    """Merge split states of one row: m, l [S], acc [S][D] -> (out [D], lse)."""
    m = np.ascontiguousarray(m, dtype=np.float64)
    l = np.ascontiguousarray(l, dtype=np.float64)
    acc = np.ascontiguousarray(acc, dtype=np.float64)
    S, D = acc.shape
    out = np.empty((D,), dtype=np.float64)
    lse = np.empty((1,), dtype=np.float64)
    _load().orc_merge(S, D, _ptr(m), _ptr(l), _ptr(acc), _ptr(out), _ptr(lse))
    return out, float(lse[0])


def max_threads() -> int:
    return int(_load().orc_max_threads())
