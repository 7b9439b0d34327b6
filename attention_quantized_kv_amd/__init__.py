"""Python binding of libkvq: attention over a Q8_0-K / Q4_0-V paged KV cache
on an AMD Instinct MI355X (gfx950).

Argument marshalling only: every step of the computation runs in the HIP
kernels of ``libkvq.so`` (built from ``csrc/`` by ``_build.build()``).  Torch
tensors supply device memory and the current HIP stream; the functions keep
the C ABI's names (include/kvq.h) and raise ``KvqError`` on a non-zero
status.  There is no CPU fallback: importing fails if the library is missing.
"""
from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.environ.get("KVQ_LIB") or os.path.join(HERE, "libkvq.so")

KVQ_OK = 0
KVQ_ERR_INVALID_ARG = -1
KVQ_ERR_UNSUPPORTED = -2
KVQ_ERR_WORKSPACE = -3
KVQ_ERR_CAPACITY = -4
KVQ_ERR_HIP = -5
KVQ_MAX_NQ_DECODE = 8
KVQ_MAX_SEQS = 64

KERNEL_AUTO, KERNEL_VALU, KERNEL_MFMA_STREAM, KERNEL_MFMA_TILED = 0, 1, 2, 3

EXPORTS = (
    "kvq_unit_bytes", "kvq_pool_bytes", "kvq_append", "kvq_workspace_bytes",
    "kvq_decode_attn", "kvq_prefill_attn", "kvq_workspace_bytes_ex", "kvq_attn_ex",
    "kvq_append_attn_workspace_bytes", "kvq_append_attn", "kvq_noalloc_scratch_bytes", "kvq_append_attn_noalloc",
    "kvq_decode_attn_batch_workspace_bytes", "kvq_decode_attn_batch", "kvq_stage_pages", "kvq_hadamard",
    "kvq_status_str", "kvq_last_error", "kvq_version",
)


class KvqError(RuntimeError):
    def __init__(self, status: int, func: str, detail: str):
        super().__init__(f"{func}: {_status_name(status)} ({status}): {detail}")
        self.status = status


KVQ_CODEC_Q8K_Q4V, KVQ_CODEC_INT2 = 0, 1


class Layout(ctypes.Structure):
    """kvq_layout: n_kv_heads, head_dim, page_size, n_pages, codec (0: K Q8_0 +
    V Q4_0, the default; 1: K and V INT2)."""
    _fields_ = [("n_kv_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("page_size", ctypes.c_int32), ("n_pages", ctypes.c_int32), ("codec", ctypes.c_int32)]

    def __repr__(self):
        return (f"Layout(n_kv_heads={self.n_kv_heads}, head_dim={self.head_dim}, "
                f"page_size={self.page_size}, n_pages={self.n_pages}, codec={self.codec})")


class AttnOpts(ctypes.Structure):
    """kvq_attn_opts: kernel, chunks_per_split, and two optional hipEvent_t
    handles recorded around the attention kernel (not the split merge)."""
    _fields_ = [("kernel", ctypes.c_int32), ("chunks_per_split", ctypes.c_int32),
                ("kernel_begin_event", ctypes.c_void_p), ("kernel_end_event", ctypes.c_void_p)]


_lib = None


def lib() -> ctypes.CDLL:
    """The loaded libkvq.so; raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it with "
                          "`python -m attention_quantized_kv_amd._build` (hipcc, gfx950)")
    L = ctypes.CDLL(LIB_PATH)
    P, i32, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t
    LP = ctypes.POINTER(Layout)
    OP = ctypes.POINTER(AttnOpts)
    SZP = ctypes.POINTER(ctypes.c_size_t)
    sig = {
        "kvq_unit_bytes": [LP, SZP],
        "kvq_pool_bytes": [LP, SZP],
        "kvq_append": [LP, P, P, i32, i32, i32, P, P, P],
        "kvq_workspace_bytes": [LP, i32, i32, i32, i32, SZP],
        "kvq_workspace_bytes_ex": [LP, i32, i32, i32, OP, SZP],
        "kvq_decode_attn": [LP, P, P, i32, i32, i32, i32, P, ctypes.c_float, P, P, P, sz, P],
        "kvq_prefill_attn": [LP, P, P, i32, i32, i32, i32, P, ctypes.c_float, P, P, P, sz, P],
        "kvq_attn_ex": [LP, P, P, i32, i32, i32, i32, P, ctypes.c_float, P, P, P, sz, OP, P],
        "kvq_append_attn_workspace_bytes": [LP, i32, i32, i32, OP, SZP],
        "kvq_append_attn": [LP, P, P, i32, i32, i32, P, P, i32, P, ctypes.c_float, P, P, P, sz, OP, P],
        "kvq_noalloc_scratch_bytes": [],
        "kvq_append_attn_noalloc": [LP, P, P, i32, i32, i32, P, P, i32, P, ctypes.c_float, P, P, OP, P],
        "kvq_decode_attn_batch_workspace_bytes": [LP, i32, P, i32, i32, SZP],
        "kvq_decode_attn_batch": [LP, P, P, i32, i32, P, i32, i32, P, ctypes.c_float, P, P, P, sz, OP, P],
        "kvq_stage_pages": [LP, P, P, i32, LP, P, i32, P],
        "kvq_hadamard": [P, ctypes.c_int64, i32, P],
        "kvq_status_str": [ctypes.c_int],
        "kvq_last_error": [],
        "kvq_version": [],
    }
    for name, args in sig.items():
        f = getattr(L, name)
        f.argtypes = args
        f.restype = ctypes.c_int
    L.kvq_noalloc_scratch_bytes.restype = ctypes.c_size_t
    L.kvq_status_str.restype = ctypes.c_char_p
    L.kvq_last_error.restype = ctypes.c_char_p
    _lib = L
    return L


def _status_name(status: int) -> str:
    try:
        return lib().kvq_status_str(status).decode()
    except Exception:
        return str(status)


def _check(status: int, func: str):
    if status != KVQ_OK:
        raise KvqError(status, func, lib().kvq_last_error().decode())


def _ptr(t) -> ctypes.c_void_p:
    """Device pointer of a tensor (or None / a raw int address)."""
    if t is None:
        return ctypes.c_void_p(0)
    if isinstance(t, int):
        return ctypes.c_void_p(t)
    return ctypes.c_void_p(t.data_ptr())


def _stream(stream) -> ctypes.c_void_p:
    if stream is None:
        import torch
        return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    if isinstance(stream, int):
        return ctypes.c_void_p(stream)
    return ctypes.c_void_p(stream.cuda_stream)


def _need(t, name, dtype=None, cuda=True):
    if t is None:
        return
    if isinstance(t, int):
        return
    if cuda and not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")


def _n_table(page_table) -> int:
    return page_table.numel() if hasattr(page_table, "numel") else int(page_table)


# --------------------------------------------------------------------------
# C ABI, one function per entry point
# --------------------------------------------------------------------------

def kvq_version() -> int:
    return lib().kvq_version()


def kvq_unit_bytes(layout: Layout) -> int:
    out = ctypes.c_size_t(0)
    _check(lib().kvq_unit_bytes(ctypes.byref(layout), ctypes.byref(out)), "kvq_unit_bytes")
    return out.value


def kvq_pool_bytes(layout: Layout) -> int:
    out = ctypes.c_size_t(0)
    _check(lib().kvq_pool_bytes(ctypes.byref(layout), ctypes.byref(out)), "kvq_pool_bytes")
    return out.value


def kvq_append(layout: Layout, pool, page_table, pos0: int, k, v, stream=None, n_table=None):
    """Quantize k, v fp32 [n_new][n_kv][D] into the pool at positions pos0.."""
    import torch
    _need(pool, "pool", torch.uint8)
    _need(page_table, "page_table", torch.int32)
    _need(k, "k", torch.float32)
    _need(v, "v", torch.float32)
    n_new = k.shape[0] if hasattr(k, "shape") else 0
    nt = _n_table(page_table) if n_table is None else n_table
    _check(lib().kvq_append(ctypes.byref(layout), _ptr(pool), _ptr(page_table), nt, int(pos0), int(n_new),
                            _ptr(k), _ptr(v), _stream(stream)), "kvq_append")


def kvq_workspace_bytes(layout: Layout, n_heads: int, ctx_len: int, n_q: int, prefill: bool = False) -> int:
    out = ctypes.c_size_t(0)
    _check(lib().kvq_workspace_bytes(ctypes.byref(layout), n_heads, ctx_len, n_q, int(bool(prefill)),
                                     ctypes.byref(out)), "kvq_workspace_bytes")
    return out.value


def kvq_workspace_bytes_ex(layout: Layout, n_heads: int, ctx_len: int, n_q: int,
                           kernel: int = 0, chunks_per_split: int = 0) -> int:
    out = ctypes.c_size_t(0)
    opts = AttnOpts(kernel, chunks_per_split)
    _check(lib().kvq_workspace_bytes_ex(ctypes.byref(layout), n_heads, ctx_len, n_q, ctypes.byref(opts),
                                        ctypes.byref(out)), "kvq_workspace_bytes_ex")
    return out.value


def _attn_args(pool, page_table, q, out, lse, ws):
    import torch
    _need(pool, "pool", torch.uint8)
    _need(page_table, "page_table", torch.int32)
    _need(q, "q", torch.float32)
    _need(out, "out", torch.float32)
    _need(lse, "lse", torch.float32)
    _need(ws, "workspace", torch.uint8)
    n_q, n_heads = q.shape[0], q.shape[1]
    ws_bytes = 0 if ws is None else (ws.numel() if hasattr(ws, "numel") else 0)
    return n_q, n_heads, ws_bytes


def kvq_decode_attn(layout: Layout, pool, page_table, ctx_len: int, q, scale: float, out, lse=None,
                    ws=None, stream=None, n_table=None):
    """Decode (n_q = 1) or verify-batch (n_q <= 8) attention; q, out [n_q][n_heads][D]."""
    n_q, n_heads, ws_bytes = _attn_args(pool, page_table, q, out, lse, ws)
    nt = _n_table(page_table) if n_table is None else n_table
    _check(lib().kvq_decode_attn(ctypes.byref(layout), _ptr(pool), _ptr(page_table), nt, int(ctx_len),
                                 n_heads, n_q, _ptr(q), float(scale), _ptr(out), _ptr(lse), _ptr(ws),
                                 ws_bytes, _stream(stream)), "kvq_decode_attn")


def kvq_prefill_attn(layout: Layout, pool, page_table, ctx_len: int, q, scale: float, out, lse=None,
                     ws=None, stream=None, n_table=None):
    """Causal chunk attention for n_q >= 1 queries ending at ctx_len."""
    n_q, n_heads, ws_bytes = _attn_args(pool, page_table, q, out, lse, ws)
    nt = _n_table(page_table) if n_table is None else n_table
    _check(lib().kvq_prefill_attn(ctypes.byref(layout), _ptr(pool), _ptr(page_table), nt, int(ctx_len),
                                  n_heads, n_q, _ptr(q), float(scale), _ptr(out), _ptr(lse), _ptr(ws),
                                  ws_bytes, _stream(stream)), "kvq_prefill_attn")


def kvq_attn_ex(layout: Layout, pool, page_table, ctx_len: int, q, scale: float, out, lse=None,
                ws=None, kernel: int = 0, chunks_per_split: int = 0, stream=None, n_table=None,
                events=None):
    """Attention with an explicit kernel and split size (tests, tuning).
    events: optional (begin, end) pair of raw hipEvent_t handles (ints) that
    the library records around the attention kernel itself."""
    n_q, n_heads, ws_bytes = _attn_args(pool, page_table, q, out, lse, ws)
    nt = _n_table(page_table) if n_table is None else n_table
    opts = AttnOpts(kernel, chunks_per_split)
    if events is not None:
        if not events[0] or not events[1]:
            raise ValueError("events must be two created hipEvent_t handles")
        opts.kernel_begin_event = events[0]
        opts.kernel_end_event = events[1]
    _check(lib().kvq_attn_ex(ctypes.byref(layout), _ptr(pool), _ptr(page_table), nt, int(ctx_len),
                             n_heads, n_q, _ptr(q), float(scale), _ptr(out), _ptr(lse), _ptr(ws),
                             ws_bytes, ctypes.byref(opts), _stream(stream)), "kvq_attn_ex")


def kvq_append_attn_workspace_bytes(layout: Layout, n_heads: int, pos0: int, n_new: int,
                                    kernel: int = 0, chunks_per_split: int = 0) -> int:
    out = ctypes.c_size_t(0)
    opts = AttnOpts(kernel, chunks_per_split)
    _check(lib().kvq_append_attn_workspace_bytes(ctypes.byref(layout), n_heads, int(pos0), int(n_new),
                                                 ctypes.byref(opts), ctypes.byref(out)),
           "kvq_append_attn_workspace_bytes")
    return out.value


def kvq_append_attn(layout: Layout, pool, page_table, pos0: int, k, v, q, scale: float, out, lse=None,
                    ws=None, kernel: int = 0, chunks_per_split: int = 0, stream=None, n_table=None,
                    events=None):
    """One decode step: append k, v [n_new][n_kv][D] at pos0, then attend the
    n_new queries q [n_new][n_heads][D] over pos0 + n_new keys.  events as for
    kvq_attn_ex (recorded around the split pass over the cached keys)."""
    import torch
    _need(k, "k", torch.float32)
    _need(v, "v", torch.float32)
    n_q, n_heads, ws_bytes = _attn_args(pool, page_table, q, out, lse, ws)
    if k.shape[0] != n_q or v.shape[0] != n_q:
        raise ValueError("k, v and q must hold the same number of rows")
    nt = _n_table(page_table) if n_table is None else n_table
    opts = AttnOpts(kernel, chunks_per_split)
    if events is not None:
        if not events[0] or not events[1]:
            raise ValueError("events must be two created hipEvent_t handles")
        opts.kernel_begin_event = events[0]
        opts.kernel_end_event = events[1]
    _check(lib().kvq_append_attn(ctypes.byref(layout), _ptr(pool), _ptr(page_table), nt, int(pos0), n_q,
                                 _ptr(k), _ptr(v), n_heads, _ptr(q), float(scale), _ptr(out), _ptr(lse),
                                 _ptr(ws), ws_bytes, ctypes.byref(opts), _stream(stream)), "kvq_append_attn")


def kvq_noalloc_scratch_bytes() -> int:
    """Bytes of the static device scratch kvq_append_attn_noalloc uses."""
    return int(lib().kvq_noalloc_scratch_bytes())


def kvq_append_attn_noalloc(layout: Layout, pool, page_table, pos0: int, k, v, q, scale: float, out, lse=None,
                            kernel: int = 0, chunks_per_split: int = 0, stream=None, n_table=None, events=None):
    """kvq_append_attn with the library's static device scratch instead of a
    workspace (no device allocation by the call)."""
    import torch
    _need(k, "k", torch.float32)
    _need(v, "v", torch.float32)
    n_q, n_heads, _ = _attn_args(pool, page_table, q, out, lse, None)
    if k.shape[0] != n_q or v.shape[0] != n_q:
        raise ValueError("k, v and q must hold the same number of rows")
    nt = _n_table(page_table) if n_table is None else n_table
    opts = AttnOpts(kernel, chunks_per_split)
    if events is not None:
        if not events[0] or not events[1]:
            raise ValueError("events must be two created hipEvent_t handles")
        opts.kernel_begin_event = events[0]
        opts.kernel_end_event = events[1]
    _check(lib().kvq_append_attn_noalloc(ctypes.byref(layout), _ptr(pool), _ptr(page_table), nt, int(pos0), n_q,
                                         _ptr(k), _ptr(v), n_heads, _ptr(q), float(scale), _ptr(out), _ptr(lse),
                                         ctypes.byref(opts), _stream(stream)), "kvq_append_attn_noalloc")


def _ctx_array(ctx_lens):
    vals = [int(c) for c in ctx_lens]
    return (ctypes.c_int32 * max(len(vals), 1))(*vals), len(vals)


def kvq_decode_attn_batch_workspace_bytes(layout: Layout, ctx_lens, n_heads: int, n_q: int) -> int:
    """Workspace bytes of kvq_decode_attn_batch for these sequences."""
    arr, n = _ctx_array(ctx_lens)
    out = ctypes.c_size_t(0)
    _check(lib().kvq_decode_attn_batch_workspace_bytes(ctypes.byref(layout), n, ctypes.cast(arr, ctypes.c_void_p),
                                                       int(n_heads), int(n_q), ctypes.byref(out)),
           "kvq_decode_attn_batch_workspace_bytes")
    return out.value


def kvq_decode_attn_batch(layout: Layout, pool, page_tables, ctx_lens, q, scale: float, out, lse=None,
                          ws=None, stream=None, events=None):
    """Decode of several sequences in one call: page_tables int32 [n_seqs][n_table]
    (device), ctx_lens a host sequence of n_seqs ints, q and out
    [n_seqs][n_q][n_heads][D], lse [n_seqs][n_q][n_heads] or None; events as
    for kvq_attn_ex (recorded around the streaming kernel)."""
    import torch
    _need(pool, "pool", torch.uint8)
    _need(page_tables, "page_tables", torch.int32)
    _need(q, "q", torch.float32)
    _need(out, "out", torch.float32)
    _need(lse, "lse", torch.float32)
    _need(ws, "workspace", torch.uint8)
    if page_tables.dim() != 2 or q.dim() != 4:
        raise ValueError("page_tables must be [n_seqs][n_table] and q [n_seqs][n_q][n_heads][D]")
    arr, n = _ctx_array(ctx_lens)
    if page_tables.shape[0] != n or q.shape[0] != n:
        raise ValueError("page_tables, ctx_lens and q must cover the same sequences")
    ws_bytes = 0 if ws is None else ws.numel()
    opts = AttnOpts(0, 0)
    if events is not None:
        if not events[0] or not events[1]:
            raise ValueError("events must be two created hipEvent_t handles")
        opts.kernel_begin_event = events[0]
        opts.kernel_end_event = events[1]
    _check(lib().kvq_decode_attn_batch(ctypes.byref(layout), _ptr(pool), _ptr(page_tables),
                                       int(page_tables.shape[1]), n, ctypes.cast(arr, ctypes.c_void_p),
                                       int(q.shape[2]), int(q.shape[1]), _ptr(q), float(scale), _ptr(out),
                                       _ptr(lse), _ptr(ws), ws_bytes, ctypes.byref(opts), _stream(stream)),
           "kvq_decode_attn_batch")


def kvq_hadamard(x, stream=None):
    """Rotate every row of x (a contiguous fp32 device tensor whose last axis,
    a power of two up to 1024, is the row) in place by H / sqrt(dim)."""
    import torch
    _need(x, "x", torch.float32)
    dim = int(x.shape[-1]) if x.dim() > 0 else 0
    n_rows = x.numel() // dim if dim > 0 else 0
    _check(lib().kvq_hadamard(_ptr(x), n_rows, dim, _stream(stream)), "kvq_hadamard")


def kvq_stage_pages(host_layout: Layout, host_pool, host_page_table, dev_layout: Layout, dev_pool,
                    dst_first: int = 0, n_copy=None, stream=None):
    """Copy the pages host_page_table names (a host int32 sequence or tensor)
    from host_pool (a CPU uint8 tensor, pinned for overlap) to consecutive
    pages of dev_pool starting at dst_first, asynchronously on `stream`."""
    import torch
    if host_pool.is_cuda:
        raise ValueError("host_pool must be a host tensor")
    if not host_pool.is_contiguous() or host_pool.dtype != torch.uint8:
        raise ValueError("host_pool must be a contiguous uint8 tensor")
    _need(dev_pool, "dev_pool", torch.uint8)
    vals = [int(x) for x in (host_page_table.tolist() if hasattr(host_page_table, "tolist") else host_page_table)]
    n = len(vals) if n_copy is None else int(n_copy)
    if n > len(vals):
        raise ValueError(f"n_copy {n} exceeds the {len(vals)} page-table entries")
    arr = (ctypes.c_int32 * max(len(vals), 1))(*vals)
    _check(lib().kvq_stage_pages(ctypes.byref(host_layout), ctypes.c_void_p(host_pool.data_ptr()),
                                 ctypes.cast(arr, ctypes.c_void_p), n, ctypes.byref(dev_layout), _ptr(dev_pool),
                                 int(dst_first), _stream(stream)), "kvq_stage_pages")
