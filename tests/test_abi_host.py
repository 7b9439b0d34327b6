"""CPU: the C-ABI library loads, exports every symbol include/kvq.h declares,
and rejects bad arguments with the documented status before touching the GPU.
"""
import ctypes
import os
import re

import pytest

import attention_quantized_kv_amd as kvq

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
FAKE = ctypes.c_void_p(0x100000)     # a non-NULL, 256-aligned address never dereferenced


def declared_functions():
    text = open(os.path.join(ROOT, "include", "kvq.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(kvq_[a-z0-9_]+)\s*\(", text)))


def test_exports_every_declared_symbol():
    names = declared_functions()
    assert len(names) >= 11
    lib = kvq.lib()
    for n in names:
        assert hasattr(lib, n), n
    assert set(names) == set(kvq.EXPORTS)


def test_sizes():
    L = kvq.Layout(4, 256, 256, 1024)
    assert kvq.kvq_unit_bytes(L) == 256 * 416                 # 416 B/token/KV head at D = 256
    assert kvq.kvq_pool_bytes(L) == 436_207_616               # one 262,144-token layer
    assert kvq.kvq_unit_bytes(kvq.Layout(1, 64, 32, 1)) == 32 * 64 * 26 // 16
    assert kvq.kvq_workspace_bytes(L, 24, 262144, 1) > 0
    assert kvq.kvq_version() >= 10000


def _status(fn, *args):
    st = fn(*args)
    return st, kvq.lib().kvq_last_error().decode()


@pytest.mark.parametrize("fields,status", [
    ((0, 256, 256, 1), kvq.KVQ_ERR_INVALID_ARG),
    ((4, 0, 256, 1), kvq.KVQ_ERR_INVALID_ARG),
    ((4, 96, 256, 1), kvq.KVQ_ERR_UNSUPPORTED),
    ((4, 32, 256, 1), kvq.KVQ_ERR_UNSUPPORTED),
    ((4, 256, 48, 1), kvq.KVQ_ERR_UNSUPPORTED),
    ((4, 256, 2048, 1), kvq.KVQ_ERR_UNSUPPORTED),
    ((4, 256, 256, 0), kvq.KVQ_ERR_INVALID_ARG),
])
def test_layout_validation(fields, status):
    L = kvq.Layout(*fields)
    out = ctypes.c_size_t(0)
    st, msg = _status(kvq.lib().kvq_pool_bytes, ctypes.byref(L), ctypes.byref(out))
    assert st == status and msg


def test_append_validation():
    lib = kvq.lib()
    L = kvq.Layout(4, 256, 256, 4)
    args = lambda pool=FAKE, pt=FAKE, nt=4, pos0=0, n=1, k=FAKE, v=FAKE: (
        ctypes.byref(L), pool, pt, nt, pos0, n, k, v, None)
    assert _status(lib.kvq_append, *args(pool=None))[0] == kvq.KVQ_ERR_INVALID_ARG
    assert _status(lib.kvq_append, *args(k=None))[0] == kvq.KVQ_ERR_INVALID_ARG
    assert _status(lib.kvq_append, *args(n=-1))[0] == kvq.KVQ_ERR_INVALID_ARG
    assert _status(lib.kvq_append, *args(pos0=-3))[0] == kvq.KVQ_ERR_INVALID_ARG
    assert _status(lib.kvq_append, *args(pos0=1000, n=25))[0] == kvq.KVQ_ERR_CAPACITY
    assert _status(lib.kvq_append, *args(nt=0))[0] == kvq.KVQ_ERR_INVALID_ARG
    assert _status(lib.kvq_append, *args(pool=ctypes.c_void_p(0x100010)))[0] == kvq.KVQ_ERR_INVALID_ARG
    assert _status(lib.kvq_append, *args(n=0))[0] == kvq.KVQ_OK          # no-op, no launch


def test_attention_validation():
    lib = kvq.lib()
    L = kvq.Layout(4, 256, 256, 8)

    def call(fn=lib.kvq_decode_attn, pool=FAKE, pt=FAKE, nt=8, ctx=1000, nh=24, nq=1, q=FAKE,
             out=FAKE, ws=FAKE, wsb=1 << 30):
        return _status(fn, ctypes.byref(L), pool, pt, nt, ctx, nh, nq, q, ctypes.c_float(0.0625), out,
                       None, ws, wsb, None)

    assert call(pool=None)[0] == kvq.KVQ_ERR_INVALID_ARG
    assert call(q=None)[0] == kvq.KVQ_ERR_INVALID_ARG
    assert call(out=None)[0] == kvq.KVQ_ERR_INVALID_ARG
    assert call(nh=25)[0] == kvq.KVQ_ERR_INVALID_ARG                   # not a multiple of 4
    assert call(nh=68)[0] == kvq.KVQ_ERR_UNSUPPORTED                   # group 17 > 16
    assert call(nq=0)[0] == kvq.KVQ_ERR_INVALID_ARG
    assert call(nq=9)[0] == kvq.KVQ_ERR_INVALID_ARG                    # decode takes n_q <= 8
    assert call(ctx=3, nq=4)[0] == kvq.KVQ_ERR_INVALID_ARG
    assert call(ctx=2049)[0] == kvq.KVQ_ERR_CAPACITY                   # 8 pages of 256
    assert call(ws=None)[0] == kvq.KVQ_ERR_WORKSPACE
    assert call(wsb=16)[0] == kvq.KVQ_ERR_WORKSPACE
    st, msg = call(wsb=16)
    assert "workspace" in msg
    # prefill accepts long chunks; its workspace errors are the same
    assert call(fn=lib.kvq_prefill_attn, nq=9, ws=None)[0] == kvq.KVQ_ERR_WORKSPACE


def test_batch_decode_validation():
    lib = kvq.lib()
    L = kvq.Layout(4, 256, 256, 64)
    ctx = (ctypes.c_int32 * 4)(1000, 1, 2048, 300)

    def call(pool=FAKE, pt=FAKE, nt=8, ns=4, cl=ctx, nh=24, nq=1, q=FAKE, out=FAKE, ws=FAKE, wsb=1 << 30,
             opts=None):
        return _status(lib.kvq_decode_attn_batch, ctypes.byref(L), pool, pt, nt, ns,
                       None if cl is None else ctypes.cast(cl, ctypes.c_void_p), nh, nq, q,
                       ctypes.c_float(0.0625), out, None, ws, wsb, opts, None)

    assert call(pool=None)[0] == kvq.KVQ_ERR_INVALID_ARG
    assert call(pt=None)[0] == kvq.KVQ_ERR_INVALID_ARG
    assert call(cl=None)[0] == kvq.KVQ_ERR_INVALID_ARG
    assert call(ns=0)[0] == kvq.KVQ_ERR_INVALID_ARG
    assert call(ns=kvq.KVQ_MAX_SEQS + 1)[0] == kvq.KVQ_ERR_INVALID_ARG
    assert call(nq=9)[0] == kvq.KVQ_ERR_INVALID_ARG
    st, msg = call(nq=2)                                            # sequence 1 has a single key
    assert st == kvq.KVQ_ERR_INVALID_ARG and "sequence 1" in msg
    st, msg = call(nt=4)                                            # sequence 2 needs 8 pages
    assert st == kvq.KVQ_ERR_CAPACITY and "sequence 2" in msg
    assert call(nh=24 * 3)[0] == kvq.KVQ_ERR_UNSUPPORTED             # 18 heads per KV head
    assert call(ws=None)[0] == kvq.KVQ_ERR_WORKSPACE
    assert call(opts=ctypes.byref(kvq.AttnOpts(3, 0)))[0] == kvq.KVQ_ERR_INVALID_ARG   # tiled kernel
    # the workspace query: bytes grow with the partials of every sequence
    one = kvq.kvq_decode_attn_batch_workspace_bytes(L, [1000], 24, 1)
    four = kvq.kvq_decode_attn_batch_workspace_bytes(L, [1000, 1, 2048, 300], 24, 1)
    assert 0 < one < four
    assert call(wsb=four - 1)[0] == kvq.KVQ_ERR_WORKSPACE


def test_stage_pages_validation():
    lib = kvq.lib()
    H = kvq.Layout(4, 256, 256, 16)
    D = kvq.Layout(4, 256, 256, 8)
    pt = (ctypes.c_int32 * 4)(3, 4, 5, 9)

    def call(hl=H, hp=FAKE, t=pt, n=4, dl=D, dp=FAKE, first=0):
        return _status(lib.kvq_stage_pages, ctypes.byref(hl), hp, None if t is None else ctypes.cast(t, ctypes.c_void_p),
                       n, ctypes.byref(dl), dp, first, None)

    assert call(hp=None)[0] == kvq.KVQ_ERR_INVALID_ARG
    assert call(dp=None)[0] == kvq.KVQ_ERR_INVALID_ARG
    assert call(t=None)[0] == kvq.KVQ_ERR_INVALID_ARG
    assert call(n=-1)[0] == kvq.KVQ_ERR_INVALID_ARG
    assert call(dl=kvq.Layout(4, 128, 256, 8))[0] == kvq.KVQ_ERR_INVALID_ARG     # head_dim differs
    assert call(dl=kvq.Layout(2, 256, 256, 8))[0] == kvq.KVQ_ERR_INVALID_ARG     # KV heads differ
    # codecs differ: the copy is sized by the host unit (416 B per token and KV
    # head) and would run past a device pool of INT2 units (144 B); also with
    # the device pool made large enough in pages
    for dl in (kvq.Layout(4, 256, 256, 8, kvq.KVQ_CODEC_INT2), kvq.Layout(4, 256, 256, 64, kvq.KVQ_CODEC_INT2)):
        st, msg = call(dl=dl)
        assert st == kvq.KVQ_ERR_INVALID_ARG and "codec" in msg
    st, msg = call(hl=kvq.Layout(4, 256, 256, 16, kvq.KVQ_CODEC_INT2))
    assert st == kvq.KVQ_ERR_INVALID_ARG and "codec" in msg
    assert call(first=5)[0] == kvq.KVQ_ERR_INVALID_ARG                           # pages 5..8 of 8
    bad = (ctypes.c_int32 * 4)(3, 4, 16, 9)                                      # page 16 of 16
    st, msg = call(t=bad)
    assert st == kvq.KVQ_ERR_INVALID_ARG and "entry 2" in msg
    assert call(n=0)[0] == kvq.KVQ_OK                                            # no-op, no copy


def test_int2_codec_layout():
    for D in (128, 256):
        L = kvq.Layout(3, D, 64, 5, kvq.KVQ_CODEC_INT2)
        assert kvq.kvq_unit_bytes(L) == 9 * 64 * D // 16              # 36 bytes per 128 values, K and V
        assert kvq.kvq_pool_bytes(L) == 3 * 5 * 9 * 64 * D // 16
    lib = kvq.lib()
    out = ctypes.c_size_t(0)
    assert lib.kvq_unit_bytes(ctypes.byref(kvq.Layout(1, 64, 64, 1, kvq.KVQ_CODEC_INT2)),
                              ctypes.byref(out)) == kvq.KVQ_ERR_UNSUPPORTED
    assert lib.kvq_unit_bytes(ctypes.byref(kvq.Layout(1, 128, 64, 1, 2)), ctypes.byref(out)) == kvq.KVQ_ERR_INVALID_ARG


def test_int2_attention_plan():
    """Attention over the INT2 codec: kernel 4 for decode with up to 16 rows
    per KV head (also batched), kernel 3 for prefill and more rows; kernels
    1 and 2 are rejected, kernel 4 outside its range too, and kernel 4
    needs the INT2 codec."""
    L = kvq.Layout(2, 256, 64, 100, kvq.KVQ_CODEC_INT2)
    assert kvq.kvq_workspace_bytes(L, 12, 5000, 1) > 0                  # 6 rows
    assert kvq.kvq_workspace_bytes_ex(L, 16, 5000, 2, kernel=4) > 0     # 16 rows
    assert kvq.kvq_workspace_bytes(L, 12, 5000, 64, True) > 0           # prefill (kernel 3)
    assert kvq.kvq_workspace_bytes(L, 12, 5000, 3) > 0                  # 18 rows (kernel 3)

    def status(fn, *args, **kw):
        with pytest.raises(kvq.KvqError) as e:
            fn(*args, **kw)
        return e.value.status
    assert status(kvq.kvq_workspace_bytes_ex, L, 12, 5000, 3, kernel=4) == kvq.KVQ_ERR_UNSUPPORTED   # 18 rows
    for kernel in (1, 2):
        assert status(kvq.kvq_workspace_bytes_ex, L, 12, 5000, 1, kernel=kernel) == kvq.KVQ_ERR_UNSUPPORTED
    assert status(kvq.kvq_workspace_bytes_ex, L, 12, 5000, 1, kernel=5) == kvq.KVQ_ERR_INVALID_ARG
    assert status(kvq.kvq_workspace_bytes_ex, kvq.Layout(2, 256, 64, 100), 12, 5000, 1,
                  kernel=4) == kvq.KVQ_ERR_INVALID_ARG
    assert kvq.kvq_decode_attn_batch_workspace_bytes(L, [100, 200], 12, 1) > 0            # batched decode
    assert status(kvq.kvq_decode_attn_batch_workspace_bytes, L, [100, 200], 12, 3) == kvq.KVQ_ERR_UNSUPPORTED


def test_hadamard_arguments():
    """kvq_hadamard rejects every bad argument before touching the GPU."""
    lib = kvq.lib()
    for dim in (0, 1, 3, 96, 2048):
        assert lib.kvq_hadamard(FAKE, 4, dim, None) == kvq.KVQ_ERR_INVALID_ARG, dim
    assert lib.kvq_hadamard(FAKE, -1, 64, None) == kvq.KVQ_ERR_INVALID_ARG
    assert lib.kvq_hadamard(FAKE, 1 << 31, 64, None) == kvq.KVQ_ERR_INVALID_ARG
    # one thread per pair of values: n_rows * dim / 2 must stay below 2^32
    assert lib.kvq_hadamard(FAKE, 1 << 23, 1024, None) == kvq.KVQ_ERR_INVALID_ARG      # exactly 2^32
    assert "2^32" in kvq.lib().kvq_last_error().decode()
    assert lib.kvq_hadamard(FAKE, 1 << 30, 8, None) == kvq.KVQ_ERR_INVALID_ARG         # 2^32 again, small dim
    assert lib.kvq_hadamard(None, 4, 64, None) == kvq.KVQ_ERR_INVALID_ARG
    assert lib.kvq_hadamard(ctypes.c_void_p(0x100002), 4, 64, None) == kvq.KVQ_ERR_INVALID_ARG   # misaligned
    assert lib.kvq_hadamard(None, 0, 64, None) == kvq.KVQ_OK                                    # no-op


def test_status_strings():
    lib = kvq.lib()
    for st, name in [(0, "KVQ_OK"), (-1, "KVQ_ERR_INVALID_ARG"), (-2, "KVQ_ERR_UNSUPPORTED"),
                     (-3, "KVQ_ERR_WORKSPACE"), (-4, "KVQ_ERR_CAPACITY"), (-5, "KVQ_ERR_HIP")]:
        assert lib.kvq_status_str(st).decode() == name


def test_binding_raises():
    with pytest.raises(kvq.KvqError) as e:
        kvq.kvq_pool_bytes(kvq.Layout(4, 100, 256, 1))
    assert e.value.status == kvq.KVQ_ERR_UNSUPPORTED


def test_noalloc_rejects_steps_beyond_its_scratch():
    """kvq_append_attn_noalloc checks on the host that the step's partials fit
    its static scratch and refuses, before any GPU call, when they do not."""
    lib = kvq.lib()
    cap = kvq.kvq_noalloc_scratch_bytes()
    assert cap == 8 << 20
    L = kvq.Layout(4, 256, 256, 2048)
    # 8 queries x 64 heads: 512 rows of 64 splits of 1 KiB partials, over 8 MiB
    assert kvq.kvq_append_attn_workspace_bytes(L, 64, 262000, 8) > cap
    st = lib.kvq_append_attn_noalloc(ctypes.byref(L), FAKE, FAKE, 2048, 262000, 8, FAKE, FAKE, 64, FAKE,
                                     ctypes.c_float(0.0625), FAKE, None, None, None)
    assert st == kvq.KVQ_ERR_WORKSPACE
    assert "static scratch" in lib.kvq_last_error().decode()
    # bad arguments are refused as by kvq_append_attn, before the size check
    assert lib.kvq_append_attn_noalloc(ctypes.byref(L), FAKE, FAKE, 2048, 100, 0, FAKE, FAKE, 24, FAKE,
                                       ctypes.c_float(0.0625), FAKE, None, None, None) == kvq.KVQ_ERR_INVALID_ARG
    # the decode workload's step fits
    assert kvq.kvq_append_attn_workspace_bytes(L, 24, 262143, 1) <= cap


def _ws_expected(rows, parts, D):
    """Workspace of `parts` partials per row: acc [rows][parts][D] floats,
    then m and l [rows][parts] floats, each rounded up to 256 bytes."""
    ml = (rows * parts * 4 + 255) // 256 * 256
    return rows * parts * D * 4 + 2 * ml


def test_int2_fused_step_plan():
    """kvq_append_attn over the INT2 codec: with cached keys and at most 16
    query rows per KV head the step is fused (the split kernel's partials
    over the cached keys plus one partial per new row); without cached keys,
    or with more rows, it is kvq_append followed by the attention call, whose
    workspace it then asks for."""
    D, n_kv, n_heads = 256, 4, 24
    L = kvq.Layout(n_kv, D, 256, 1100, kvq.KVQ_CODEC_INT2)
    pos0 = 262143
    # the attention plan over the cached keys alone gives the split count
    attn = kvq.kvq_workspace_bytes_ex(L, n_heads, pos0, 1, kernel=4)
    rows = 1 * n_heads
    splits = [s for s in range(1, 4097) if _ws_expected(rows, s, D) == attn]
    assert len(splits) == 1
    fused = kvq.kvq_append_attn_workspace_bytes(L, n_heads, pos0, 1)
    assert fused == _ws_expected(rows, splits[0] + 1, D)
    # no cached keys: kvq_append, then attention over the one new key
    assert kvq.kvq_append_attn_workspace_bytes(L, n_heads, 0, 1) == kvq.kvq_workspace_bytes_ex(L, n_heads, 1, 1)
    # 18 rows per KV head (three queries, group 6: past the INT2 streaming
    # kernel's 16): not fused
    assert kvq.kvq_append_attn_workspace_bytes(L, n_heads, 5000, 3) == kvq.kvq_workspace_bytes_ex(L, n_heads, 5003, 3)
    # 12 rows (two queries, group 6): fused
    a12 = kvq.kvq_workspace_bytes_ex(L, n_heads, 5000, 2, kernel=4)
    s12 = [s for s in range(1, 4097) if _ws_expected(2 * n_heads, s, D) == a12]
    assert len(s12) == 1
    assert kvq.kvq_append_attn_workspace_bytes(L, n_heads, 5000, 2) == _ws_expected(2 * n_heads, s12[0] + 2, D)
    # 8 rows (four queries, group 2) with kernel 4 asked for: fused
    L2 = kvq.Layout(2, 128, 32, 300, kvq.KVQ_CODEC_INT2)
    a2 = kvq.kvq_workspace_bytes_ex(L2, 4, 901, 4, kernel=4)
    s2 = [s for s in range(1, 4097) if _ws_expected(16, s, 128) == a2]
    assert len(s2) == 1
    assert kvq.kvq_append_attn_workspace_bytes(L2, 4, 901, 4, kernel=4) == _ws_expected(16, s2[0] + 4, 128)
