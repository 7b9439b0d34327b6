"""GPU: kvq_append_attn_noalloc (the decode step with the library's static
device scratch instead of a caller workspace) against kvq_append_attn.

Two calls in a row on one pool and its twin, the second with a smaller input
(a 4-row verify step over 20,000 cached keys, then a 1-row decode step over
5,000 on another sequence), so the scratch holds the first call's partials
when the second runs.  After each call the two pools are identical byte for
byte (the same codes and scales written for the new rows, checked against the
oracle's quantizer too), and the outputs and lse of both calls match the
oracle within |o - ref| <= 2e-3 + 1e-3 |ref| (lse 1e-4 + 1e-5 |ref|) and each
other within the same bound.  The same over the INT2 cache (one decode row
over 20,000 cached keys, then two new rows over 3,000), where the INT2
streaming kernel appends the new rows itself; its pools are checked against
the oracle's INT2 quantizer.
"""
import math

import numpy as np
import pytest

import oracle
from tests import kvq_testutil as tu

pytestmark = pytest.mark.gpu


def _sequence(rng, ctx, n_kv, D):
    k = rng.standard_normal((ctx, n_kv, D)).astype(np.float32)
    v = rng.standard_normal((ctx, n_kv, D)).astype(np.float32)
    return k, v


def test_noalloc_matches_the_workspace_call_twice():
    import torch
    import attention_quantized_kv_amd as kvq
    n_kv, G, D, P = 4, 6, 256, 256
    n_heads = n_kv * G
    rng = np.random.default_rng(2024)
    steps = [(20000, 4), (5000, 1)]          # (cached keys, new rows): the second call is smaller
    n_pages = sum((pos0 + n + P - 1) // P for pos0, n in steps) + 2
    L = tu.layout(n_kv, D, P, n_pages)
    pool_a = tu.alloc_pool(L, fill=0x5A)
    pool_b = tu.alloc_pool(L, fill=0x5A)
    first = 0
    for call, (pos0, n_new) in enumerate(steps):
        ctx = pos0 + n_new
        n_pg = (ctx + P - 1) // P
        pt_np = np.arange(first, first + n_pg, dtype=np.int32)[::-1].copy()   # this sequence's pages, reversed
        first += n_pg
        pt = torch.from_numpy(pt_np).cuda()
        k, v = _sequence(rng, ctx, n_kv, D)
        q = rng.standard_normal((n_new, n_heads, D)).astype(np.float32)
        for pool in (pool_a, pool_b):
            kvq.kvq_append(L, pool, pt, 0, torch.from_numpy(k[:pos0]).cuda(), torch.from_numpy(v[:pos0]).cuda())
        kn, vn, qd = (torch.from_numpy(x).cuda() for x in (k[pos0:], v[pos0:], q))
        scale = 1.0 / math.sqrt(D)
        out_a = torch.full((n_new, n_heads, D), float("nan"), device="cuda")
        lse_a = torch.full((n_new, n_heads), float("nan"), device="cuda")
        out_b, lse_b = out_a.clone(), lse_a.clone()
        ws = torch.empty(max(kvq.kvq_append_attn_workspace_bytes(L, n_heads, pos0, n_new), 256), dtype=torch.uint8,
                         device="cuda")
        assert kvq.kvq_append_attn_workspace_bytes(L, n_heads, pos0, n_new) <= kvq.kvq_noalloc_scratch_bytes()
        kvq.kvq_append_attn(L, pool_a, pt, pos0, kn, vn, qd, scale, out_a, lse_a, ws)
        kvq.kvq_append_attn_noalloc(L, pool_b, pt, pos0, kn, vn, qd, scale, out_b, lse_b)
        torch.cuda.synchronize()
        assert torch.equal(pool_a, pool_b), f"call {call}: pools differ"
        kc, ks, vc, vs = tu.decode_pool(pool_b.cpu().numpy(), L, pt_np, ctx)
        okc, oks = oracle.quantize_q8_0(k)
        ovc, ovs = oracle.quantize_q4_0(v)
        assert np.array_equal(kc, okc) and np.array_equal(ks, oks), f"call {call}: K codes/scales"
        assert np.array_equal(vc, ovc) and np.array_equal(vs, ovs), f"call {call}: V codes/scales"
        ref, ref_lse, _ = oracle.attention(q, oracle.QuantCache.from_float(k, v), scale)
        a, la, b, lb = out_a.cpu().numpy(), lse_a.cpu().numpy(), out_b.cpu().numpy(), lse_b.cpu().numpy()
        tu.assert_close(a, ref, la, ref_lse, f"call {call}: kvq_append_attn")
        tu.assert_close(b, ref, lb, ref_lse, f"call {call}: kvq_append_attn_noalloc")
        tu.assert_close(b, a, lb, la, f"call {call}: noalloc vs workspace call")


def test_noalloc_int2_fused_step_twice():
    """The same over the INT2 cache, where the INT2 streaming kernel appends
    the new rows itself (up to 8 query rows per KV head): one decode row over
    20,000 cached keys, then two new rows over 3,000 on another sequence."""
    import torch
    import attention_quantized_kv_amd as kvq
    n_kv, G, D, P = 4, 4, 256, 256
    n_heads = n_kv * G
    rng = np.random.default_rng(2025)
    steps = [(20000, 1), (3000, 2)]
    n_pages = sum((pos0 + n + P - 1) // P for pos0, n in steps) + 2
    L = tu.layout(n_kv, D, P, n_pages, codec=kvq.KVQ_CODEC_INT2)
    pool_a = tu.alloc_pool(L, fill=0x5A)
    pool_b = tu.alloc_pool(L, fill=0x5A)
    first = 0
    for call, (pos0, n_new) in enumerate(steps):
        ctx = pos0 + n_new
        n_pg = (ctx + P - 1) // P
        pt_np = np.arange(first, first + n_pg, dtype=np.int32)[::-1].copy()
        first += n_pg
        pt = torch.from_numpy(pt_np).cuda()
        k, v = _sequence(rng, ctx, n_kv, D)
        q = rng.standard_normal((n_new, n_heads, D)).astype(np.float32)
        for pool in (pool_a, pool_b):
            kvq.kvq_append(L, pool, pt, 0, torch.from_numpy(k[:pos0]).cuda(), torch.from_numpy(v[:pos0]).cuda())
        kn, vn, qd = (torch.from_numpy(x).cuda() for x in (k[pos0:], v[pos0:], q))
        scale = 1.0 / math.sqrt(D)
        out_a = torch.full((n_new, n_heads, D), float("nan"), device="cuda")
        lse_a = torch.full((n_new, n_heads), float("nan"), device="cuda")
        out_b, lse_b = out_a.clone(), lse_a.clone()
        need = kvq.kvq_append_attn_workspace_bytes(L, n_heads, pos0, n_new)
        assert need <= kvq.kvq_noalloc_scratch_bytes()
        ws = torch.empty(max(need, 256), dtype=torch.uint8, device="cuda")
        kvq.kvq_append_attn(L, pool_a, pt, pos0, kn, vn, qd, scale, out_a, lse_a, ws)
        kvq.kvq_append_attn_noalloc(L, pool_b, pt, pos0, kn, vn, qd, scale, out_b, lse_b)
        torch.cuda.synchronize()
        assert torch.equal(pool_a, pool_b), f"call {call}: pools differ"
        got = tu.decode_pool_int2(pool_b.cpu().numpy(), L, pt_np, ctx)
        want = oracle.quantize_int2(k) + oracle.quantize_int2(v)
        for name, g_, w_ in zip(("K codes", "K scales", "K zeros", "V codes", "V scales", "V zeros"), got, want):
            assert np.array_equal(g_, w_.reshape(g_.shape)), f"call {call}: {name}"
        ref, ref_lse, _ = oracle.attention(q, oracle.Int2Cache.from_float(k, v), scale)
        a, la, b, lb = out_a.cpu().numpy(), lse_a.cpu().numpy(), out_b.cpu().numpy(), lse_b.cpu().numpy()
        tu.assert_close(a, ref, la, ref_lse, f"call {call}: kvq_append_attn")
        tu.assert_close(b, ref, lb, ref_lse, f"call {call}: kvq_append_attn_noalloc")
        tu.assert_close(b, a, lb, la, f"call {call}: noalloc vs workspace call")
