"""GPU: the workloads at their full sizes, in the launch configuration the
benchmark times (automatic kernel and split plan, in-order page table, cache
filled by kvq_append in chunks and the new rows appended at their position;
for the decode and verify workloads also through the fused decode step,
kvq_append_attn, which appends the new rows and attends in one call).

Inputs come from the seeded host generators (synth), so the oracle sees the
same fp32 values.  Checked against the oracle:
  * K/V codes and scales of sampled pages (first, middle, the appended tail),
    bit for bit;
  * for the 2-bit cache (int2decode262k, also through the fused step, and
    int2prefill262k: K and V INT2, decoded with the header's layout) codes,
    scales and zero-points of sampled pages (the appended tail among them),
    bit for bit, and the outputs of every query row (decode) or of the
    sampled rows (prefill);
  * attention outputs and lse of every query row for the decode and verify
    workloads, and of sampled rows (first and last queries of the chunk, the
    page edges 255/256, seeded random ones; heads of every KV group) for the
    prefill chunk, to |o - ref| <= 2e-3 + 1e-3 |ref| and lse to 1e-4 + 1e-5 |ref|.
"""
import numpy as np
import pytest

import oracle
import synth
from tests import kvq_testutil as tu

pytestmark = pytest.mark.gpu

FILL_CHUNK = 16384


def _run(w, fused=False):
    import torch
    import attention_quantized_kv_amd as kvq
    k, v = synth.layer_kv(w, 0)
    q = synth.layer_q(w, 0)
    L = tu.layout(w.n_kv, w.head_dim, w.page_size, w.n_pages, codec=w.codec)
    pool = tu.alloc_pool(L)
    pt_dev, pt = tu.page_table_for(w.ctx, w.page_size, w.n_pages)
    for r in range(0, w.cached, FILL_CHUNK):
        n = min(FILL_CHUNK, w.cached - r)
        kvq.kvq_append(L, pool, pt_dev, r, torch.from_numpy(k[r:r + n]).cuda(), torch.from_numpy(v[r:r + n]).cuda())
    qd = torch.from_numpy(q).cuda()
    out = torch.full((w.n_q, w.n_heads, w.head_dim), float("nan"), device="cuda")
    lse = torch.full((w.n_q, w.n_heads), float("nan"), device="cuda")
    if fused:                                   # the decode step: append + attention in one call
        ws = torch.empty(max(kvq.kvq_append_attn_workspace_bytes(L, w.n_heads, w.cached, w.n_q), 256),
                         dtype=torch.uint8, device="cuda")
        kvq.kvq_append_attn(L, pool, pt_dev, w.cached, torch.from_numpy(k[w.cached:]).cuda(),
                            torch.from_numpy(v[w.cached:]).cuda(), qd, w.scale, out, lse, ws)
        torch.cuda.synchronize()
        return k, v, q, L, pool, pt, out.cpu().numpy(), lse.cpu().numpy()
    kvq.kvq_append(L, pool, pt_dev, w.cached, torch.from_numpy(k[w.cached:]).cuda(),
                   torch.from_numpy(v[w.cached:]).cuda())
    prefill = w.n_q > kvq.KVQ_MAX_NQ_DECODE
    ws = torch.empty(max(kvq.kvq_workspace_bytes(L, w.n_heads, w.ctx, w.n_q, prefill), 1), dtype=torch.uint8,
                     device="cuda")
    fn = kvq.kvq_prefill_attn if prefill else kvq.kvq_decode_attn
    fn(L, pool, pt_dev, w.ctx, qd, w.scale, out, lse, ws)
    torch.cuda.synchronize()
    return k, v, q, L, pool, pt, out.cpu().numpy(), lse.cpu().numpy()


def _check_codes(w, cache, L, pool, pt):
    pool_np = pool.cpu().numpy()
    ub = tu.unit_bytes(w.head_dim, w.page_size)
    for lp in sorted({0, w.n_pages // 2, (w.cached // w.page_size), w.n_pages - 1}):
        for g in range(w.n_kv):
            phys = int(pt[lp])
            unit = pool_np[(phys * w.n_kv + g) * ub:(phys * w.n_kv + g + 1) * ub]
            kc, ks, vc, vs = tu.decode_unit(unit, w.head_dim, w.page_size)
            s0 = lp * w.page_size
            n = min(w.page_size, w.ctx - s0)
            assert np.array_equal(kc[:n], cache.k_codes[s0:s0 + n, g]), f"K codes page {lp} head {g}"
            assert np.array_equal(ks[:n], cache.k_scales[s0:s0 + n, g]), f"K scales page {lp} head {g}"
            assert np.array_equal(vc[:n], cache.v_codes[s0:s0 + n, g]), f"V codes page {lp} head {g}"
            assert np.array_equal(vs[:n], cache.v_scales[s0:s0 + n, g]), f"V scales page {lp} head {g}"


def _rows(w):
    if w.n_q <= 8:
        return [(i, h) for i in range(w.n_q) for h in range(w.n_heads)]
    rng = np.random.default_rng(7)
    qs = sorted({0, 1, 255, 256, w.n_q // 2, w.n_q - 2, w.n_q - 1, *rng.integers(0, w.n_q, 5).tolist()})
    G = w.n_heads // w.n_kv
    hs = sorted({0, G - 1, G, 2 * G + 1, w.n_heads - 1})
    return [(i, h) for i in qs for h in hs]


@pytest.mark.parametrize("name,fused", [("tiny", False), ("decode65k", False), ("decode262k", False),
                                        ("verify131k", False), ("prefill262k", False), ("tiny", True),
                                        ("decode262k", True), ("verify131k", True)])
def test_full_size(name, fused):
    w = synth.WORKLOADS[name]
    k, v, q, L, pool, pt, out, lse = _run(w, fused)
    cache = oracle.QuantCache.from_float(k, v)
    del k, v
    _check_codes(w, cache, L, pool, pt)
    rows = _rows(w)
    ref, ref_lse = oracle.attention(q, cache, w.scale, rows=rows)
    got = np.stack([out[i, h] for i, h in rows])
    got_lse = np.array([lse[i, h] for i, h in rows])
    tu.assert_close(got, ref, got_lse, ref_lse, f"{name}{' fused' if fused else ''} ({len(rows)} rows)")


@pytest.mark.parametrize("name,fused", [("int2decode262k", False), ("int2prefill262k", False),
                                        ("int2decode262k", True)])
def test_full_size_int2(name, fused):
    w = synth.WORKLOADS[name]
    k, v, q, L, pool, pt, out, lse = _run(w, fused)
    cache = oracle.Int2Cache.from_float(k, v)
    del k, v
    pool_np = pool.cpu().numpy()
    names = ("K codes", "K scales", "K zeros", "V codes", "V scales", "V zeros")
    for lp in sorted({0, w.n_pages // 2, w.cached // w.page_size, w.n_pages - 1}):
        s0 = lp * w.page_size
        n = min(w.page_size, w.ctx - s0)
        got = tu.decode_pool_int2(pool_np, L, np.array([pt[lp]], dtype=np.int32), n)
        for name, g, want in zip(names, got, cache.k + cache.v):
            assert np.array_equal(g, want[s0:s0 + n]), f"{name} of page {lp}"
    rows = _rows(w)
    ref, ref_lse = oracle.attention(q, cache, w.scale, rows=rows)
    got = np.stack([out[i, h] for i, h in rows])
    got_lse = np.array([lse[i, h] for i, h in rows])
    tu.assert_close(got, ref, got_lse, ref_lse, f"{name}{' fused' if fused else ''} ({len(rows)} rows)")
