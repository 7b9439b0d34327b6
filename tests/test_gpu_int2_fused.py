"""GPU: the fused decode step over the INT2 cache (kvq_append_attn with up to
16 query rows per KV head and cached keys before the new rows), where the INT2
streaming kernel also quantizes the new rows into the pool and scores them.

For every case the pool after the fused step must equal, byte for byte, the
pool after kvq_append of the same rows (the new rows' codes, scales and
zero-points, and the untouched codes of the other tokens that share their V
dwords), and the output must match the oracle's fp64 attention over the
whole cache (cached keys plus the new rows, causal among the new rows).
Cases: one decode row over four KV heads, several new rows spanning two
8-token groups, a new-row run across a page boundary, head_dim 128 and 256,
a single cached key, eight new rows with group 1, 12 and 16 query rows (two
per wave in the end phase), a split count forced low
(many chunks per wave), and a bad page entry for the new rows (NaN, nothing
written).
"""
import numpy as np
import pytest

import oracle
from tests import kvq_testutil as tu

pytestmark = pytest.mark.gpu


def _setup(seed, D, P, pos0, n_new, n_kv, G, outliers=False):
    import torch
    import attention_quantized_kv_amd as kvq
    rng = np.random.default_rng(seed)
    n = pos0 + n_new
    k = rng.standard_normal((n, n_kv, D)).astype(np.float32)
    v = rng.standard_normal((n, n_kv, D)).astype(np.float32)
    if outliers:
        k[rng.random(k.shape) < 0.01] *= 20
        v[rng.random(v.shape) < 0.01] *= 20
    q = rng.standard_normal((n_new, n_kv * G, D)).astype(np.float32)
    n_pages = (n + P - 1) // P + 3
    L = tu.layout(n_kv, D, P, n_pages, codec=kvq.KVQ_CODEC_INT2)
    pool = tu.alloc_pool(L, fill=0xFF)          # unwritten slots read as NaN scales
    pt_dev, pt = tu.page_table_for(n, P, n_pages, seed)
    kvq.kvq_append(L, pool, pt_dev, 0, torch.from_numpy(k[:pos0]).cuda(), torch.from_numpy(v[:pos0]).cuda())
    torch.cuda.synchronize()
    return k, v, q, L, pool, pt_dev, pt


def _step(L, pool, pt_dev, pos0, k_new, v_new, q, scale, cps=0):
    import torch
    import attention_quantized_kv_amd as kvq
    n_new, n_heads, D = q.shape
    out = torch.full((n_new, n_heads, D), float("nan"), device="cuda")
    lse = torch.full((n_new, n_heads), float("nan"), device="cuda")
    opts = dict(kernel=4, chunks_per_split=cps) if cps else {}
    ws = torch.empty(max(1, kvq.kvq_append_attn_workspace_bytes(L, n_heads, pos0, n_new, **opts)),
                     dtype=torch.uint8, device="cuda")
    kvq.kvq_append_attn(L, pool, pt_dev, pos0, torch.from_numpy(k_new).cuda(), torch.from_numpy(v_new).cuda(),
                        torch.from_numpy(q).cuda(), scale, out, lse, ws, **opts)
    torch.cuda.synchronize()
    return out.cpu().numpy(), lse.cpu().numpy()


@pytest.mark.parametrize("seed,D,P,pos0,n_new,n_kv,G,cps", [
    (1, 256, 256, 3000, 1, 4, 6, 0),       # one decode row, GQA 6, four KV heads
    (2, 128, 32, 901, 4, 2, 2, 0),         # 8 rows; new rows 901..904 span two 8-token groups
    (3, 256, 64, 638, 3, 1, 2, 0),         # new rows 638..640 across a page boundary
    (4, 128, 32, 1, 8, 2, 1, 0),           # a single cached key, eight new rows
    (5, 256, 32, 20000, 1, 2, 8, 40),      # group 8; few splits, many chunks per wave
    (6, 128, 64, 4093, 2, 1, 4, 0),        # ragged last chunk, causal pair
    (9, 256, 64, 5000, 2, 2, 6, 0),        # 12 rows: the 16-row layout, two query rows per wave
    (10, 128, 32, 1234, 4, 1, 4, 0),       # 16 rows, four causal new rows in one group
    (11, 256, 256, 30000, 2, 4, 8, 0),     # 16 rows over four KV heads
])
def test_int2_fused_step_matches_append_and_oracle(seed, D, P, pos0, n_new, n_kv, G, cps):
    import torch
    import attention_quantized_kv_amd as kvq
    k, v, q, L, pool, pt_dev, pt = _setup(seed, D, P, pos0, n_new, n_kv, G, outliers=seed % 2 == 0)
    ref_pool = pool.clone()
    kvq.kvq_append(L, ref_pool, pt_dev, pos0, torch.from_numpy(k[pos0:]).cuda(), torch.from_numpy(v[pos0:]).cuda())
    torch.cuda.synchronize()
    out, lse = _step(L, pool, pt_dev, pos0, k[pos0:], v[pos0:], q, 0.0625, cps)
    got, want = pool.cpu().numpy(), ref_pool.cpu().numpy()
    if not np.array_equal(got, want):
        i = np.flatnonzero(got != want)
        raise AssertionError(f"pool differs from kvq_append's at {i.size} bytes, first {i[:8]}")
    ref, ref_lse, _ = oracle.attention(q, oracle.Int2Cache.from_float(k, v), 0.0625)
    tu.assert_close(out, ref, lse, ref_lse, "fused INT2 decode step")


def test_int2_fused_step_bad_page():
    """The new rows' page entry lies outside the pool: every query sees new
    row 0, so every output is NaN, and the pool is left as it was."""
    import torch
    pos0, n_new, D, P = 512, 2, 256, 256      # the new rows start page 2
    k, v, q, L, pool, pt_dev, pt = _setup(7, D, P, pos0, n_new, 2, 3)
    bad = pt.copy()
    bad[pos0 // P] = L.n_pages + 5
    bad_dev = torch.from_numpy(bad.astype(np.int32)).cuda()
    before = pool.cpu().numpy()
    out, lse = _step(L, pool, bad_dev, pos0, k[pos0:], v[pos0:], q, 0.0625)
    assert np.isnan(out).all() and np.isnan(lse).all()
    assert np.array_equal(pool.cpu().numpy(), before)


def test_int2_fused_step_repeated():
    """Three fused steps in a row, each appending one row after the last:
    the pool matches three kvq_append calls and every step's output matches
    the oracle over the cache so far."""
    import torch
    import attention_quantized_kv_amd as kvq
    pos0, D, P, n_kv, G = 765, 128, 32, 2, 6
    k, v, _, L, pool, pt_dev, _ = _setup(8, D, P, pos0, 3, n_kv, G)
    ref_pool = pool.clone()
    rng = np.random.default_rng(9)
    for s in range(3):
        p = pos0 + s
        qs = rng.standard_normal((1, n_kv * G, D)).astype(np.float32)
        out, lse = _step(L, pool, pt_dev, p, k[p:p + 1], v[p:p + 1], qs, 0.08)
        kvq.kvq_append(L, ref_pool, pt_dev, p, torch.from_numpy(k[p:p + 1]).cuda(),
                       torch.from_numpy(v[p:p + 1]).cuda())
        torch.cuda.synchronize()
        assert np.array_equal(pool.cpu().numpy(), ref_pool.cpu().numpy()), f"step {s}: pool differs"
        ref, ref_lse, _ = oracle.attention(qs, oracle.Int2Cache.from_float(k[:p + 1], v[:p + 1]), 0.08)
        tu.assert_close(out, ref, lse, ref_lse, f"fused INT2 step {s}")
