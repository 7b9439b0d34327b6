"""GPU: the fused decode step kvq_append_attn -- append n_new rows at pos0,
then attend the n_new queries over the pos0 + n_new keys.

Checked against the oracle on the same seeded fp32 rows:
  * afterwards the pool holds the oracle's codes and scales for every
    position, the new rows included, bit for bit, whatever bytes the pool held
    before (it starts filled with 0xFF);
  * outputs and lse of every query row, to the attention tolerance;
  * the other kernel choices (VALU, LDS-tiled) give the same through
    kvq_append + attention;
  * edges: pos0 = 0 (no cached keys), odd pos0 (the first new V nibble shares
    its byte with a cached row), new rows across chunk and page edges,
    n_new = 1..8, GQA groups 1..8, head_dim 64 / 128 / 256, shuffled pages;
  * a page-table entry outside the pool for a new row: NaN, no fault, and
    nothing written for that row.
"""
import math

import numpy as np
import pytest

import oracle
from tests import kvq_testutil as tu

pytestmark = pytest.mark.gpu


def _run(seed, D, n_kv, G, P, pos0, n_new, kernel=0, perm_seed=None, bad_new_page=False, outliers=False):
    import torch
    import attention_quantized_kv_amd as kvq
    rng = np.random.default_rng(seed)
    ctx = pos0 + n_new
    n_heads = n_kv * G
    k = rng.standard_normal((ctx, n_kv, D)).astype(np.float32)
    v = rng.standard_normal((ctx, n_kv, D)).astype(np.float32)
    if outliers:
        k[rng.random(k.shape) < 0.01] *= 20
        v[rng.random(v.shape) < 0.01] *= 20
    q = rng.standard_normal((n_new, n_heads, D)).astype(np.float32)
    n_pages = (ctx + P - 1) // P + 3
    L = tu.layout(n_kv, D, P, n_pages)
    pool = tu.alloc_pool(L, fill=0xFF)
    pt_dev, pt = tu.page_table_for(ctx, P, n_pages, perm_seed)
    if pos0 > 0:
        kvq.kvq_append(L, pool, pt_dev, 0, torch.from_numpy(k[:pos0]).cuda(), torch.from_numpy(v[:pos0]).cuda())
    if bad_new_page:
        pt_dev = pt_dev.clone()
        pt_dev[(ctx - 1) // P] = n_pages + 7
    out = torch.full((n_new, n_heads, D), float("nan"), device="cuda")
    lse = torch.full((n_new, n_heads), float("nan"), device="cuda")
    nbytes = kvq.kvq_append_attn_workspace_bytes(L, n_heads, pos0, n_new, kernel=kernel)
    ws = torch.empty(max(nbytes, 256), dtype=torch.uint8, device="cuda")
    scale = 1.0 / math.sqrt(D)
    kvq.kvq_append_attn(L, pool, pt_dev, pos0, torch.from_numpy(k[pos0:]).cuda(),
                        torch.from_numpy(v[pos0:]).cuda(), torch.from_numpy(q).cuda(), scale, out, lse, ws,
                        kernel=kernel)
    torch.cuda.synchronize()
    return k, v, q, scale, L, pool.cpu().numpy(), pt, out.cpu().numpy(), lse.cpu().numpy()


def _check_pool(k, v, L, pool_np, pt, ctx):
    kc, ks, vc, vs = tu.decode_pool(pool_np, L, pt, ctx)
    okc, oks = oracle.quantize_q8_0(k)
    ovc, ovs = oracle.quantize_q4_0(v)
    assert np.array_equal(ks, oks), f"K scales differ at {np.argwhere(ks != oks)[:5]}"
    assert np.array_equal(kc, okc), f"K codes differ at {np.argwhere(kc != okc)[:5]}"
    assert np.array_equal(vs, ovs), f"V scales differ at {np.argwhere(vs != ovs)[:5]}"
    assert np.array_equal(vc, ovc), f"V codes differ at {np.argwhere(vc != ovc)[:5]}"


CASES = [
    # seed, D, n_kv, G, P, pos0, n_new
    (1, 64, 1, 2, 64, 0, 1),          # no cached keys
    (2, 64, 2, 1, 32, 1, 1),          # odd pos0, one cached key
    (3, 128, 2, 4, 64, 255, 1),       # odd pos0, new row opens a page
    (4, 128, 1, 8, 128, 300, 8),      # 8 new rows, 64 rows per KV head
    (5, 256, 4, 6, 256, 4095, 1),     # decode shape, odd pos0 at a page edge
    (6, 256, 2, 6, 256, 1000, 4),     # verify shape
    (7, 256, 1, 4, 32, 61, 7),        # new rows across a chunk and a page edge
    (8, 64, 3, 5, 96, 190, 3),        # page size not a power of two
    (9, 256, 4, 6, 256, 0, 4),        # verify with no cached keys
    (10, 256, 4, 6, 256, 131072, 4),  # the verify workload's positions (two pairs of new rows)
    (12, 128, 3, 2, 64, 33, 8),       # odd pos0, 8 rows: three pairs of new rows, the last row alone
]


@pytest.mark.parametrize("case", CASES, ids=[f"D{c[1]}_g{c[3]}_P{c[4]}_pos{c[5]}_n{c[6]}" for c in CASES])
def test_fused_step_matches_oracle(case):
    seed, D, n_kv, G, P, pos0, n_new = case
    k, v, q, scale, L, pool_np, pt, out, lse = _run(seed, D, n_kv, G, P, pos0, n_new,
                                                    perm_seed=seed if seed % 2 else None)
    _check_pool(k, v, L, pool_np, pt, pos0 + n_new)
    ref, ref_lse, _ = oracle.attention(q, oracle.QuantCache.from_float(k, v), scale)
    tu.assert_close(out, ref, lse, ref_lse, f"fused step {case}")


def test_fused_step_outliers():
    k, v, q, scale, L, pool_np, pt, out, lse = _run(11, 256, 2, 6, 256, 2047, 2, outliers=True)
    _check_pool(k, v, L, pool_np, pt, 2049)
    ref, ref_lse, _ = oracle.attention(q, oracle.QuantCache.from_float(k, v), scale)
    tu.assert_close(out, ref, lse, ref_lse, "fused step, outliers x20")


@pytest.mark.parametrize("kernel", [1, 3])
def test_other_kernels_append_then_attend(kernel):
    k, v, q, scale, L, pool_np, pt, out, lse = _run(21, 128, 2, 3, 64, 517, 3, kernel=kernel)
    _check_pool(k, v, L, pool_np, pt, 520)
    ref, ref_lse, _ = oracle.attention(q, oracle.QuantCache.from_float(k, v), scale)
    tu.assert_close(out, ref, lse, ref_lse, f"kernel {kernel} append + attention")


def test_new_row_page_outside_pool_gives_nan():
    D, P, pos0, n_new = 64, 64, 128, 2         # the new rows open page 2, which is made invalid
    k, v, q, scale, L, pool_np, pt, out, lse = _run(31, D, 1, 2, P, pos0, n_new, bad_new_page=True)
    assert np.isnan(out).all() and np.isnan(lse).all()
    # the cached rows are intact; the page the table would have used was not touched
    kc, ks, vc, vs = tu.decode_pool(pool_np, L, pt, pos0)
    okc, oks = oracle.quantize_q8_0(k[:pos0])
    assert np.array_equal(kc, okc) and np.array_equal(ks, oks)
    ub = tu.unit_bytes(D, P)
    phys = int(pt[pos0 // P])
    assert (pool_np[phys * ub:(phys + 1) * ub] == 0xFF).all()


def test_rejects_bad_arguments():
    import torch
    import attention_quantized_kv_amd as kvq
    L = tu.layout(1, 64, 64, 4)
    pool = tu.alloc_pool(L)
    pt_dev, _ = tu.page_table_for(256, 64, 4)
    q = torch.zeros(9, 2, 64, device="cuda")
    kv = torch.zeros(9, 1, 64, device="cuda")
    out = torch.zeros_like(q)
    with pytest.raises(kvq.KvqError) as e:          # 9 new rows > KVQ_MAX_NQ_DECODE
        kvq.kvq_append_attn(L, pool, pt_dev, 0, kv, kv, q, 0.125, out)
    assert e.value.status == kvq.KVQ_ERR_INVALID_ARG
    q1, kv1, out1 = q[:1], kv[:1], out[:1]
    with pytest.raises(kvq.KvqError) as e:          # position 256 is past the page table
        kvq.kvq_append_attn(L, pool, pt_dev, 256, kv1, kv1, q1, 0.125, out1)
    assert e.value.status == kvq.KVQ_ERR_CAPACITY


def test_workspace_garbage_and_reuse():
    """The streaming kernel's arrival counters live in the workspace: any old
    bytes there (random, or the previous call's counters) must not matter."""
    import torch
    import attention_quantized_kv_amd as kvq
    rng = np.random.default_rng(41)
    D, n_kv, G, P, ctx = 128, 2, 4, 64, 3000
    k = rng.standard_normal((ctx, n_kv, D)).astype(np.float32)
    v = rng.standard_normal((ctx, n_kv, D)).astype(np.float32)
    L = tu.layout(n_kv, D, P, (ctx + P - 1) // P)
    pool = tu.alloc_pool(L)
    pt_dev, _ = tu.page_table_for(ctx, P, L.n_pages)
    kvq.kvq_append(L, pool, pt_dev, 0, torch.from_numpy(k).cuda(), torch.from_numpy(v).cuda())
    cache = oracle.QuantCache.from_float(k, v)
    nbytes = kvq.kvq_workspace_bytes(L, n_kv * G, ctx, 1)
    ws = torch.from_numpy(rng.integers(0, 256, nbytes, dtype=np.uint8)).cuda()
    for it in range(3):
        q = rng.standard_normal((1, n_kv * G, D)).astype(np.float32)
        out = torch.full((1, n_kv * G, D), float("nan"), device="cuda")
        lse = torch.full((1, n_kv * G), float("nan"), device="cuda")
        kvq.kvq_decode_attn(L, pool, pt_dev, ctx, torch.from_numpy(q).cuda(), 0.09, out, lse, ws)
        torch.cuda.synchronize()
        ref, ref_lse, _ = oracle.attention(q, cache, 0.09)
        tu.assert_close(out.cpu().numpy(), ref, lse.cpu().numpy(), ref_lse, f"call {it}")
