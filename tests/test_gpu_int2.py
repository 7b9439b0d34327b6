"""GPU: the INT2 cache codec (K and V both 2-bit, 128-value blocks with an
fp16 scale and zero-point) against the oracle.

kvq_append with codec KVQ_CODEC_INT2 must leave, for every position, the
oracle's codes, scales and zero-points bit for bit (decoded from the pool
with the header's layout), for ragged appends (groups of 8 positions cut at
both ends, across chunks and pages), shuffled pages, head_dim 128 and 256,
outliers, and a pool that starts full of other bytes.
"""
import numpy as np
import pytest

import oracle
from tests import kvq_testutil as tu

pytestmark = pytest.mark.gpu


def _fill(seed, ctx, n_kv, D, P, cuts, perm=True, outliers=False):
    import torch
    import attention_quantized_kv_amd as kvq
    rng = np.random.default_rng(seed)
    k = rng.standard_normal((ctx, n_kv, D)).astype(np.float32)
    v = rng.standard_normal((ctx, n_kv, D)).astype(np.float32)
    if outliers:
        k[rng.random(k.shape) < 0.01] *= 20
        v[rng.random(v.shape) < 0.01] *= 20
    n_pages = (ctx + P - 1) // P + 2
    L = tu.layout(n_kv, D, P, n_pages, codec=kvq.KVQ_CODEC_INT2)
    pool = tu.alloc_pool(L, fill=0xA5)
    pt_dev, pt = tu.page_table_for(ctx, P, n_pages, seed if perm else None)
    edges = [0] + list(cuts) + [ctx]
    for a, b in zip(edges[:-1], edges[1:]):
        if b > a:
            kvq.kvq_append(L, pool, pt_dev, a, torch.from_numpy(k[a:b]).cuda(), torch.from_numpy(v[a:b]).cuda())
    torch.cuda.synchronize()
    return k, v, L, pool.cpu().numpy(), pt


@pytest.mark.parametrize("D,P,ctx,cuts", [
    (128, 32, 200, [5, 13, 64, 65, 130]),     # group and chunk edges cut
    (256, 64, 300, [1, 2, 3, 100, 257]),
    (256, 256, 700, [256, 511]),
])
def test_append_int2_bit_exact(D, P, ctx, cuts):
    k, v, L, pool_np, pt = _fill(7 + D + ctx, ctx, 2, D, P, cuts)
    kc, ks, kz, vc, vs, vz = tu.decode_pool_int2(pool_np, L, pt, ctx)
    okc, oks, okz = oracle.quantize_int2(k)
    ovc, ovs, ovz = oracle.quantize_int2(v)
    for name, got, want in (("K codes", kc, okc), ("K scales", ks, oks), ("K zeros", kz, okz),
                            ("V codes", vc, ovc), ("V scales", vs, ovs), ("V zeros", vz, ovz)):
        assert np.array_equal(got, want), f"{name} differ at {np.argwhere(got != want)[:5]}"


def test_append_int2_outliers_bit_exact():
    k, v, L, pool_np, pt = _fill(3, 160, 1, 256, 32, [33], outliers=True)
    kc, ks, kz, vc, vs, vz = tu.decode_pool_int2(pool_np, L, pt, 160)
    okc, oks, okz = oracle.quantize_int2(k)
    ovc, ovs, ovz = oracle.quantize_int2(v)
    assert np.array_equal(kc, okc) and np.array_equal(ks, oks) and np.array_equal(kz, okz)
    assert np.array_equal(vc, ovc) and np.array_equal(vs, ovs) and np.array_equal(vz, ovz)
