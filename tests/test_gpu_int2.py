"""GPU: the INT2 cache codec (K and V both 2-bit, 128-value blocks with an
fp16 scale and zero-point) against the oracle.

kvq_append with codec KVQ_CODEC_INT2 must leave, for every position, the
oracle's codes, scales and zero-points bit for bit (decoded from the pool
with the header's layout), for ragged appends (groups of 8 positions cut at
both ends, across chunks and pages), shuffled pages, head_dim 128 and 256,
outliers, and a pool that starts full of other bytes.

Decode over the INT2 cache (kernel 4) must match the oracle's fp64 attention
over the dequantized cache within the shared tolerance: a single key, ragged
chunks, up to 8 and up to 16 rows, causal verify rows, many partials, page
entries refetched after 64 chunks of a wave, outliers, prefixes of a longer
cache, split invariance, a bad page (NaN), and append + attention.
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


# ---- attention over the INT2 cache (kernel 4) against the fp64 oracle over
# the dequantized cache

def _attend(L, pool, pt_dev, ctx, q, scale, kernel=0, cps=0):
    import torch
    import attention_quantized_kv_amd as kvq
    n_q, n_heads, D = q.shape
    out = torch.full((n_q, n_heads, D), float("nan"), device="cuda")
    lse = torch.full((n_q, n_heads), float("nan"), device="cuda")
    ws = torch.empty(max(1, kvq.kvq_workspace_bytes_ex(L, n_heads, ctx, n_q, kernel, cps)), dtype=torch.uint8,
                     device="cuda")
    kvq.kvq_attn_ex(L, pool, pt_dev, ctx, torch.from_numpy(q).cuda(), scale, out, lse, ws, kernel=kernel,
                    chunks_per_split=cps)
    torch.cuda.synchronize()
    return out.cpu().numpy(), lse.cpu().numpy()


def _int2_pool(seed, ctx, n_kv, D, P, outliers=False, spare=2):
    import torch
    import attention_quantized_kv_amd as kvq
    rng = np.random.default_rng(seed)
    k = rng.standard_normal((ctx, n_kv, D)).astype(np.float32)
    v = rng.standard_normal((ctx, n_kv, D)).astype(np.float32)
    if outliers:
        k[rng.random(k.shape) < 0.01] *= 20
        v[rng.random(v.shape) < 0.01] *= 20
    n_pages = (ctx + P - 1) // P + spare
    L = tu.layout(n_kv, D, P, n_pages, codec=kvq.KVQ_CODEC_INT2)
    pool = tu.alloc_pool(L, fill=0xFF)          # unwritten slots read as NaN scales
    pt_dev, _ = tu.page_table_for(ctx, P, n_pages, seed)
    kvq.kvq_append(L, pool, pt_dev, 0, torch.from_numpy(k).cuda(), torch.from_numpy(v).cuda())
    return rng, L, pool, pt_dev, oracle.Int2Cache.from_float(k, v)


@pytest.mark.parametrize("D,P,ctx,n_kv,G,n_q,cps", [
    (128, 32, 1, 1, 1, 1, 0),          # a single key
    (128, 32, 31, 2, 4, 1, 0),         # one ragged chunk
    (256, 64, 1000, 2, 6, 1, 0),       # 6 rows: two per lane group
    (256, 256, 5000, 4, 6, 1, 1),      # one chunk per wave: many partials
    (256, 32, 3001, 1, 8, 2, 0),       # 16 rows, causal verify pair
    (128, 64, 777, 2, 16, 1, 0),       # group 16
    (256, 128, 2049, 2, 2, 4, 2),      # 8 rows, causal verify of 4
    (128, 32, 40000, 1, 4, 1, 100),    # ~80 chunks per wave: page entries refetched
])
def test_int2_decode_matches_oracle(D, P, ctx, n_kv, G, n_q, cps):
    rng, L, pool, pt_dev, cache = _int2_pool(11 + ctx + D, ctx, n_kv, D, P)
    q = rng.standard_normal((n_q, n_kv * G, D)).astype(np.float32)
    scale = 1.0 / np.sqrt(D)
    out, lse = _attend(L, pool, pt_dev, ctx, q, scale, cps=cps)
    ref, ref_lse, _ = oracle.attention(q, cache, scale)
    tu.assert_close(out, ref, lse, ref_lse, f"INT2 D={D} P={P} ctx={ctx} G={G} n_q={n_q} cps={cps}")


def test_int2_decode_outliers_and_prefix():
    """Outlier channels (wide blocks), and attention over a prefix of the
    cache (keys past ctx hold data that must not be read as keys)."""
    rng, L, pool, pt_dev, cache = _int2_pool(5, 4100, 2, 256, 64, outliers=True)
    q = rng.standard_normal((1, 12, 256)).astype(np.float32) * 2
    for ctx in (4100, 4097, 33):
        out, lse = _attend(L, pool, pt_dev, ctx, q, 0.0625)
        ref, ref_lse, _ = oracle.attention(q, cache, 0.0625, ctx=ctx)
        tu.assert_close(out, ref, lse, ref_lse, f"INT2 outliers ctx={ctx}")


def test_int2_split_invariance():
    """Every split of the keys gives the oracle's result.  (Splits differ from
    one another by more than fp32 rounding: each partial rounds its weights
    p * d to fp16 against its own running maximum.)"""
    rng, L, pool, pt_dev, cache = _int2_pool(9, 6000, 2, 128, 32)
    q = rng.standard_normal((1, 8, 128)).astype(np.float32)
    ref, ref_lse, _ = oracle.attention(q, cache, 0.1)
    for c in (0, 1, 3, 24, 188):
        out, lse = _attend(L, pool, pt_dev, 6000, q, 0.1, kernel=4, cps=c)
        tu.assert_close(out, ref, lse, ref_lse, f"INT2 chunks_per_split={c}")


def test_int2_bad_page_gives_nan():
    rng, L, pool, pt_dev, cache = _int2_pool(4, 3000, 2, 256, 64)
    bad = pt_dev.clone()
    bad[20] = L.n_pages + 7
    q = rng.standard_normal((1, 4, 256)).astype(np.float32)
    out, lse = _attend(L, pool, bad, 3000, q, 0.0625)
    assert np.isnan(out).all() and np.isnan(lse).all()


def test_int2_append_attn():
    """kvq_append_attn over the INT2 codec: append, then decode."""
    import torch
    import attention_quantized_kv_amd as kvq
    rng, L, pool, pt_dev, cache = _int2_pool(6, 900, 1, 128, 32, spare=3)
    k_new = rng.standard_normal((2, 1, 128)).astype(np.float32)
    v_new = rng.standard_normal((2, 1, 128)).astype(np.float32)
    q = rng.standard_normal((2, 6, 128)).astype(np.float32)
    out = torch.empty((2, 6, 128), device="cuda")
    lse = torch.empty((2, 6), device="cuda")
    ws = torch.empty(max(1, kvq.kvq_append_attn_workspace_bytes(L, 6, 900, 2)), dtype=torch.uint8, device="cuda")
    kvq.kvq_append_attn(L, pool, pt_dev, 900, torch.from_numpy(k_new).cuda(), torch.from_numpy(v_new).cuda(),
                        torch.from_numpy(q).cuda(), 0.09, out, lse, ws)
    torch.cuda.synchronize()
    kc, ks, kz = cache.k
    vc, vs, vz = cache.v
    nk = oracle.quantize_int2(k_new)
    nv = oracle.quantize_int2(v_new)
    full = oracle.Int2Cache(*(np.concatenate([a, b]) for a, b in zip((kc, ks, kz, vc, vs, vz), nk + nv)))
    ref, ref_lse, _ = oracle.attention(q, full, 0.09)
    tu.assert_close(out.cpu().numpy(), ref, lse.cpu().numpy(), ref_lse, "INT2 append + attention")


def test_int2_wide_value_ranges():
    """Wide blocks (V scales up to about 3,000, K x30): the output stays
    finite and matches the oracle."""
    import torch
    import attention_quantized_kv_amd as kvq
    rng = np.random.default_rng(12)
    ctx, n_kv, D, P = 700, 1, 256, 64
    k = (rng.standard_normal((ctx, n_kv, D)) * 30).astype(np.float32)
    v = (rng.standard_normal((ctx, n_kv, D)) * 1200).astype(np.float32)
    n_pages = (ctx + P - 1) // P
    L = tu.layout(n_kv, D, P, n_pages, codec=kvq.KVQ_CODEC_INT2)
    pool = tu.alloc_pool(L)
    pt_dev, _ = tu.page_table_for(ctx, P, n_pages, 12)
    kvq.kvq_append(L, pool, pt_dev, 0, torch.from_numpy(k).cuda(), torch.from_numpy(v).cuda())
    cache = oracle.Int2Cache.from_float(k, v)
    assert float(np.max(cache.v[1].view(np.float16).astype(np.float32))) > 2000.0
    q = rng.standard_normal((1, 4, D)).astype(np.float32) * 0.05
    out, lse = _attend(L, pool, pt_dev, ctx, q, 1.0 / 16)
    ref, ref_lse, _ = oracle.attention(q, cache, 1.0 / 16)
    assert np.isfinite(out).all()
    # The outputs are near-cancelling averages of values of size ~1,200; the
    # weights are fp16 (2^-12 relative) on the GPU, so the error scales with
    # the values, not with the small result: compare in units of the value
    # scale (the tolerance assumes unit-scale values).
    tu.assert_close(out / 1200.0, ref / 1200.0, lse, ref_lse, "INT2 wide ranges (in units of 1,200)")


# ---- prefill (and decode with more than 16 rows) over the INT2 cache: the
# LDS-tiled kernel (kernel 3)

@pytest.mark.parametrize("D,P,cached,n_q,n_kv,G,kernel,cps", [
    (256, 64, 500, 300, 2, 6, 0, 0),     # a chunk after a cache: several row tiles, ragged
    (128, 32, 0, 97, 1, 1, 0, 0),        # no cache: causal inside the chunk only
    (256, 256, 3000, 64, 1, 8, 0, 4),    # many splits, merged
    (256, 64, 130, 4, 2, 6, 0, 0),       # verify with 24 rows: kernel 3 picked
    (128, 64, 900, 2, 1, 6, 3, 0),       # kernel 3 asked for a small decode
])
def test_int2_prefill_matches_oracle(D, P, cached, n_q, n_kv, G, kernel, cps):
    ctx = cached + n_q
    rng, L, pool, pt_dev, cache = _int2_pool(300 + ctx + D, ctx, n_kv, D, P)
    q = rng.standard_normal((n_q, n_kv * G, D)).astype(np.float32)
    scale = 1.0 / np.sqrt(D)
    out, lse = _attend(L, pool, pt_dev, ctx, q, scale, kernel=kernel, cps=cps)
    ref, ref_lse, _ = oracle.attention(q, cache, scale)
    tu.assert_close(out, ref, lse, ref_lse, f"INT2 prefill D={D} ctx={ctx} n_q={n_q} G={G} cps={cps}")


def test_int2_prefill_outliers():
    ctx, n_q = 1500, 200
    rng, L, pool, pt_dev, cache = _int2_pool(41, ctx, 2, 256, 64, outliers=True)
    q = rng.standard_normal((n_q, 8, 256)).astype(np.float32)
    out, lse = _attend(L, pool, pt_dev, ctx, q, 0.0625)
    ref, ref_lse, _ = oracle.attention(q, cache, 0.0625)
    tu.assert_close(out, ref, lse, ref_lse, "INT2 prefill with outliers")
