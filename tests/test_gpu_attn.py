"""GPU: attention through the C ABI against the fp64 oracle.

Every case: fp32 K/V rows from the seeded generators are appended with
kvq_append (GPU) and quantized independently by the oracle; outputs must be
within |o - ref| <= 2e-3 + 1e-3|ref| of the oracle and lse within
1e-4 + 1e-5|ref|.
"""
import math

import numpy as np
import pytest

import oracle
import synth
from tests import kvq_testutil as tu

pytestmark = pytest.mark.gpu

KERNELS = {"valu": 1, "mfma_stream": 2, "mfma_tiled": 3}


def _torch():
    import torch
    return torch


class Case:
    """A filled one-layer cache on the GPU plus its oracle twin."""

    def __init__(self, k, v, P=256, n_pages=None, perm_seed=None):
        torch = _torch()
        import attention_quantized_kv_amd as kvq
        self.kvq = kvq
        ctx, n_kv, D = k.shape
        need = (ctx + P - 1) // P
        n_pages = n_pages or need
        self.L = tu.layout(n_kv, D, P, n_pages)
        self.pool = tu.alloc_pool(self.L)
        self.pt_dev, self.pt = tu.page_table_for(ctx, P, n_pages, perm_seed)
        kd, vd = torch.from_numpy(k).cuda(), torch.from_numpy(v).cuda()
        step = 8192
        for r in range(0, ctx, step):
            kvq.kvq_append(self.L, self.pool, self.pt_dev, r, kd[r:r + step].contiguous(),
                           vd[r:r + step].contiguous())
        del kd, vd
        self.cache = oracle.QuantCache.from_float(k, v)
        self.ctx, self.D = ctx, D

    def run(self, q, scale, kernel=0, cps=0, prefill=None, ctx=None):
        torch = _torch()
        kvq = self.kvq
        ctx = self.ctx if ctx is None else ctx
        n_q, n_heads, D = q.shape
        qd = torch.from_numpy(np.ascontiguousarray(q)).cuda()
        out = torch.full((n_q, n_heads, D), float("nan"), device="cuda")
        lse = torch.full((n_q, n_heads), float("nan"), device="cuda")
        ws_n = kvq.kvq_workspace_bytes_ex(self.L, n_heads, ctx, n_q, kernel, cps)
        ws = torch.empty((max(ws_n, 1),), dtype=torch.uint8, device="cuda")
        if prefill is None and kernel == 0 and cps == 0:
            prefill = n_q > 8
        if kernel == 0 and cps == 0:
            fn = kvq.kvq_prefill_attn if prefill else kvq.kvq_decode_attn
            fn(self.L, self.pool, self.pt_dev, ctx, qd, scale, out, lse, ws)
        else:
            kvq.kvq_attn_ex(self.L, self.pool, self.pt_dev, ctx, qd, scale, out, lse, ws,
                            kernel=kernel, chunks_per_split=cps)
        torch.cuda.synchronize()
        return out.cpu().numpy(), lse.cpu().numpy()

    def ref(self, q, scale, ctx=None, rows=None):
        if rows is None:
            o, l, _ = oracle.attention(q, self.cache, scale, ctx=ctx)
            return o, l
        return oracle.attention(q, self.cache, scale, rows=rows, ctx=ctx)


def _rand_case(seed, ctx, n_kv, D, P=256, perm=True, mag=1.0):
    rng = np.random.default_rng(seed)
    k = (rng.standard_normal((ctx, n_kv, D)) * mag).astype(np.float32)
    v = (rng.standard_normal((ctx, n_kv, D)) * mag).astype(np.float32)
    n_pages = (ctx + P - 1) // P + 3
    return Case(k, v, P=P, n_pages=n_pages, perm_seed=seed if perm else None), rng


@pytest.fixture(scope="module", params=["valu", "mfma_stream", "mfma_tiled"])
def kernel(request):
    return KERNELS[request.param]


def test_tiny_workload(kernel):
    w = synth.WORKLOADS["tiny"]
    k, v = synth.layer_kv(w, 0)
    c = Case(k, v, P=w.page_size)
    q = synth.layer_q(w, 0)
    out, lse = c.run(q, w.scale, kernel=kernel)
    ref, ref_lse = c.ref(q, w.scale)
    tu.assert_close(out, ref, lse, ref_lse, "tiny")


@pytest.mark.parametrize("D,G,ctx,n_q", [
    (64, 1, 1, 1), (64, 2, 255, 1), (128, 6, 256, 1), (256, 6, 257, 1), (256, 6, 1000, 4),
    (64, 8, 300, 8), (128, 2, 513, 3), (256, 1, 2049, 2), (64, 16, 97, 4),
    (128, 6, 700, 3),       # 18 rows: a second row tile with 2 rows
    (64, 11, 800, 3),       # 33 rows: a second row group with one row
])
def test_decode_shapes(kernel, D, G, ctx, n_q):
    c, rng = _rand_case(D * 1000 + G * 10 + n_q, ctx, 2, D, P=64 if ctx < 600 else 256)
    q = rng.standard_normal((n_q, 2 * G, D)).astype(np.float32)
    scale = 1 / math.sqrt(D)
    out, lse = c.run(q, scale, kernel=kernel)
    ref, ref_lse = c.ref(q, scale)
    tu.assert_close(out, ref, lse, ref_lse, f"D={D} G={G} ctx={ctx} n_q={n_q}")


@pytest.mark.parametrize("cps", [1, 2, 3, 1000])
def test_split_invariance(kernel, cps):
    c, rng = _rand_case(77, 3000, 4, 256)
    q = rng.standard_normal((1, 24, 256)).astype(np.float32)
    out, lse = c.run(q, 1 / 16, kernel=kernel, cps=cps)
    ref, ref_lse = c.ref(q, 1 / 16)
    tu.assert_close(out, ref, lse, ref_lse, f"cps={cps}")


def test_max_over_full_scores(kernel):
    """Keys whose first-half partial dot products are large but whose full
    scores are small: the softmax max must come from complete scores."""
    D, ctx = 256, 96
    rng = np.random.default_rng(5)
    k = rng.standard_normal((ctx, 1, D)).astype(np.float32) * 0.1
    k[::3, 0, :D // 2] = 4.0
    k[::3, 0, D // 2:] = -4.0
    k[1::7, 0, :] = 0.7
    v = rng.standard_normal((ctx, 1, D)).astype(np.float32)
    c = Case(k, v, P=32)
    q = np.ones((1, 6, D), np.float32)
    q[0, 3:] *= 2.0
    for scale in (1 / 16, 1.0):
        out, lse = c.run(q, scale, kernel=kernel)
        ref, ref_lse = c.ref(q, scale)
        tu.assert_close(out, ref, lse, ref_lse, f"scale={scale}")


def test_asymmetric_zero_k_or_v(kernel):
    D, ctx = 128, 700
    rng = np.random.default_rng(9)
    rnd = rng.standard_normal((ctx, 2, D)).astype(np.float32)
    zero = np.zeros_like(rnd)
    q = rng.standard_normal((2, 4, D)).astype(np.float32)
    # zero V, random K: output exactly 0
    c1 = Case(rnd, zero, P=64)
    out, lse = c1.run(q, 0.1, kernel=kernel)
    ref, ref_lse = c1.ref(q, 0.1)
    assert np.all(out == 0.0)
    tu.assert_close(out, ref, lse, ref_lse, "zero V")
    # zero K, random V: uniform weights, mean of the visible values
    c2 = Case(zero, rnd, P=64)
    out, lse = c2.run(q, 0.1, kernel=kernel)
    ref, ref_lse = c2.ref(q, 0.1)
    tu.assert_close(out, ref, lse, ref_lse, "zero K")


def test_page_permutation_invariance(kernel):
    rng = np.random.default_rng(21)
    k = rng.standard_normal((900, 2, 128)).astype(np.float32)
    v = rng.standard_normal((900, 2, 128)).astype(np.float32)
    q = rng.standard_normal((1, 8, 128)).astype(np.float32)
    a = Case(k, v, P=64, n_pages=20, perm_seed=None).run(q, 0.09, kernel=kernel)
    b = Case(k, v, P=64, n_pages=20, perm_seed=3).run(q, 0.09, kernel=kernel)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


def test_large_magnitudes(kernel):
    c, rng = _rand_case(31, 777, 2, 64, P=32, mag=30.0)
    q = (rng.standard_normal((3, 4, 64)) * 3).astype(np.float32)
    out, lse = c.run(q, 0.125, kernel=kernel)
    ref, ref_lse = c.ref(q, 0.125)
    tu.assert_close(out, ref, lse, ref_lse, "large")


@pytest.mark.parametrize("D,ctx,n_q,G,P", [
    (128, 1200, 200, 6, 64),    # ragged last chunk, 10 row tiles
    (256, 2500, 64, 6, 256),    # head_dim 256: three row tiles, ragged last chunk
    (64, 700, 100, 4, 32),
])
def test_prefill_chunk(kernel, D, ctx, n_q, G, P):
    c, rng = _rand_case(41 + D, ctx, 2, D, P=P)
    q = rng.standard_normal((n_q, 2 * G, D)).astype(np.float32)
    if kernel == KERNELS["mfma_stream"]:
        import attention_quantized_kv_amd as kvq
        with pytest.raises(kvq.KvqError) as e:      # more than 64 rows per KV head
            c.run(q, 1 / math.sqrt(D), kernel=kernel, prefill=True)
        assert e.value.status == kvq.KVQ_ERR_UNSUPPORTED
        return
    out, lse = c.run(q, 1 / math.sqrt(D), kernel=kernel, prefill=True)
    ref, ref_lse = c.ref(q, 1 / math.sqrt(D))
    tu.assert_close(out, ref, lse, ref_lse, f"prefill D={D} ctx={ctx} n_q={n_q}")


def test_invalid_page_entry_gives_nan_not_fault(kernel):
    torch = _torch()
    c, rng = _rand_case(51, 600, 1, 64, P=64, perm=False)
    bad = c.pt_dev.clone()
    bad[3] = c.L.n_pages + 5           # outside the pool: must not be dereferenced
    bad[5] = -1
    good = c.pt_dev
    c.pt_dev = bad
    q = rng.standard_normal((1, 2, 64)).astype(np.float32)
    out, lse = c.run(q, 0.125, kernel=kernel)
    assert np.isnan(out).all() and np.isnan(lse).all()
    c.pt_dev = good
    out, lse = c.run(q, 0.125, kernel=kernel)
    assert np.isfinite(out).all()
    torch.cuda.synchronize()
