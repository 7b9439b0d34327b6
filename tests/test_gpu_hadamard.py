"""GPU: kvq_hadamard against the oracle's rotation, and the rotated 2-bit
cache end to end.

The rotation (x H / sqrt(dim), fp32 butterflies) must match the oracle's
fp64 product to fp32 accuracy for every supported kind of size (2 .. 1024,
one row to many), undo itself, and leave rows it does not cover alone.  End
to end, keys and values with outlier channels are rotated on the GPU,
appended to an INT2 cache, attended by rotated queries, and the output is
rotated back; the result must match the oracle doing the same steps with its
own rotation (the pages' recipe: "OSCAR2 KV Cache benchmark", rotation model
conversion).  Its inputs are multiples of 1/8, whose rotation is exact in
fp32 at head_dim 256, so both sides quantize the same values (an ulp of
difference could otherwise move a value across a 2-bit code boundary).
"""
import math

import numpy as np
import pytest

import oracle
from tests import kvq_testutil as tu

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("dim,n_rows", [(2, 3), (64, 1), (128, 37), (256, 1000), (1024, 5)])
def test_rotation_matches_oracle(dim, n_rows):
    import torch
    import attention_quantized_kv_amd as kvq
    x = np.random.default_rng(dim + n_rows).standard_normal((n_rows, dim)).astype(np.float32)
    x[:, 3 % dim] *= 50.0
    t = torch.from_numpy(x).cuda()
    kvq.kvq_hadamard(t)
    got = t.cpu().numpy().astype(np.float64)
    want = oracle.hadamard(x)
    # fp32 butterflies: log2(dim) roundings of values up to the row norm
    tol = 4e-7 * math.log2(dim) * np.linalg.norm(x, axis=1, keepdims=True) + 1e-30
    assert np.all(np.abs(got - want) <= tol), float(np.max(np.abs(got - want) / tol))


def test_rotation_is_an_involution_and_local():
    import torch
    import attention_quantized_kv_amd as kvq
    x = np.random.default_rng(1).standard_normal((6, 256)).astype(np.float32)
    t = torch.from_numpy(x.copy()).cuda()
    kvq.kvq_hadamard(t[:4])                      # rows 4, 5 untouched
    kvq.kvq_hadamard(t[:4])
    got = t.cpu().numpy()
    np.testing.assert_allclose(got[:4], x[:4], rtol=0, atol=2e-6)
    assert np.array_equal(got[4:], x[4:])
    empty = torch.empty((0, 64), device="cuda")
    kvq.kvq_hadamard(empty)                      # no rows: a no-op


def test_rotated_int2_decode():
    import torch
    import attention_quantized_kv_amd as kvq
    rng = np.random.default_rng(21)
    ctx, n_kv, G, D, P = 3000, 2, 6, 256, 64

    def eighths(shape):
        # multiples of 1/8 (x20 on the outlier channels still is): every
        # butterfly sum is exact in fp32 and 1/sqrt(256) = 1/16, so the GPU's
        # rotation equals the oracle's and both quantize the same values
        return (np.round(rng.standard_normal(shape) * 8) / 8).astype(np.float32)
    k = eighths((ctx, n_kv, D))
    v = eighths((ctx, n_kv, D))
    for x in (k, v):
        x[:, :, [9, 100, 180, 250]] *= 20.0
    q = eighths((1, n_kv * G, D))
    scale = 1.0 / 16
    # GPU: rotate, append, attend with rotated queries, rotate the output back
    n_pages = (ctx + P - 1) // P
    L = tu.layout(n_kv, D, P, n_pages, codec=kvq.KVQ_CODEC_INT2)
    pool = tu.alloc_pool(L)
    pt_dev, _ = tu.page_table_for(ctx, P, n_pages, 21)
    kd, vd, qd = (torch.from_numpy(a.copy()).cuda() for a in (k, v, q))
    for t in (kd, vd, qd):
        kvq.kvq_hadamard(t)
    kvq.kvq_append(L, pool, pt_dev, 0, kd, vd)
    out = torch.empty_like(qd)
    lse = torch.empty((1, n_kv * G), device="cuda")
    ws = torch.empty(kvq.kvq_workspace_bytes(L, n_kv * G, ctx, 1), dtype=torch.uint8, device="cuda")
    kvq.kvq_decode_attn(L, pool, pt_dev, ctx, qd, scale, out, lse, ws)
    kvq.kvq_hadamard(out)
    torch.cuda.synchronize()
    # oracle: the same steps with its own rotation (fp64, then fp32 inputs)
    kr, vr, qr = (oracle.hadamard(a).astype(np.float32) for a in (k, v, q))
    ref_r, ref_lse, _ = oracle.attention(qr, oracle.Int2Cache.from_float(kr, vr), scale)
    ref = oracle.hadamard(ref_r)
    assert np.array_equal(kr, oracle.hadamard(k).astype(np.float32))
    tu.assert_close(out.cpu().numpy(), ref, lse.cpu().numpy(), ref_lse, "rotated INT2 decode")
