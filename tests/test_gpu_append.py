"""GPU: kvq_append writes bit-exact Q8_0 / Q4_0 codes and scales.

Compared with the oracle's quantizer on the same fp32 rows: every code and
every fp16 scale bit must be identical (sign of zero included).
"""
import numpy as np
import pytest

import oracle
import synth
from tests import kvq_testutil as tu

pytestmark = pytest.mark.gpu


def _torch():
    import torch
    return torch


def _append_and_decode(k, v, P, n_pages, pieces=None, perm_seed=None, pos0=0, pool_fill=0):
    torch = _torch()
    import attention_quantized_kv_amd as kvq
    ctx, n_kv, D = k.shape
    L = tu.layout(n_kv, D, P, n_pages)
    pool = tu.alloc_pool(L, fill=pool_fill)
    pt_dev, pt = tu.page_table_for(pos0 + ctx, P, n_pages, perm_seed)
    kd = torch.from_numpy(k).cuda()
    vd = torch.from_numpy(v).cuda()
    pieces = pieces or [ctx]
    r = 0
    for n in pieces:
        kvq.kvq_append(L, pool, pt_dev, pos0 + r, kd[r:r + n].contiguous(), vd[r:r + n].contiguous())
        r += n
    assert r == ctx
    torch.cuda.synchronize()
    kc, ks, vc, vs = tu.decode_pool(pool.cpu().numpy(), L, pt, pos0 + ctx)
    return kc[pos0:], ks[pos0:], vc[pos0:], vs[pos0:]


def _check_exact(k, v, got):
    kc, ks, vc, vs = got
    okc, oks = oracle.quantize_q8_0(k)
    ovc, ovs = oracle.quantize_q4_0(v)
    assert np.array_equal(ks, oks), f"K scales differ at {np.argwhere(ks != oks)[:5]}"
    assert np.array_equal(kc, okc), f"K codes differ at {np.argwhere(kc != okc)[:5]}"
    assert np.array_equal(vs, ovs), f"V scales differ at {np.argwhere(vs != ovs)[:5]}"
    assert np.array_equal(vc, ovc), f"V codes differ at {np.argwhere(vc != ovc)[:5]}"


def test_tiny_workload_all_blocks_bit_exact():
    w = synth.WORKLOADS["tiny"]
    k, v = synth.layer_kv(w, 0)
    got = _append_and_decode(k, v, P=256, n_pages=2)
    _check_exact(k, v, got)


@pytest.mark.parametrize("D", [64, 128, 256])
def test_ragged_appends_and_shuffled_pages(D):
    rng = np.random.default_rng(D)
    ctx = 1000
    mags = (10.0 ** rng.uniform(-4, 4, size=(ctx, 3, 1))).astype(np.float32)
    k = (rng.standard_normal((ctx, 3, D)) * mags).astype(np.float32)
    v = (rng.standard_normal((ctx, 3, D)) * mags).astype(np.float32)
    # odd-sized pieces: pairs of positions split across calls (nibble merge)
    pieces = [1, 3, 7, 2, 256, 255, 1, 475]
    got = _append_and_decode(k, v, P=64, n_pages=40, pieces=pieces, perm_seed=5, pos0=0,
                             pool_fill=0xA5)
    _check_exact(k, v, got)


def test_odd_start_position():
    rng = np.random.default_rng(11)
    k = rng.standard_normal((37, 2, 64)).astype(np.float32)
    v = rng.standard_normal((37, 2, 64)).astype(np.float32)
    got = _append_and_decode(k, v, P=32, n_pages=4, pieces=[5, 1, 31], pos0=59, pool_fill=0x3C)
    _check_exact(k, v, got)


def test_crafted_blocks_ties_zeros_signs():
    D = 64
    rows = []
    z = np.zeros(D, np.float32)
    rows.append(z.copy())                                             # zero blocks
    rows.append(np.full(D, -0.0, np.float32))                         # negative zeros
    r = z.copy(); r[:9] = [127, 0.5, 2.5, -0.5, -2.5, 1.5, -1.5, 0.49, -126.5]; rows.append(r)
    r = z.copy(); r[0], r[1] = 16.0, -16.0; r[32], r[33] = -16.0, 16.0; rows.append(r)
    r = z.copy(); r[:7] = [-8, 2.5, -2.5, 7.5, 0.49, -0.5, 3.4999]; rows.append(r)
    r = np.full(D, 3.0, np.float32); r[5] = -3.0; rows.append(r)       # magnitude tie, later index
    r = z.copy(); r[31] = 1e-30; rows.append(r)                        # tiny scale (fp16 zero)
    r = z.copy(); r[0] = 6e5; rows.append(r)                           # scale past fp16 max
    x = np.stack(rows)[:, None, :]
    got = _append_and_decode(x, x, P=32, n_pages=1)
    _check_exact(x, x, got)


def test_near_ties_bit_exact():
    # values placed on and next to code boundaries exercise the separate
    # roundings of x*(1/d) and of the +8.5
    rng = np.random.default_rng(3)
    n = 4096
    amax = rng.uniform(0.5, 2.0, size=(n, 1, 1)).astype(np.float32)
    codes = rng.integers(-127, 128, size=(n, 1, 64)).astype(np.float32)
    base = (codes + 0.5) * (amax / 127.0)
    jitter = np.float32(1.0) + rng.integers(-3, 4, size=base.shape).astype(np.float32) * np.float32(2.0 ** -23)
    k = (base * jitter).astype(np.float32)
    k[:, :, 0] = amax[:, :, 0]
    k[:, :, 32] = -amax[:, :, 0]
    v4 = rng.integers(-8, 8, size=(n, 1, 64)).astype(np.float32) + np.float32(0.5)
    v = (v4 * (amax / 8.0) * jitter).astype(np.float32)
    v[:, :, 0] = -amax[:, :, 0]
    v[:, :, 32] = amax[:, :, 0]
    got = _append_and_decode(k, v, P=256, n_pages=16)
    _check_exact(k, v, got)
