"""GPU: decode (up to 8 query rows per KV head) on a longer cache with many
KV heads, where every workgroup of the streaming kernel hands several chunks
to each of its waves from its LDS list.  Checked against the fp64 oracle:
  * outputs and lse, with shuffled pages, over several calls on one
    workspace that starts filled with random bytes;
  * the fused decode step (kvq_append_attn) on such a cache;
  * a page-table entry outside the pool for a late chunk: NaN, no fault, and
    right again with the good table on the same workspace.
"""
import math

import numpy as np
import pytest

import oracle
from tests import kvq_testutil as tu
from tests.test_gpu_attn import Case

pytestmark = pytest.mark.gpu

# 8 KV heads of head_dim 64 with 64-token pages: 32 workgroups per KV head
# share its 1,250 chunks.
N_KV, D, P, CTX = 8, 64, 64, 40000


@pytest.fixture(scope="module")
def case():
    rng = np.random.default_rng(71)
    k = rng.standard_normal((CTX, N_KV, D)).astype(np.float32)
    v = rng.standard_normal((CTX, N_KV, D)).astype(np.float32)
    return Case(k, v, P=P, n_pages=(CTX + P - 1) // P + 5, perm_seed=71)


@pytest.mark.parametrize("G,n_q", [(1, 1), (2, 1), (6, 1), (2, 4), (8, 1)])
def test_long_decode_matches_oracle_over_reused_garbage_workspace(case, G, n_q):
    import torch
    import attention_quantized_kv_amd as kvq
    rng = np.random.default_rng(100 + G * 10 + n_q)
    n_heads = N_KV * G
    nbytes = kvq.kvq_workspace_bytes(case.L, n_heads, CTX, n_q)
    ws = torch.from_numpy(rng.integers(0, 256, nbytes, dtype=np.uint8)).cuda()
    scale = 1.0 / math.sqrt(D)
    for it in range(3):
        q = rng.standard_normal((n_q, n_heads, D)).astype(np.float32)
        out = torch.full((n_q, n_heads, D), float("nan"), device="cuda")
        lse = torch.full((n_q, n_heads), float("nan"), device="cuda")
        kvq.kvq_decode_attn(case.L, case.pool, case.pt_dev, CTX, torch.from_numpy(q).cuda(), scale, out, lse, ws)
        torch.cuda.synchronize()
        ref, ref_lse = case.ref(q, scale)
        tu.assert_close(out.cpu().numpy(), ref, lse.cpu().numpy(), ref_lse, f"G={G} n_q={n_q} call {it}")


def test_long_fused_step(case):
    """kvq_append_attn over the case's first CTX - 3 rows plus 3 new ones (in a
    pool of its own, so the module's cache stays intact)."""
    import torch
    import attention_quantized_kv_amd as kvq
    rng = np.random.default_rng(73)
    G, n_new = 2, 3
    n_heads = N_KV * G
    pos0 = CTX - n_new
    k = rng.standard_normal((CTX, N_KV, D)).astype(np.float32)
    v = rng.standard_normal((CTX, N_KV, D)).astype(np.float32)
    L = tu.layout(N_KV, D, P, (CTX + P - 1) // P + 2)
    pool = tu.alloc_pool(L, fill=0xFF)
    pt_dev, pt = tu.page_table_for(CTX, P, L.n_pages, perm_seed=73)
    kd, vd = torch.from_numpy(k).cuda(), torch.from_numpy(v).cuda()
    kvq.kvq_append(L, pool, pt_dev, 0, kd[:pos0].contiguous(), vd[:pos0].contiguous())
    q = rng.standard_normal((n_new, n_heads, D)).astype(np.float32)
    out = torch.full((n_new, n_heads, D), float("nan"), device="cuda")
    lse = torch.full((n_new, n_heads), float("nan"), device="cuda")
    nbytes = kvq.kvq_append_attn_workspace_bytes(L, n_heads, pos0, n_new)
    ws = torch.from_numpy(rng.integers(0, 256, nbytes, dtype=np.uint8)).cuda()
    scale = 1.0 / math.sqrt(D)
    kvq.kvq_append_attn(L, pool, pt_dev, pos0, kd[pos0:].contiguous(), vd[pos0:].contiguous(),
                        torch.from_numpy(q).cuda(), scale, out, lse, ws)
    torch.cuda.synchronize()
    ref, ref_lse, _ = oracle.attention(q, oracle.QuantCache.from_float(k, v), scale)
    tu.assert_close(out.cpu().numpy(), ref, lse.cpu().numpy(), ref_lse, "fused step, long cache")


def test_long_invalid_page_gives_nan_not_fault(case):
    import torch
    import attention_quantized_kv_amd as kvq
    rng = np.random.default_rng(75)
    n_heads = N_KV * 2
    bad = case.pt_dev.clone()
    bad[(CTX - 1000) // P] = case.L.n_pages + 9      # a late chunk
    q = rng.standard_normal((1, n_heads, D)).astype(np.float32)
    out = torch.full((1, n_heads, D), 0.0, device="cuda")
    lse = torch.full((1, n_heads), 0.0, device="cuda")
    ws = torch.empty(kvq.kvq_workspace_bytes(case.L, n_heads, CTX, 1), dtype=torch.uint8, device="cuda")
    kvq.kvq_decode_attn(case.L, case.pool, bad, CTX, torch.from_numpy(q).cuda(), 0.125, out, lse, ws)
    torch.cuda.synchronize()
    assert np.isnan(out.cpu().numpy()).all() and np.isnan(lse.cpu().numpy()).all()
    # the same workspace, the good table: finite and right again
    kvq.kvq_decode_attn(case.L, case.pool, case.pt_dev, CTX, torch.from_numpy(q).cuda(), 0.125, out, lse, ws)
    torch.cuda.synchronize()
    ref, ref_lse = case.ref(q, 0.125)
    tu.assert_close(out.cpu().numpy(), ref, lse.cpu().numpy(), ref_lse, "after the bad table")
