"""GPU: the decode step captured in a HIP graph.

The library's calls are asynchronous, allocation-free and make no
device-wide call once a kernel has run on the device, so a caller can record
them in a graph.  Three layers of kvq_append_attn are captured in one graph;
the graph is replayed several times with the program's own eager work and a
synchronization between the replays, and every replay must match the
oracle, like the eager call before it (the step appends the same rows at the
same position, so replaying it is idempotent on the pool).  The same for the
INT2 cache (append, its streaming kernel, the merge).
"""
import math

import numpy as np
import pytest

import oracle
from tests import kvq_testutil as tu

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("codec", [0, 1])
def test_decode_step_graph_replays_match_oracle(codec):
    import torch
    import attention_quantized_kv_amd as kvq
    rng = np.random.default_rng(81)
    n_kv, G, D, P, pos0, n_new = 2, 3, 128, 64, 3000, 2
    n_heads, ctx = n_kv * G, pos0 + n_new
    scale = 1.0 / math.sqrt(D)
    layers = []
    for li in range(3):
        k = rng.standard_normal((ctx, n_kv, D)).astype(np.float32)
        v = rng.standard_normal((ctx, n_kv, D)).astype(np.float32)
        q = rng.standard_normal((n_new, n_heads, D)).astype(np.float32)
        L = tu.layout(n_kv, D, P, (ctx + P - 1) // P + 2, codec=codec)
        pool = tu.alloc_pool(L, fill=0xFF)
        pt_dev, _ = tu.page_table_for(ctx, P, L.n_pages, perm_seed=li)
        kd, vd = torch.from_numpy(k).cuda(), torch.from_numpy(v).cuda()
        kvq.kvq_append(L, pool, pt_dev, 0, kd[:pos0].contiguous(), vd[:pos0].contiguous())
        cache = (oracle.Int2Cache if codec == kvq.KVQ_CODEC_INT2 else oracle.QuantCache).from_float(k, v)
        ref, ref_lse, _ = oracle.attention(q, cache, scale)
        layers.append(dict(L=L, pool=pool, pt=pt_dev, k=kd[pos0:].contiguous(), v=vd[pos0:].contiguous(),
                           q=torch.from_numpy(q).cuda(), ref=ref, ref_lse=ref_lse,
                           out=torch.full((n_new, n_heads, D), float("nan"), device="cuda"),
                           lse=torch.full((n_new, n_heads), float("nan"), device="cuda")))
    nbytes = kvq.kvq_append_attn_workspace_bytes(layers[0]["L"], n_heads, pos0, n_new)
    ws = torch.empty(nbytes, dtype=torch.uint8, device="cuda")

    def step():
        for ly in layers:
            kvq.kvq_append_attn(ly["L"], ly["pool"], ly["pt"], pos0, ly["k"], ly["v"], ly["q"], scale,
                                ly["out"], ly["lse"], ws)

    def check(what):
        for i, ly in enumerate(layers):
            tu.assert_close(ly["out"].cpu().numpy(), ly["ref"], ly["lse"].cpu().numpy(), ly["ref_lse"],
                            f"{what}, layer {i}")

    step()                                   # eager: also the first launch of every kernel on the device
    torch.cuda.synchronize()
    check("eager")
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    torch.cuda.synchronize()
    for r in range(4):
        for ly in layers:                    # the program's own eager work between replays
            ly["out"].fill_(float("nan"))
            ly["lse"].fill_(float("nan"))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        check(f"replay {r}")
