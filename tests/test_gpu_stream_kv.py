"""GPU: host-resident KV streaming (kvq_stage_pages).

The cache of a layer lives in a pinned host pool with scattered pages; its
pages are copied to consecutive pages of a device pool and attention runs
there with the identity-shifted page table.  Checked against the fp64
oracle: one staged layer (a shuffled host table with runs and gaps), and a
three-layer pipeline in which the copy of layer l + 1 (on a stream of its
own, into the other of two device buffers) overlaps the attention of layer l,
ordered by events.
"""
import math

import numpy as np
import pytest

import oracle
from tests import kvq_testutil as tu

pytestmark = pytest.mark.gpu

N_KV, D, P = 2, 128, 64


def _host_layer(seed, ctx, extra_pages=6):
    """A layer's cache quantized on the GPU into a pool with a shuffled page
    table, then moved to pinned host memory."""
    import torch
    import attention_quantized_kv_amd as kvq
    rng = np.random.default_rng(seed)
    k = rng.standard_normal((ctx, N_KV, D)).astype(np.float32)
    v = rng.standard_normal((ctx, N_KV, D)).astype(np.float32)
    n_pages = (ctx + P - 1) // P + extra_pages
    L = tu.layout(N_KV, D, P, n_pages)
    pool = tu.alloc_pool(L, fill=0xFF)
    # a table with runs of consecutive pages and jumps between them
    perm = np.concatenate([np.arange(4, 9), rng.permutation(np.arange(9, n_pages)), np.arange(0, 4)])
    pt = perm[:(ctx + P - 1) // P].astype(np.int32)
    kvq.kvq_append(L, pool, torch.from_numpy(pt).cuda(), 0, torch.from_numpy(k).cuda(), torch.from_numpy(v).cuda())
    host = torch.empty(pool.numel(), dtype=torch.uint8, pin_memory=True)
    host.copy_(pool)
    torch.cuda.synchronize()
    return L, host, pt, oracle.QuantCache.from_float(k, v), rng


def _decode(L, pool, table, ctx, q, scale):
    import torch
    import attention_quantized_kv_amd as kvq
    n_q, n_heads = q.shape[0], q.shape[1]
    out = torch.full((n_q, n_heads, D), float("nan"), device="cuda")
    lse = torch.full((n_q, n_heads), float("nan"), device="cuda")
    ws = torch.empty(kvq.kvq_workspace_bytes(L, n_heads, ctx, n_q), dtype=torch.uint8, device="cuda")
    kvq.kvq_decode_attn(L, pool, table, ctx, q, scale, out, lse, ws)
    return out, lse


def test_one_staged_layer():
    import torch
    import attention_quantized_kv_amd as kvq
    ctx = 5000
    HL, host, pt, cache, rng = _host_layer(101, ctx)
    n = len(pt)
    DL = tu.layout(N_KV, D, P, n + 3)
    dev = tu.alloc_pool(DL, fill=0)
    kvq.kvq_stage_pages(HL, host, pt, DL, dev, dst_first=2)
    table = torch.arange(2, 2 + n, dtype=torch.int32, device="cuda")
    q = rng.standard_normal((1, N_KV * 3, D)).astype(np.float32)
    scale = 1.0 / math.sqrt(D)
    out, lse = _decode(DL, dev, table, ctx, torch.from_numpy(q).cuda(), scale)
    torch.cuda.synchronize()
    ref, ref_lse, _ = oracle.attention(q, cache, scale)
    tu.assert_close(out.cpu().numpy(), ref, lse.cpu().numpy(), ref_lse, "staged layer")


def test_overlapped_pipeline_three_layers():
    import torch
    import attention_quantized_kv_amd as kvq
    ctxs = [3000, 4500, 2000]
    layers = [_host_layer(200 + i, c) for i, c in enumerate(ctxs)]
    n_max = max(len(ly[2]) for ly in layers)
    DL = tu.layout(N_KV, D, P, n_max)
    bufs = [tu.alloc_pool(DL, fill=0), tu.alloc_pool(DL, fill=0)]
    table = torch.arange(n_max, dtype=torch.int32, device="cuda")
    scale = 1.0 / math.sqrt(D)
    qs = [torch.from_numpy(ly[4].standard_normal((2, N_KV * 4, D)).astype(np.float32)).cuda() for ly in layers]
    compute = torch.cuda.current_stream()
    copy = torch.cuda.Stream()
    copied = [torch.cuda.Event(), torch.cuda.Event()]
    used = [torch.cuda.Event(), torch.cuda.Event()]
    for e in used:
        e.record(compute)
    with torch.cuda.stream(copy):
        kvq.kvq_stage_pages(layers[0][0], layers[0][1], layers[0][2], DL, bufs[0], stream=copy)
        copied[0].record(copy)
    outs = []
    for i, (HL, host, pt, cache, rng) in enumerate(layers):
        b = i % 2
        if i + 1 < len(layers):               # the next layer's copy overlaps this layer's attention
            nb = (i + 1) % 2
            with torch.cuda.stream(copy):
                copy.wait_event(used[nb])
                nxt = layers[i + 1]
                kvq.kvq_stage_pages(nxt[0], nxt[1], nxt[2], DL, bufs[nb], stream=copy)
                copied[nb].record(copy)
        compute.wait_event(copied[b])
        outs.append(_decode(DL, bufs[b], table, ctxs[i], qs[i], scale))
        used[b].record(compute)
    torch.cuda.synchronize()
    for i, (HL, host, pt, cache, rng) in enumerate(layers):
        ref, ref_lse, _ = oracle.attention(qs[i].cpu().numpy(), cache, scale)
        tu.assert_close(outs[i][0].cpu().numpy(), ref, outs[i][1].cpu().numpy(), ref_lse, f"pipelined layer {i}")
