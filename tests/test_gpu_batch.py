"""GPU: batched decode (kvq_decode_attn_batch) against the fp64 oracle.

Several sequences share one page pool, each with its own page-table row
(disjoint, shuffled pages) and context length; every sequence's output and
lse must match the oracle run on that sequence alone.  Cases: ragged lengths
from 8 to 20,000 keys (a single key in the largest batch), n_q = 1..8 over
every row layout of the streaming kernel (up to 8 rows, one 16-row tile, two
tiles per wave -- full at 32 rows, half at 24 -- and two row groups at 48
rows), the largest batch (64 sequences), and a page-table entry outside the
pool in one sequence (that sequence NaN, the others exact).
The same over the INT2 cache (its streaming kernel, up to 16 rows).
"""
import math

import numpy as np
import pytest

import oracle
from tests import kvq_testutil as tu

pytestmark = pytest.mark.gpu


class Batch:
    def __init__(self, seed, ctx_lens, n_kv, D, P, codec=0):
        import torch
        import attention_quantized_kv_amd as kvq
        self.kvq = kvq
        rng = np.random.default_rng(seed)
        pages = [(c + P - 1) // P for c in ctx_lens]
        n_pages = sum(pages) + 3
        self.L = tu.layout(n_kv, D, P, n_pages, codec=codec)
        self.pool = tu.alloc_pool(self.L, fill=0xFF)
        perm = rng.permutation(n_pages).astype(np.int32)
        n_table = max(pages)
        pt = np.full((len(ctx_lens), n_table), -1, dtype=np.int32)
        used = 0
        for b, n in enumerate(pages):
            pt[b, :n] = perm[used:used + n]
            used += n
        self.pt = torch.from_numpy(pt).cuda()
        self.caches = []
        for b, c in enumerate(ctx_lens):
            k = rng.standard_normal((c, n_kv, D)).astype(np.float32)
            v = rng.standard_normal((c, n_kv, D)).astype(np.float32)
            kvq.kvq_append(self.L, self.pool, self.pt[b].contiguous(), 0, torch.from_numpy(k).cuda(),
                           torch.from_numpy(v).cuda())
            self.caches.append((oracle.Int2Cache if codec == kvq.KVQ_CODEC_INT2 else oracle.QuantCache).from_float(k, v))
        self.ctx_lens, self.n_kv, self.D, self.rng = list(ctx_lens), n_kv, D, rng

    def run(self, G, n_q, pt=None):
        import torch
        kvq = self.kvq
        n_heads, B = self.n_kv * G, len(self.ctx_lens)
        q = self.rng.standard_normal((B, n_q, n_heads, self.D)).astype(np.float32)
        out = torch.full((B, n_q, n_heads, self.D), float("nan"), device="cuda")
        lse = torch.full((B, n_q, n_heads), float("nan"), device="cuda")
        nbytes = kvq.kvq_decode_attn_batch_workspace_bytes(self.L, self.ctx_lens, n_heads, n_q)
        ws = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
        scale = 1.0 / math.sqrt(self.D)
        kvq.kvq_decode_attn_batch(self.L, self.pool, self.pt if pt is None else pt, self.ctx_lens,
                                  torch.from_numpy(q).cuda(), scale, out, lse, ws)
        torch.cuda.synchronize()
        return q, scale, out.cpu().numpy(), lse.cpu().numpy()


@pytest.fixture(scope="module")
def ragged():
    return Batch(91, [8, 97, 3000, 257, 20000, 64, 9], n_kv=2, D=128, P=64)


@pytest.mark.parametrize("G,n_q", [(4, 1), (4, 2), (4, 4), (4, 8), (6, 4), (8, 6), (1, 1)])
def test_batch_matches_oracle_per_sequence(ragged, G, n_q):
    q, scale, out, lse = ragged.run(G, n_q)
    for b, c in enumerate(ragged.ctx_lens):
        ref, ref_lse, _ = oracle.attention(q[b], ragged.caches[b], scale)
        tu.assert_close(out[b], ref, lse[b], ref_lse, f"sequence {b} (ctx {c}), G={G} n_q={n_q}")


def test_largest_batch():
    lens = [1 + (37 * i) % 600 for i in range(64)]     # sequence 0 has a single key
    bt = Batch(93, lens, n_kv=1, D=64, P=32)
    q, scale, out, lse = bt.run(2, 1)
    for b, c in enumerate(lens):
        ref, ref_lse, _ = oracle.attention(q[b], bt.caches[b], scale)
        tu.assert_close(out[b], ref, lse[b], ref_lse, f"sequence {b} of 64 (ctx {c})")


def test_invalid_page_in_one_sequence(ragged):
    bad = ragged.pt.clone()
    bad[2, 10] = ragged.L.n_pages + 4     # sequence 2 (3,000 keys) only
    q, scale, out, lse = ragged.run(4, 1, pt=bad)
    assert np.isnan(out[2]).all() and np.isnan(lse[2]).all()
    for b, c in enumerate(ragged.ctx_lens):
        if b == 2:
            continue
        ref, ref_lse, _ = oracle.attention(q[b], ragged.caches[b], scale)
        tu.assert_close(out[b], ref, lse[b], ref_lse, f"sequence {b} beside the bad one")


@pytest.fixture(scope="module")
def ragged_int2():
    import attention_quantized_kv_amd as kvq
    return Batch(95, [8, 97, 3000, 257, 9000, 64, 2], n_kv=2, D=256, P=64, codec=kvq.KVQ_CODEC_INT2)


@pytest.mark.parametrize("G,n_q", [(6, 1), (4, 2), (8, 2), (1, 1)])
def test_int2_batch_matches_oracle_per_sequence(ragged_int2, G, n_q):
    q, scale, out, lse = ragged_int2.run(G, n_q)
    for b, c in enumerate(ragged_int2.ctx_lens):
        ref, ref_lse, _ = oracle.attention(q[b], ragged_int2.caches[b], scale)
        tu.assert_close(out[b], ref, lse[b], ref_lse, f"INT2 sequence {b} (ctx {c}), G={G} n_q={n_q}")


def test_int2_batch_bad_page_and_d128():
    import attention_quantized_kv_amd as kvq
    bt = Batch(97, [1 + (53 * i) % 700 for i in range(20)], n_kv=1, D=128, P=32, codec=kvq.KVQ_CODEC_INT2)
    bad = bt.pt.clone()
    bad[5, 3] = bt.L.n_pages + 1              # sequence 5 only (it has more than 3 pages)
    assert bt.ctx_lens[5] > 3 * 32
    q, scale, out, lse = bt.run(4, 1, pt=bad)
    assert np.isnan(out[5]).all() and np.isnan(lse[5]).all()
    for b, c in enumerate(bt.ctx_lens):
        if b == 5:
            continue
        ref, ref_lse, _ = oracle.attention(q[b], bt.caches[b], scale)
        tu.assert_close(out[b], ref, lse[b], ref_lse, f"INT2 sequence {b} of 20 (ctx {c}) beside a bad one")
