"""GPU: the streaming MFMA kernel's fixed-order chunk path against the oracle.

The kernel hands a workgroup's chunks to its waves in two ways.  With one row
group (at most 32 query rows per KV head: a wave holds one 16-row tile, or
two for 17-32 rows) and at most 256 chunks per workgroup, the chunks form a
list in LDS that waves pop as they go.  With two row groups (33-64 rows), or
more than 256 chunks per workgroup, every wave walks a fixed round-robin
order instead and picks its page-table entries out of a register that holds
the next 64 of them, reloading it every 64 chunks.  These cases force that path with one split
(chunks_per_split large), so each wave walks more than 128 chunks and the
entries are reloaded at least twice, and check every output element against
the fp64 oracle (|o - ref| <= 2e-3 + 1e-3 |ref|, lse within 1e-4 + 1e-5
|ref|).  The fixed order is deterministic, so two runs agree bit for bit.
"""
import math

import numpy as np
import pytest

from tests import kvq_testutil as tu
from tests.test_gpu_attn import Case

pytestmark = pytest.mark.gpu

STREAM = 2


def _case(seed, ctx, n_kv, D, perm=True):
    rng = np.random.default_rng(seed)
    k = rng.standard_normal((ctx, n_kv, D)).astype(np.float32)
    v = rng.standard_normal((ctx, n_kv, D)).astype(np.float32)
    n_pages = (ctx + 255) // 256 + 5
    return Case(k, v, P=256, n_pages=n_pages, perm_seed=seed if perm else None), rng


@pytest.mark.parametrize("n_q,G,ctx", [
    (4, 6, 34000),     # 24 rows: one row group, two tiles per wave, ~133 chunks per wave
    (3, 8, 34000),     # 24 rows, the other grouping of heads
    (8, 8, 17000),     # 64 rows: two row groups of four waves, ~133 chunks per wave
    (2, 16, 34567),    # 32 rows, ragged tail page
    (5, 8, 17000),     # 40 rows: the second group's second tile holds no row
])
def test_verify_rows_walk_more_than_64_chunks(n_q, G, ctx):
    n_kv, D = 2, 256
    c, rng = _case(1000 * n_q + G, ctx, n_kv, D)
    q = rng.standard_normal((n_q, n_kv * G, D)).astype(np.float32)
    scale = 1 / math.sqrt(D)
    out, lse = c.run(q, scale, kernel=STREAM, cps=1000)
    ref, ref_lse = c.ref(q, scale)
    tu.assert_close(out, ref, lse, ref_lse, f"n_q={n_q} G={G} ctx={ctx}")
    again, again_lse = c.run(q, scale, kernel=STREAM, cps=1000)
    assert np.array_equal(out, again) and np.array_equal(lse, again_lse)


@pytest.mark.parametrize("D,G,ctx", [(256, 6, 40000), (128, 8, 33000), (64, 2, 41000)])
def test_one_row_group_with_more_than_256_chunks(D, G, ctx):
    """At most 16 rows but one split of over 256 chunks: no LDS list, the
    fixed order; each of the 8 waves walks more than 128 chunks."""
    n_kv = 2
    c, rng = _case(77 + D, ctx, n_kv, D)
    q = rng.standard_normal((1, n_kv * G, D)).astype(np.float32)
    scale = 1 / math.sqrt(D)
    out, lse = c.run(q, scale, kernel=STREAM, cps=1000)
    ref, ref_lse = c.ref(q, scale)
    tu.assert_close(out, ref, lse, ref_lse, f"D={D} G={G} ctx={ctx}")
    again, again_lse = c.run(q, scale, kernel=STREAM, cps=1000)
    assert np.array_equal(out, again) and np.array_equal(lse, again_lse)


@pytest.mark.parametrize("n_q,G,ctx,bad_page", [
    (4, 6, 34000, 80),     # two tiles per wave: page 80 at a wave's chunk ~80
    (1, 6, 40000, 120),    # one row group, fixed order: page 120 at a wave's chunk ~120
])
def test_bad_page_after_the_first_64_entries(n_q, G, ctx, bad_page):
    """A page-table entry outside the pool that a wave only reads from its
    reloaded entries turns every row that sees it into NaN, and nothing is
    read from it; with the table restored the same call matches the oracle."""
    n_kv, D = 2, 256
    c, rng = _case(500 + bad_page, ctx, n_kv, D)
    q = rng.standard_normal((n_q, n_kv * G, D)).astype(np.float32)
    scale = 1 / 16
    good = c.pt_dev
    bad = good.clone()
    bad[bad_page] = c.L.n_pages + 3
    c.pt_dev = bad
    out, lse = c.run(q, scale, kernel=STREAM, cps=1000)
    assert np.isnan(out).all() and np.isnan(lse).all()
    c.pt_dev = good
    out, lse = c.run(q, scale, kernel=STREAM, cps=1000)
    ref, ref_lse = c.ref(q, scale)
    tu.assert_close(out, ref, lse, ref_lse, "restored table")


def test_verify_batch_with_several_splits_matches_one_split():
    """The same verify batch with the automatic plan (several splits, merged)
    and with one split: both match the oracle."""
    n_kv, D, n_q, G, ctx = 2, 256, 4, 6, 17000
    c, rng = _case(4242, ctx, n_kv, D)
    q = rng.standard_normal((n_q, n_kv * G, D)).astype(np.float32)
    ref, ref_lse = c.ref(q, 1 / 16)
    for cps in (0, 3, 1000):
        out, lse = c.run(q, 1 / 16, kernel=STREAM, cps=cps)
        tu.assert_close(out, ref, lse, ref_lse, f"cps={cps}")
