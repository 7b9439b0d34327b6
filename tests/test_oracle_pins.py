"""The oracle pinned to facts other than itself (CPU only).

Pins: numbers printed on the pages (tests/golden/page_numbers.json), hand-
derived quantization blocks, the IEEE binary16 rounding of numpy, error
bounds of the quantizers, closed forms of attention (one key; equal scores),
split-and-merge algebra, GQA replication, a numpy/scipy route, and
pure-Python brute force (oracle/brute.py).
"""
import json
import math
import os

import numpy as np
import pytest
from scipy.special import logsumexp

import oracle
from oracle import brute
import synth

GOLDEN = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "page_numbers.json")))


# --------------------------------------------------------------------------
# byte formulas against the pages' printed numbers
# --------------------------------------------------------------------------

def test_fp16_worked_example():
    g = GOLDEN["fp16_worked_example"]
    assert oracle.kv_bytes_per_token_f16(g["layers"], g["kv_heads"], g["head_dim"]) == g["bytes_per_token"]


def test_fp16_growth_rows():
    g = GOLDEN["fp16_growth_table"]
    per_tok = oracle.kv_bytes_per_token_f16(32, 8, 128)
    assert per_tok == g["bytes_per_token"]
    for tokens, gb in g["rows"]:
        assert abs(tokens * per_tok / 1e9 - gb) <= g["rel_tol"] * gb


def test_q8k_q4v_bytes_per_token_and_q4_block_size():
    g = GOLDEN["q8k_q4v_bytes_per_token"]
    assert oracle.kv_bytes_per_token_q8k_q4v(g["layers"], g["kv_heads"], g["head_dim"]) == g["bytes_per_token"]
    # the total forces the Q4_0 block size once the Q8_0 block is 34 bytes
    blocks = g["layers"] * g["kv_heads"] * g["head_dim"] // 32
    assert g["bytes_per_token"] // blocks - oracle.q8_0_block_bytes() == 18 == oracle.q4_0_block_bytes()


def test_kv_bytes_at_262k():
    g = GOLDEN["kv_bytes_262k"]
    total = oracle.kv_bytes_per_token_q8k_q4v(16, 4, 256) * g["tokens"]
    assert total == 6_979_321_856
    assert round(total / 1e9, 2) == g["gb"]


def test_compression_table():
    g = GOLDEN["compression_table"]
    q8_per_128 = (128 // 32) * oracle.q8_0_block_bytes()
    assert q8_per_128 == g["q8_0"]["bytes_per_128"]
    assert q8_per_128 * 8 / 128 == g["q8_0"]["bits"]
    f16_per_128 = oracle.kv_bytes_per_token_f16(1, 1, 128) // 2   # one of K/V
    assert f16_per_128 == g["f16"]["bytes_per_128"]


# --------------------------------------------------------------------------
# fp16 rounding against numpy's IEEE binary16
# --------------------------------------------------------------------------

def test_f16_conversion_matches_numpy():
    rng = np.random.default_rng(1)
    vals = np.concatenate([
        rng.standard_normal(4000).astype(np.float32) * np.float32(10.0) ** rng.integers(-9, 6, 4000),
        np.array([0.0, -0.0, 65504.0, 65519.99, 65520.0, 1e9, -1e9, 2.0 ** -24, 2.0 ** -25,
                  2.0 ** -25 * 1.0000001, 3 * 2.0 ** -26, 2.0 ** -14, 2.0 ** -14 * (1 - 2.0 ** -11),
                  1.0 + 2.0 ** -11, 1.0 + 3 * 2.0 ** -11, 2049.0, 2051.0], dtype=np.float32),
    ]).astype(np.float32)
    want = vals.astype(np.float16).view(np.uint16)
    got = np.array([oracle.f32_to_f16_bits(v) for v in vals], dtype=np.uint16)
    assert np.array_equal(got, want)
    back = np.array([oracle.f16_bits_to_f32(int(b)) for b in want], dtype=np.float32)
    assert np.array_equal(back, want.view(np.float16).astype(np.float32))


# --------------------------------------------------------------------------
# hand-derived blocks (the readings of the block rules)
# --------------------------------------------------------------------------

def _block(vals):
    x = np.zeros((1, 32), dtype=np.float32)
    x[0, :len(vals)] = vals
    return x


def test_q8_0_ties_round_away_from_zero():
    # max |x| = 127 gives d = 1 exactly; halves round away from zero
    x = _block([127.0, 0.5, 2.5, -0.5, -2.5, 1.5, -1.5, 0.49, -126.5])
    codes, scales = oracle.quantize_q8_0(x)
    assert codes[0, :9].tolist() == [127, 1, 3, -1, -3, 2, -2, 0, -127]
    assert codes[0, 9:].tolist() == [0] * 23
    assert scales.tolist() == [[0x3C00]]


def test_q4_0_magnitude_tie_keeps_first_index():
    # x0 = 16 and x1 = -16 tie on |x|: the first wins, m = 16, d = -2
    codes, scales = oracle.quantize_q4_0(_block([16.0, -16.0]))
    assert scales.tolist() == [[0xC000]]
    assert codes[0].tolist() == [0, 15] + [8] * 30
    vhat = oracle.dequant_q4_0(codes, scales)
    assert vhat[0, :3].tolist() == [16.0, -14.0, 0.0]


def test_q4_0_rounding_and_clamp():
    # m = -8 gives d = 1: code = min(15, floor(x + 8.5))
    codes, scales = oracle.quantize_q4_0(_block([-8.0, 2.5, -2.5, 7.5, 0.49, -0.5, 3.4999]))
    assert scales.tolist() == [[0x3C00]]
    assert codes[0, :7].tolist() == [0, 11, 6, 15, 8, 8, 11]


def test_zero_blocks():
    kc, ks = oracle.quantize_q8_0(_block([]))
    assert ks.tolist() == [[0x0000]] and kc[0].tolist() == [0] * 32
    vc, vs = oracle.quantize_q4_0(_block([]))
    assert vs.tolist() == [[0x8000]] and vc[0].tolist() == [8] * 32     # d = +0 / -8 = -0
    neg0 = np.full((1, 32), -0.0, dtype=np.float32)
    assert oracle.quantize_q4_0(neg0)[1].tolist() == [[0x8000]]
    assert oracle.quantize_q8_0(neg0)[1].tolist() == [[0x0000]]


# --------------------------------------------------------------------------
# quantizer error bounds on random blocks
# --------------------------------------------------------------------------

@pytest.mark.parametrize("mag", [1e-3, 1.0, 37.0, 1e3])
def test_quant_error_bounds(mag):
    rng = np.random.default_rng(7)
    x = (rng.standard_normal((500, 32)) * mag).astype(np.float32)
    x64 = x.astype(np.float64)
    kc, ks = oracle.quantize_q8_0(x)
    khat = oracle.dequant_q8_0(kc, ks)
    d = np.abs(x64).max(axis=1) / 127.0
    h = oracle.f16_bits_to_f64_array(ks)[:, 0]
    bound = d / 2 * (1 + 1e-4) + 127 * np.abs(h - d)
    assert np.all(np.abs(x64 - khat).max(axis=1) <= bound)
    assert np.all(np.abs(kc.astype(int)) <= 127)

    vc, vs = oracle.quantize_q4_0(x)
    vhat = oracle.dequant_q4_0(vc, vs)
    k = np.argmax(np.abs(x64), axis=1)
    m = x64[np.arange(500), k]
    dv = m / -8.0
    hv = oracle.f16_bits_to_f64_array(vs)[:, 0]
    # the largest-magnitude element maps to code 0 and reconstructs up to fp16(d)
    assert np.all(vc[np.arange(500), k] == 0)
    assert np.all(np.abs(vhat[np.arange(500), k] - m) <= 8 * np.abs(hv - dv) + 1e-12)
    # every element within |d| (half a step, a full step on the clamped top code)
    assert np.all(np.abs(x64 - vhat).max(axis=1) <= np.abs(dv) * (1 + 1e-4) + 8 * np.abs(hv - dv))
    assert vc.max() <= 15


# --------------------------------------------------------------------------
# attention: closed forms and invariants
# --------------------------------------------------------------------------

def _random_cache(rng, ctx, n_kv, D, scale_k=1.0, scale_v=1.0):
    k = (rng.standard_normal((ctx, n_kv, D)) * scale_k).astype(np.float32)
    v = (rng.standard_normal((ctx, n_kv, D)) * scale_v).astype(np.float32)
    return k, v, oracle.QuantCache.from_float(k, v)


def _numpy_attention(q, cache, scale, ctx=None):
    """Independent route: dequantize, then matmul / logsumexp from numpy+scipy."""
    ctx = cache.ctx if ctx is None else ctx
    khat, vhat = cache.k_hat()[:ctx], cache.v_hat()[:ctx]
    n_q, n_heads, D = q.shape
    G = n_heads // cache.n_kv
    out = np.zeros((n_q, n_heads, D))
    lse = np.zeros((n_q, n_heads))
    for h in range(n_heads):
        kk, vv = khat[:, h // G, :], vhat[:, h // G, :]
        s = scale * (q[:, h, :].astype(np.float64) @ kk.T)       # [n_q][ctx]
        pos = ctx - n_q + np.arange(n_q)
        s = np.where(np.arange(ctx)[None, :] <= pos[:, None], s, -np.inf)
        lse[:, h] = logsumexp(s, axis=1)
        out[:, h, :] = np.exp(s - lse[:, h:h + 1]) @ vv
    return out, lse


def test_single_key_returns_its_value():
    rng = np.random.default_rng(2)
    k, v, cache = _random_cache(rng, 1, 2, 64)
    q = rng.standard_normal((1, 6, 64)).astype(np.float32)
    out, lse, _ = oracle.attention(q, cache, 0.125)
    vhat, khat = cache.v_hat(), cache.k_hat()
    for h in range(6):
        assert np.array_equal(out[0, h], vhat[0, h // 3])
        assert lse[0, h] == pytest.approx(0.125 * float(q[0, h].astype(np.float64) @ khat[0, h // 3]), rel=1e-13, abs=1e-13)


def test_equal_scores_give_mean_of_values():
    rng = np.random.default_rng(3)
    k, v, cache = _random_cache(rng, 37, 1, 64)
    # q = 0: every score is 0
    out, lse, _ = oracle.attention(np.zeros((1, 2, 64), np.float32), cache, 0.125)
    assert np.allclose(out[0, 0], cache.v_hat()[:, 0].mean(axis=0), rtol=0, atol=1e-13)
    assert lse[0, 0] == pytest.approx(math.log(37), rel=1e-14)
    # every key the same row: scores equal for any q
    k_same = np.repeat(k[:1], 37, axis=0)
    cache2 = oracle.QuantCache.from_float(k_same, v)
    q = rng.standard_normal((1, 2, 64)).astype(np.float32)
    out2, _, _ = oracle.attention(q, cache2, 0.125)
    assert np.allclose(out2[0, 1], cache2.v_hat()[:, 0].mean(axis=0), rtol=0, atol=1e-13)


@pytest.mark.parametrize("n_q,G,D", [(1, 6, 64), (4, 3, 32), (5, 1, 96)])
def test_matches_numpy_route(n_q, G, D):
    rng = np.random.default_rng(4 + n_q)
    k, v, cache = _random_cache(rng, 300, 2, D)
    q = rng.standard_normal((n_q, 2 * G, D)).astype(np.float32)
    out, lse, _ = oracle.attention(q, cache, 1 / math.sqrt(D))
    ref_out, ref_lse = _numpy_attention(q, cache, 1 / math.sqrt(D))
    assert np.allclose(out, ref_out, rtol=1e-12, atol=1e-13)
    assert np.allclose(lse, ref_lse, rtol=1e-13, atol=1e-13)


def test_split_merge_equals_unsplit():
    rng = np.random.default_rng(5)
    k, v, cache = _random_cache(rng, 700, 2, 64, scale_k=3.0)
    q = rng.standard_normal((3, 4, 64)).astype(np.float32)
    out, lse, _ = oracle.attention(q, cache, 0.125)
    for cuts in ([0, 256, 512, 700], [0, 1, 699, 700], sorted({0, 700, *rng.integers(1, 700, 9).tolist()}),
                 [0, 698, 700, 700]):
        parts = [oracle.attention_partial(q, cache, 0.125, a, b) for a, b in zip(cuts[:-1], cuts[1:])]
        for i in range(3):
            for h in range(4):
                m = np.array([p[0][i, h] for p in parts])
                l = np.array([p[1][i, h] for p in parts])
                acc = np.stack([p[2][i, h] for p in parts])
                o, ls = oracle.merge(m, l, acc)
                assert np.allclose(o, out[i, h], rtol=1e-12, atol=1e-14)
                assert ls == pytest.approx(lse[i, h], rel=1e-13, abs=1e-13)


def test_gqa_equals_replicated_heads():
    rng = np.random.default_rng(6)
    k, v, cache = _random_cache(rng, 90, 2, 64)
    q = rng.standard_normal((2, 6, 64)).astype(np.float32)
    out, lse, _ = oracle.attention(q, cache, 0.125)
    rep = oracle.QuantCache.from_float(np.repeat(k, 3, axis=1), np.repeat(v, 3, axis=1))
    out_r, lse_r, _ = oracle.attention(q, rep, 0.125)
    assert np.array_equal(out, out_r) and np.array_equal(lse, lse_r)


def test_causality_and_rows_subset():
    rng = np.random.default_rng(8)
    k, v, cache = _random_cache(rng, 50, 1, 32)
    q = rng.standard_normal((4, 2, 32)).astype(np.float32)
    out, lse, _ = oracle.attention(q, cache, 0.2)
    # changing the last key leaves every query but the last unchanged
    k2 = k.copy(); k2[-1] += 5.0
    v2 = v.copy(); v2[-1] -= 3.0
    out2, _, _ = oracle.attention(q, oracle.QuantCache.from_float(k2, v2), 0.2)
    assert np.array_equal(out[:3], out2[:3]) and not np.allclose(out[3], out2[3])
    sub, sub_lse = oracle.attention(q, cache, 0.2, rows=[(3, 1), (0, 0)])
    assert np.array_equal(sub[0], out[3, 1]) and np.array_equal(sub[1], out[0, 0])
    assert sub_lse[0] == lse[3, 1]
    # a shorter ctx is the same as a cache holding only the first ctx tokens
    short, _, _ = oracle.attention(q, cache, 0.2, ctx=20)
    short_ref, _, _ = oracle.attention(q, oracle.QuantCache.from_float(k[:20], v[:20]), 0.2)
    assert np.array_equal(short, short_ref)


# --------------------------------------------------------------------------
# brute force: pure-Python loops agree with the C oracle
# --------------------------------------------------------------------------

@pytest.mark.parametrize("seed,ctx,n_kv,G,D,n_q,mag", [
    (0, 5, 1, 2, 32, 1, 1.0),
    (1, 9, 2, 3, 64, 3, 1.0),
    (2, 7, 1, 1, 32, 2, 1e-3),
    (3, 6, 2, 2, 32, 6, 250.0),
])
def test_brute_force_agrees(seed, ctx, n_kv, G, D, n_q, mag):
    rng = np.random.default_rng(100 + seed)
    k = (rng.standard_normal((ctx, n_kv, D)) * mag).astype(np.float32)
    v = (rng.standard_normal((ctx, n_kv, D)) * mag).astype(np.float32)
    # plant exact ties and zero blocks
    k[0, 0, :32] = 0.0
    v[-1, 0, 3] = -np.abs(v[-1, 0]).max()
    v[-1, 0, 4] = -v[-1, 0, 3]
    q = rng.standard_normal((n_q, n_kv * G, D)).astype(np.float32)
    cache = oracle.QuantCache.from_float(k, v)
    bkc, bks = brute.quantize_rows(k.reshape(-1, D).tolist(), "q8_0")
    bvc, bvs = brute.quantize_rows(v.reshape(-1, D).tolist(), "q4_0")
    assert np.array_equal(cache.k_codes.reshape(-1, D), np.array(bkc))
    assert np.array_equal(cache.k_scales.reshape(-1, D // 32), np.array(bks))
    assert np.array_equal(cache.v_codes.reshape(-1, D), np.array(bvc))
    assert np.array_equal(cache.v_scales.reshape(-1, D // 32), np.array(bvs))
    scale = 1 / math.sqrt(D)
    out, lse, _ = oracle.attention(q, cache, scale)
    bout, blse = brute.attention(q.tolist(), k.tolist(), v.tolist(), n_kv, scale)
    assert np.allclose(out, np.array(bout), rtol=1e-12, atol=1e-12 * mag)
    assert np.allclose(lse, np.array(blse), rtol=1e-12, atol=1e-12)


# --------------------------------------------------------------------------
# input generator properties (shared by both sides)
# --------------------------------------------------------------------------

def test_synth_prefix_and_thread_independence():
    a = synth.normal((0, 9, 0, 1), (5000, 4, 256), threads=1)
    b = synth.normal((0, 9, 0, 1), (5000, 4, 256), threads=8)
    c = synth.normal((0, 9, 0, 1), (4097, 4, 256))
    assert np.array_equal(a, b)
    assert np.array_equal(a[:4097], c)
    assert a.dtype == np.float32 and abs(float(a.mean())) < 0.01 and abs(float(a.std()) - 1) < 0.01
