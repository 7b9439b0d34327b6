"""The oracle's INT2 codec and dense attention, pinned (CPU only).

The codec: blocks of 128 values of one (token, KV head) row, an fp16 scale
d = (max - min) / 3 and an fp16 zero-point (the minimum), 2-bit codes; the
page fixes its size ("OSCAR2 KV Cache benchmark", compression-ratio table:
36 bytes per 128 values, 2.25 bit) and that K and V use the same codec.
Pins: that printed size, hand blocks (levels, ties, a constant block, a
negative range), the reconstruction error bound, pure-Python brute force bit
for bit, and attention over the dequantized cache against the Q8_0/Q4_0
attention (the same definition) and its closed forms.
"""
import json
import math
import os

import numpy as np
import pytest

import oracle
from oracle import brute

GOLDEN = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "page_numbers.json")))


def _f16(x):
    return float(np.float16(x))


def test_int2_block_size_is_the_printed_one():
    g = GOLDEN["compression_table"]["oscar2"]
    assert oracle.int2_block_bytes() == g["bytes_per_128"] == 36
    assert oracle.int2_block_bytes() * 8 / 128 == g["bits"] == 2.25


def test_levels_are_exact():
    x = np.array([0, 1, 2, 3] * 32, dtype=np.float32)[None]
    c, s, z = oracle.quantize_int2(x)
    assert np.array_equal(c[0], x[0].astype(np.uint8))
    assert s[0, 0] == 0x3C00 and z[0, 0] == 0x0000                 # scale 1.0, zero 0.0
    assert np.array_equal(oracle.dequant_int2(c, s, z), x.astype(np.float64))


def test_ties_go_up_and_ends_map_to_0_and_3():
    x = np.zeros(128, dtype=np.float32)
    x[1], x[2], x[3], x[4] = 3.0, 0.5, 1.5, 2.5                      # d = 1, min 0
    c, s, z = oracle.quantize_int2(x[None])
    assert c[0, 0] == 0 and c[0, 1] == 3
    assert (c[0, 2], c[0, 3], c[0, 4]) == (1, 2, 3)                  # halfway values round up


def test_constant_block():
    x = np.full((1, 128), 5.25, dtype=np.float32)
    c, s, z = oracle.quantize_int2(x)
    assert (c == 0).all() and s[0, 0] == 0 and z[0, 0] == 0x4540    # fp16(5.25)
    assert (oracle.dequant_int2(c, s, z) == 5.25).all()


def test_negative_range():
    x = np.linspace(-3.0, 0.0, 128, dtype=np.float32)[None]          # min -3, max 0, d = 1
    c, s, z = oracle.quantize_int2(x)
    assert s[0, 0] == 0x3C00 and z[0, 0] == 0xC200                  # 1.0 and -3.0
    want = np.minimum(3, np.floor((x[0].astype(np.float64) + 3.0) + 0.5)).astype(np.uint8)
    assert np.array_equal(c[0], want)


@pytest.mark.parametrize("mag", [1.0, 30.0, 1e-3])
def test_error_bound(mag):
    rng = np.random.default_rng(7)
    x = (rng.standard_normal((64, 256)) * mag).astype(np.float32)
    c, s, z = oracle.quantize_int2(x)
    xh = oracle.dequant_int2(c, s, z)
    xb = x.reshape(64, 2, 128).astype(np.float64)
    mn, mx = xb.min(-1), xb.max(-1)
    d = (mx - mn) / 3
    hd = oracle.f16_bits_to_f64_array(s)
    hz = oracle.f16_bits_to_f64_array(z)
    bound = d / 2 + 3 * np.abs(hd - d) + np.abs(hz - mn) + 1e-6 * mag
    err = np.abs(xh.reshape(64, 2, 128) - xb).max(-1)
    assert (err <= bound).all()


def test_brute_force_bit_exact():
    rng = np.random.default_rng(11)
    blocks = [rng.standard_normal(128).astype(np.float32) * m for m in (1.0, 7.0, 0.01)]
    # a block with exact halfway values on a grid
    grid = np.array([0.0, 1.5, 3.0] + [0.5, 2.5] * 62 + [1.0], dtype=np.float32)
    blocks.append(grid)
    for xb in blocks:
        c, s, z = oracle.quantize_int2(xb[None])
        bc, bs, bz = brute.quant_int2_block(xb.tolist())
        assert list(c[0]) == bc and s[0, 0] == bs and z[0, 0] == bz


def test_dense_attention_equals_quantized_attention():
    """attention_dense over the dequantized Q8_0/Q4_0 cache is the same
    definition as the pinned Q8_0/Q4_0 attention."""
    rng = np.random.default_rng(13)
    k = rng.standard_normal((300, 2, 128)).astype(np.float32)
    v = rng.standard_normal((300, 2, 128)).astype(np.float32)
    q = rng.standard_normal((3, 6, 128)).astype(np.float32)
    cache = oracle.QuantCache.from_float(k, v)
    a, la, _ = oracle.attention(q, cache, 0.1)
    b, lb, _ = oracle.attention_dense(q, cache.k_hat(), cache.v_hat(), 0.1)
    assert np.allclose(a, b, rtol=1e-12, atol=1e-12) and np.allclose(la, lb, rtol=1e-12, atol=1e-12)


def test_int2_attention_closed_forms():
    rng = np.random.default_rng(17)
    k = rng.standard_normal((1, 1, 128)).astype(np.float32)
    v = rng.standard_normal((1, 1, 128)).astype(np.float32)
    q = rng.standard_normal((1, 2, 128)).astype(np.float32)
    c = oracle.Int2Cache.from_float(k, v)
    out, lse, _ = oracle.attention(q, c, 0.2)
    vh = c.v_hat()[0, 0]
    assert np.allclose(out[0], vh[None], rtol=0, atol=1e-14)         # one key: its value
    s0 = 0.2 * float(q[0, 0].astype(np.float64) @ c.k_hat()[0, 0])
    assert abs(lse[0, 0] - s0) < 1e-12
    # q = 0: every score equal, the output is the mean of the values
    k = rng.standard_normal((50, 1, 128)).astype(np.float32)
    v = rng.standard_normal((50, 1, 128)).astype(np.float32)
    c = oracle.Int2Cache.from_float(k, v)
    out, lse, _ = oracle.attention(np.zeros((1, 1, 128), np.float32), c, 0.2)
    assert np.allclose(out[0, 0], c.v_hat()[:, 0].mean(0), rtol=1e-12, atol=1e-14)
    assert abs(lse[0, 0] - math.log(50)) < 1e-12
