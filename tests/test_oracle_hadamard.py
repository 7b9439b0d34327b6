"""The oracle's Hadamard rotation, pinned (CPU only).

The pages rotate K and V by a Hadamard matrix (per head of dimension 256)
before the 2-bit cache stores them ("OSCAR2 KV Cache benchmark", rotation
model conversion).  Pins: the matrix equals scipy's Hadamard matrix; it is
orthogonal up to n; the normalized rotation is an involution and keeps
norms; rotating q, k and v and rotating the output back gives the same
attention (float, dense); and, on keys and values with outlier channels, the
rotated 2-bit cache is more accurate than the plain one (the rotation's
purpose).
"""
import numpy as np
import pytest
import scipy.linalg

import oracle


@pytest.mark.parametrize("n", [1, 2, 4, 8, 64, 128, 256, 1024])
def test_matrix_is_scipys(n):
    assert np.array_equal(oracle.hadamard_matrix(n), scipy.linalg.hadamard(n).astype(np.float64))


@pytest.mark.parametrize("n", [2, 64, 256])
def test_orthogonal_involution_norm(n):
    h = oracle.hadamard_matrix(n)
    assert np.array_equal(h @ h.T, n * np.eye(n))
    x = np.random.default_rng(n).standard_normal((5, n))
    y = oracle.hadamard(x)
    np.testing.assert_allclose(oracle.hadamard(y), x, rtol=0, atol=1e-12)
    np.testing.assert_allclose(np.linalg.norm(y, axis=1), np.linalg.norm(x, axis=1), rtol=1e-12)


def test_known_rotation():
    # a unit vector e_0 maps to the constant row 1/sqrt(n); the constant row back to e_0
    y = oracle.hadamard(np.eye(4)[:1])
    assert np.allclose(y, 0.5)
    assert np.allclose(oracle.hadamard(np.full((1, 4), 0.5)), np.eye(4)[:1])


def test_rotated_attention_is_the_same_attention():
    rng = np.random.default_rng(3)
    ctx, n_kv, G, D = 300, 2, 3, 128
    q = rng.standard_normal((2, n_kv * G, D)).astype(np.float32)
    k = rng.standard_normal((ctx, n_kv, D))
    v = rng.standard_normal((ctx, n_kv, D))
    ref, ref_lse, _ = oracle.attention_dense(q, k, v, 0.1)
    qr = oracle.hadamard(q).astype(np.float32)
    out_r, lse_r, _ = oracle.attention_dense(qr, oracle.hadamard(k), oracle.hadamard(v), 0.1)
    # q is rounded to fp32 after rotating (the attention takes fp32 queries)
    np.testing.assert_allclose(oracle.hadamard(out_r), ref, rtol=0, atol=2e-6)
    np.testing.assert_allclose(lse_r, ref_lse, rtol=0, atol=2e-6)


def test_rotation_helps_the_2bit_cache_with_outliers():
    rng = np.random.default_rng(8)
    ctx, n_kv, G, D = 2048, 1, 4, 256
    k = rng.standard_normal((ctx, n_kv, D)).astype(np.float32)
    v = rng.standard_normal((ctx, n_kv, D)).astype(np.float32)
    for x in (k, v):                                   # 4 outlier channels, x20
        x[:, :, [5, 77, 130, 201]] *= 20.0
    q = rng.standard_normal((1, n_kv * G, D)).astype(np.float32)
    scale = 1.0 / 16
    exact, _, _ = oracle.attention_dense(q, k, v, scale)
    plain, _, _ = oracle.attention(q, oracle.Int2Cache.from_float(k, v), scale)
    kr = oracle.hadamard(k).astype(np.float32)
    vr = oracle.hadamard(v).astype(np.float32)
    qr = oracle.hadamard(q).astype(np.float32)
    rot, _, _ = oracle.attention(qr, oracle.Int2Cache.from_float(kr, vr), scale)

    def rms(a):
        return float(np.sqrt(np.mean(np.square(a))))
    # the stored values: the rotation spreads the outliers over every channel
    # of the row, so the 128-value blocks are narrower (the rotation keeps
    # norms, so the errors are comparable)
    for x, xr in ((k, kr), (v, vr)):
        c, cr = oracle.Int2Cache.from_float(x, x), oracle.Int2Cache.from_float(xr, xr)
        assert rms(cr.k_hat() - xr) < 0.5 * rms(c.k_hat() - x)
    # the attention output (rms: a few outlier keys decide the maximum error)
    err_plain = rms(plain - exact)
    err_rot = rms(oracle.hadamard(rot) - exact)
    assert err_rot < 0.6 * err_plain, (err_rot, err_plain)
