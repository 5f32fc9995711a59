"""Pins of the oracle's rotations (Hadamard, RoPE) -- no GPU."""

import math

import numpy as np
import pytest

from oracle import transform


@pytest.mark.parametrize("n", [8, 16, 32, 64, 128, 256])
def test_hadamard_orthogonal_symmetric(n):
    H = transform.hadamard_dense(n)
    assert np.array_equal(H, H.T)
    assert np.array_equal(H @ H.T, n * np.eye(n))
    assert np.all(np.abs(H) == 1.0)
    # Sylvester recursion H_2n = [[H, H], [H, -H]]
    if n >= 16:
        h = transform.hadamard_dense(n // 2)
        assert np.array_equal(H, np.block([[h, h], [h, -h]]))


@pytest.mark.parametrize("n", [8, 64, 128, 256])
def test_fast_transform_equals_dense(n):
    rng = np.random.default_rng(n)
    H = transform.hadamard_dense(n)
    vi = rng.integers(-1000, 1000, size=(50, n)).astype(np.float64)
    assert np.array_equal(transform.fwht_f64(vi), vi @ H.T)
    # integer-valued fp32 inputs stay exact in fp32 (|sums| < 2^24)
    assert np.array_equal(transform.fwht_f32(vi.astype(np.float32)), (vi @ H.T).astype(np.float32))
    v = rng.normal(size=(50, n))
    np.testing.assert_allclose(transform.fwht_f64(v), v @ H.T, rtol=0, atol=1e-12 * n)
    # fp32 transform: error bounded by log2(n) roundings of partial sums
    v32 = v.astype(np.float32)
    ref = v32.astype(np.float64) @ H.T
    err = np.abs(transform.fwht_f32(v32) - ref).max(axis=1)
    bound = math.log2(n) * 2.0 ** -24 * np.abs(v32).sum(axis=1) * 2
    assert np.all(err <= bound)
    # norm preservation of the orthonormal rotation
    np.testing.assert_allclose(np.linalg.norm(transform.fwht_f64(v), axis=1) / math.sqrt(n),
                               np.linalg.norm(v, axis=1), rtol=1e-13)


def test_fwht_is_its_own_inverse_up_to_n():
    rng = np.random.default_rng(0)
    v = rng.normal(size=(10, 128))
    np.testing.assert_allclose(transform.fwht_f64(transform.fwht_f64(v)) / 128, v, atol=1e-13)


@pytest.mark.parametrize("d,theta", [(128, 5e5), (96, 1e4), (128, 1e6), (8, 1e4)])
def test_rope_roundtrip_and_invariants(d, theta):
    rng = np.random.default_rng(d)
    T = 300
    pos = np.concatenate([np.arange(T - 3), [32767, 65535, 131071]])
    x = rng.normal(size=(2, T, d))
    y = transform.rope_forward_f64(x, pos, theta)
    np.testing.assert_allclose(transform.rope_inverse_f64(y, pos, theta), x, atol=1e-12)
    h = d // 2
    # each (i, i + d/2) pair is rotated, so its norm is kept
    np.testing.assert_allclose(y[..., :h] ** 2 + y[..., h:] ** 2,
                               x[..., :h] ** 2 + x[..., h:] ** 2, rtol=1e-12)
    # position 0 is the identity
    assert np.array_equal(transform.rope_forward_f64(x[:, :1], [0], theta), x[:, :1])
    # frequencies: omega_0 = 1, strictly decreasing for theta > 1
    w = transform.rope_freqs(theta, d)
    assert w[0] == 1.0 and np.all(np.diff(w) < 0)
    np.testing.assert_allclose(w[-1], theta ** (-(d - 2) / d), rtol=1e-15)
    # fp32 removal against fp64 removal
    c32, s32 = transform.rope_table_f32(pos, theta, d)
    y32 = y.astype(np.float32)
    got = transform.rope_inverse_f32(y32, c32, s32)
    ref = transform.rope_inverse_f64(y32.astype(np.float64), pos, theta)
    assert np.max(np.abs(got - ref)) < 4 * 2.0 ** -24 * np.abs(y32).max() * 2
    c0, s0 = transform.rope_table_f32([0], theta, d)
    assert np.all(c0 == 1) and np.all(s0 == 0)
