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


LLAMA31 = transform.RopeScaling("llama3", 8.0, 1.0, 4.0, 8192)


def test_rope_scaling_factor_one_is_identity():
    w = transform.rope_freqs(5e5, 128)
    assert np.array_equal(transform.rope_freqs(5e5, 128, transform.RopeScaling("linear", 1.0)), w)
    one = transform.RopeScaling("llama3", 1.0, 1.0, 4.0, 8192)
    np.testing.assert_allclose(transform.rope_freqs(5e5, 128, one), w, rtol=2e-16)


def test_linear_scaling_is_position_division():
    """RoPE with linear factor f at position p equals unscaled RoPE at p / f."""
    rng = np.random.default_rng(1)
    x = rng.normal(size=(3, 40, 64))
    pos = np.arange(40) * 4 + 8000
    lin = transform.RopeScaling("linear", 4.0)
    a = transform.rope_forward_f64(x, pos, 1e4, lin)
    b = transform.rope_forward_f64(x, pos // 4, 1e4)
    np.testing.assert_allclose(a, b, atol=1e-9)
    np.testing.assert_allclose(transform.rope_inverse_f64(a, pos, 1e4, lin), x, atol=1e-12)


def test_llama3_scaling_bands():
    """Llama-3.1-8B: theta 5e5, d 128, factor 8, low 1, high 4, C 8192.
    By hand: w_i > 2 pi / 2048 (kept) for i <= 28, w_i < 2 pi / 8192
    (divided by 8) for i >= 35, i = 29..34 in between."""
    w = transform.rope_freqs(5e5, 128)
    ws = transform.rope_freqs(5e5, 128, LLAMA31)
    assert np.array_equal(ws[:29], w[:29])
    assert np.array_equal(ws[35:], w[35:] / 8.0)
    mid = ws[29:35] / w[29:35]
    assert np.all((mid > 1 / 8) & (mid < 1))
    # between w / f and w, and falling with i like the unscaled frequencies
    assert np.all(ws <= w) and np.all(ws >= w / 8)
    assert np.all(np.diff(ws) < 0)
    # the ratio w'/w falls monotonically across the middle band
    assert np.all(np.diff(mid) < 0)


def test_llama3_scaling_continuous_at_band_edges():
    """At wavelength C / high the scaled frequency is w itself, at C / low it
    is w / f, approached from either side."""
    s = LLAMA31
    w_hi = 2 * math.pi * s.high_freq_factor / s.original_max   # edge of the kept band
    w_lo = 2 * math.pi * s.low_freq_factor / s.original_max    # edge of the divided band
    eps = 1e-9
    out = transform.scale_freqs([w_hi * (1 + eps), w_hi * (1 - eps),
                                 w_lo * (1 + eps), w_lo * (1 - eps)], s)
    np.testing.assert_allclose(out[:2], w_hi, rtol=1e-7)
    np.testing.assert_allclose(out[2:], w_lo / s.factor, rtol=1e-7)
    # scaling then inverting the rotation is the identity
    rng = np.random.default_rng(2)
    x = rng.normal(size=(2, 30, 128))
    pos = np.arange(30) + 60000
    y = transform.rope_forward_f64(x, pos, 5e5, s)
    np.testing.assert_allclose(transform.rope_inverse_f64(y, pos, 5e5, s), x, atol=1e-12)


@pytest.mark.parametrize("d,theta", [(128, 5e5), (96, 1e4), (8, 1e4)])
def test_rope_direction_hand_value(d, theta):
    """Split-half RoPE in the rotate-half convention rotates the pair
    (x_i, x_{i+d/2}) by +p w_i: by hand, e_0 at position 1 (w_0 = 1) becomes
    cos(1) e_0 + sin(1) e_{d/2}, and e_1 at position 2 becomes
    cos(2 w_1) e_1 + sin(2 w_1) e_{1+d/2} with w_1 = theta^(-2/d).  Removal
    turns e_0 at position 1 into cos(1) e_0 - sin(1) e_{d/2}.  A flipped sign
    of sin anywhere fails these (round trips alone do not see it)."""
    h = d // 2
    e0 = np.zeros((1, 1, d))
    e0[..., 0] = 1.0
    want = np.zeros(d)
    want[0], want[h] = math.cos(1.0), math.sin(1.0)
    np.testing.assert_allclose(transform.rope_forward_f64(e0, [1], theta)[0, 0], want,
                               rtol=0, atol=1e-15)
    want_inv = want.copy()
    want_inv[h] = -want[h]
    np.testing.assert_allclose(transform.rope_inverse_f64(e0, [1], theta)[0, 0], want_inv,
                               rtol=0, atol=1e-15)
    e1 = np.zeros((1, 1, d))
    e1[..., 1] = 1.0
    w1 = theta ** (-2.0 / d)
    want1 = np.zeros(d)
    want1[1], want1[1 + h] = math.cos(2 * w1), math.sin(2 * w1)
    np.testing.assert_allclose(transform.rope_forward_f64(e1, [2], theta)[0, 0], want1,
                               rtol=0, atol=1e-15)
    # the fp32 diagnostic removal turns the same way
    c32, s32 = transform.rope_table_f32([1], theta, d)
    got = transform.rope_inverse_f32(e0.astype(np.float32)[0], c32, s32)[0]
    np.testing.assert_allclose(got, want_inv, rtol=0, atol=1e-7)


def test_generator_rotates_forward():
    """The seeded key generator applies RoPE in the forward direction (the
    same hand value), so removing it with the codec's inverse undoes it."""
    import torch

    from e8_lattice_vector_amd import synth

    d, h = 16, 8
    x = torch.zeros((1, 3, d), dtype=torch.float64)
    x[0, :, 0] = 1.0
    y = synth._rotary(x, 1e4, positions=[0, 1, 2])[0].numpy()
    for p in range(3):
        want = np.zeros(d)
        want[0], want[h] = math.cos(p), math.sin(p)
        np.testing.assert_allclose(y[p], want, rtol=0, atol=1e-15)
