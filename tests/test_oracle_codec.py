"""Pins of the oracle codec (scale, pack, dequantize, score) -- no GPU."""

import json
import math
import os

import numpy as np
import pytest

from oracle import codec as oc
from oracle import lattice, transform

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "kv_bytes.json")))


def _x(shape, seed, outliers=True):
    rng = np.random.default_rng(seed)
    x = rng.normal(size=shape)
    if outliers:
        x[..., rng.integers(0, shape[-1], 4)] *= 8
    return x.astype(np.float16)


def test_fp16_bytes_per_token_match_pages():
    for m in GOLD["models"]:
        assert oc.fp16_kv_bytes(m["layers"], m["kv_heads"], m["head_dim"]) == m["bytes_per_token"]


def test_bits_per_element_accounting():
    # pages' bpe counts codes + fp16 scale per 128; ours adds one coset bit per 8
    for row in GOLD["bpe"]["rows"]:
        k = oc.Codec(128, row["k"], 128)
        v = oc.Codec(128, row["v"], 128)
        ours = (k.vector_bytes + v.vector_bytes) * 8 / 256
        assert ours - 1 / 8 == pytest.approx(row["bpe"])
    # Llama k2v2, G=128: 36 B per vector -> 18,432 B per token (32 x 8 x 2 vectors)
    assert oc.Codec(128, 2, 128).vector_bytes == 36
    assert 32 * 8 * 2 * 36 == 18432
    # Mistral K3 G=64 (54 B) + V2 G=64 (38 B)
    assert oc.Codec(128, 3, 64).vector_bytes == 54 and oc.Codec(128, 2, 64).vector_bytes == 38


@pytest.mark.parametrize("bits", [2, 3])
@pytest.mark.parametrize("n", [8, 64, 128, 256])
def test_pack_roundtrip(bits, n):
    rng = np.random.default_rng(bits * n)
    idx = rng.integers(0, 1 << bits, size=(3, 5, n)).astype(np.uint8)
    packed = oc.pack_codes(idx, bits)
    assert packed.shape[-1] == n * bits // 8
    assert np.array_equal(oc.unpack_codes(packed, bits, n), idx)
    # coordinate j sits at bits [j*b, j*b + b) of the little-endian stream
    j = n // 2 + 1
    stream = int.from_bytes(packed[1, 2].tobytes(), "little")
    assert (stream >> (j * bits)) & ((1 << bits) - 1) == idx[1, 2, j]
    c = rng.integers(0, 2, size=(3, 5, n // 8)).astype(np.uint8)
    cb = oc.pack_cosets(c, (n // 8 + 7) // 8)
    assert np.array_equal(oc.unpack_cosets(cb, n // 8), c)


@pytest.mark.parametrize("cfg", [
    oc.Codec(128, 2, 0, strict=False, rope_theta=5e5),
    oc.Codec(128, 3, 64, strict=False, rope_theta=1e6),
    oc.Codec(96, 2, 0, strict=True, rope_theta=1e4),
    oc.Codec(8, 2, 8, strict=True),
])
def test_quantize_invariants(cfg):
    x = _x((2, 3, 40, cfg.head_dim), 7)
    for is_key in (False, True):
        q = oc.quantize(x, cfg, is_key=is_key)
        y, a = q["y"], q["a"]
        g = np.abs(y).reshape(y.shape[:-1] + (cfg.n // cfg.G, cfg.G)).max(-1)
        # the group maximum lands on L/2 up to one fp32 rounding of u * r
        assert np.all(np.abs(g - cfg.L / 2) <= cfg.L / 2 * 2.0 ** -23)
        assert q["codes"].shape[-1] == cfg.code_bytes
        assert q["cosets"].shape[-1] == cfg.coset_bytes
        assert q["scales"].shape[-1] == cfg.n_scales
        p = lattice.codeword_points(q["idx"].reshape(-1, 8), q["c"].reshape(-1), cfg.L)
        assert np.all(lattice.in_lattice(p, cfg.strict))
        if cfg.strict:
            assert np.all(q["idx"].reshape(-1, 8).astype(int).sum(-1) % 2 == 0)
        # stored scale is sigma = a / ((L/2) sqrt(n)) rounded once to fp16
        sig = a.astype(np.float64) / ((cfg.L / 2) * math.sqrt(cfg.n))
        assert np.array_equal(q["scales"], sig.astype(np.float16))


def test_zero_vector():
    cfg = oc.Codec(128, 2, 0, strict=True, rope_theta=5e5)
    x = np.zeros((1, 1, 3, 128), np.float16)
    q = oc.quantize(x, cfg, is_key=True)
    assert np.all(q["idx"] == 2) and np.all(q["c"] == 0)
    r = oc.dequantize(q["codes"], q["cosets"], q["scales"], cfg, is_key=True)
    assert np.all(r == 0)


@pytest.mark.parametrize("cfg", [oc.Codec(128, 2, 0), oc.Codec(128, 3, 64, strict=True),
                                 oc.Codec(64, 2, 32)])
def test_dequantize_error_equals_lattice_error(cfg):
    """With d = n and no RoPE the rotation is orthonormal, so the
    reconstruction error equals sum_g sigma16_g^2 |y_g - p_g|^2 (up to the
    fp16/fp32 roundings of the scale and of y)."""
    x = _x((1, 2, 64, cfg.head_dim), 11)
    q = oc.quantize(x, cfg)
    r = oc.dequantize(q["codes"], q["cosets"], q["scales"], cfg)
    err = ((r - x.astype(np.float64)) ** 2).sum(-1)
    p = lattice.codeword_points(q["idx"].reshape(-1, 8), q["c"].reshape(-1), cfg.L)
    p = p.reshape(q["y"].shape)
    s16 = np.repeat(q["scales"].astype(np.float64), cfg.G, -1)
    # z-frame residual with the stored scale: s16 * p vs z = sqrt-normalised u
    z = transform.fwht_f64(np.pad(x.astype(np.float64),
                                  [(0, 0)] * 3 + [(0, cfg.n - cfg.head_dim)])) / math.sqrt(cfg.n)
    pred = ((s16 * p - z) ** 2).sum(-1)
    np.testing.assert_allclose(err, pred, rtol=1e-9, atol=1e-12)
    # and that residual is the lattice error up to the scale rounding
    sig = np.repeat(q["a"].astype(np.float64) / ((cfg.L / 2) * math.sqrt(cfg.n)), cfg.G, -1)
    lat = ((sig * (p - q["y"])) ** 2).sum(-1)
    np.testing.assert_allclose(pred, lat, rtol=5e-3, atol=1e-6)


def test_dequantize_reapplies_rope():
    cfg = oc.Codec(128, 2, 0, rope_theta=5e5)
    x = _x((1, 1, 50, 128), 3)
    pos = np.arange(1000, 1050)
    q = oc.quantize(x, cfg, positions=pos, is_key=True)
    k = oc.dequantize(q["codes"], q["cosets"], q["scales"], cfg, positions=pos, is_key=True)
    k0 = oc.dequantize(q["codes"], q["cosets"], q["scales"], cfg, apply_rope=False)
    np.testing.assert_allclose(transform.rope_inverse_f64(k, pos, 5e5), k0, atol=1e-12)
    rel = np.linalg.norm(k - x.astype(np.float64)) / np.linalg.norm(x.astype(np.float64))
    assert rel < 0.35  # 2-bit: a coarse but bounded reconstruction


def test_score_equals_rotated_query_form():
    """Oracle score (dequantize-then-dot) against the rotated-query form
    q~ . (s16 * p), q~ = H pad(q) / sqrt(n): the identity the table kernel
    uses, computed here independently of codec.score."""
    cfg = oc.Codec(96, 2, 32, strict=True)
    S, H, Hq, T = 2, 2, 6, 30
    k = _x((S, H, T, 96), 5)
    q = _x((S, Hq, 96), 6, outliers=False)
    pk = oc.quantize(k, cfg)
    s = oc.score(q, pk["codes"], pk["cosets"], pk["scales"], cfg)
    qt = transform.fwht_f64(np.pad(q.astype(np.float64), [(0, 0), (0, 0), (0, 32)])) / math.sqrt(128)
    p = lattice.codeword_points(pk["idx"].reshape(-1, 8), pk["c"].reshape(-1), cfg.L).reshape(S, H, T, 128)
    sc = np.repeat(pk["scales"].astype(np.float64), 32, -1)
    for h in range(Hq):
        ref = np.einsum("sd,std->st", qt[:, h], sc[:, h // 3] * p[:, h // 3])
        np.testing.assert_allclose(s[:, h], ref, rtol=1e-12, atol=1e-12)


def test_attend_pins():
    """attend(): one-hot weights give dequantized rows; the sum equals the
    codec-frame form (H sum_t w_t s_t p_t / sqrt(n))[:d] computed here
    independently; linear in the weights."""
    cfg = oc.Codec(96, 2, 32, strict=True)
    S, H, Hq, T = 2, 2, 4, 37
    v = _x((S, H, T, 96), 9, outliers=False)
    pv = oc.quantize(v, cfg)
    planes = (pv["codes"], pv["cosets"], pv["scales"])
    vd = oc.dequantize(*planes, cfg)
    rng = np.random.default_rng(10)
    w = rng.uniform(0, 1, size=(S, Hq, T))
    out = oc.attend(w, *planes, cfg)
    # one-hot weights
    onehot = np.zeros((S, Hq, T))
    onehot[:, :, 5] = 1.0
    np.testing.assert_allclose(oc.attend(onehot, *planes, cfg),
                               np.repeat(vd[:, :, 5, :], Hq // H, axis=1), atol=1e-12)
    # codec-frame identity
    p = lattice.codeword_points(pv["idx"].reshape(-1, 8), pv["c"].reshape(-1), cfg.L).reshape(S, H, T, 128)
    sc = np.repeat(pv["scales"].astype(np.float64), 32, -1)
    for h in range(Hq):
        z = np.einsum("st,stj->sj", w[:, h], sc[:, h // 2] * p[:, h // 2])
        ref = transform.fwht_f64(z)[:, :96] / math.sqrt(128)
        np.testing.assert_allclose(out[:, h], ref, rtol=1e-12, atol=1e-12)
    # linearity
    w2 = rng.normal(size=w.shape)
    np.testing.assert_allclose(oc.attend(2 * w - 3 * w2, *planes, cfg),
                               2 * out - 3 * oc.attend(w2, *planes, cfg), atol=1e-10)


def test_compact_packing_is_a_bijection_on_strict_codewords():
    """Every strict 2-bit cube codeword (36,049) survives fold -> pack ->
    unpack -> unfold; the packed group is exactly 16 bits."""
    P = lattice.enumerate_cube_codebook(4, True)
    assert len(P) == 36049
    c = (np.abs(P[:, 0] - np.round(P[:, 0])) > 0.25).astype(np.uint8)   # half-integer coset
    idx = (P + 2 - c[:, None] / 2).astype(np.uint8)
    assert np.all(idx.astype(int).sum(-1) % 2 == 0)
    packed = oc.pack_codes(oc.fold_cosets(idx, c), 2)
    assert packed.shape == (len(P), 2)
    i2, c2 = oc.unfold_cosets(oc.unpack_codes(packed, 2, 8))
    assert np.array_equal(i2, idx) and np.array_equal(c2, c)
    # 36,049 distinct codewords -> 36,049 distinct 16-bit words
    assert len(np.unique(packed.view(np.uint16))) == len(P)


def test_compact_needs_strict_parity():
    with pytest.raises(ValueError):
        oc.Codec(128, 2, 0, strict=False, compact=True)
    # a relaxed half-integer codeword with an odd index sum does not survive
    idx = np.array([[3, 2, 2, 2, 2, 2, 2, 2]], np.uint8)   # p = (1.5, .5, ..., .5), c = 1
    i2, c2 = oc.unfold_cosets(oc.fold_cosets(idx, [1]))
    assert not np.array_equal(i2, idx)


@pytest.mark.parametrize("bits,G,d", [(2, 0, 128), (3, 64, 128), (2, 32, 96), (3, 8, 8)])
def test_compact_same_reconstruction_as_standard(bits, G, d):
    std = oc.Codec(d, bits, G, strict=True)
    cmp_ = oc.Codec(d, bits, G, strict=True, compact=True)
    assert cmp_.coset_bytes == 0 and cmp_.code_bytes == std.code_bytes
    assert cmp_.vector_bytes * 8 == cmp_.n * bits + 16 * cmp_.n_scales
    x = _x((2, 2, 33, d), 21)
    a, b = oc.quantize(x, std), oc.quantize(x, cmp_)
    assert np.array_equal(a["idx"], b["idx"]) and np.array_equal(a["c"], b["c"])
    assert b["cosets"].shape[-1] == 0
    # the two packings differ exactly in the low bit of idx_7 of each group
    ua = oc.unpack_codes(a["codes"], bits, cmp_.n).reshape(-1, 8)
    ub = oc.unpack_codes(b["codes"], bits, cmp_.n).reshape(-1, 8)
    assert np.array_equal(ua[:, :7], ub[:, :7]) and np.array_equal(ua[:, 7] >> 1, ub[:, 7] >> 1)
    assert np.array_equal(ub[:, 7] & 1, a["c"].reshape(-1))
    ra = oc.dequantize(a["codes"], a["cosets"], a["scales"], std)
    rb = oc.dequantize(b["codes"], b["cosets"], b["scales"], cmp_)
    assert np.array_equal(ra, rb)


@pytest.mark.parametrize("n", [8, 64, 128, 256])
def test_coset_plane_bit_position(n):
    """Group m's coset bit is bit m of the vector's little-endian coset field
    (byte m // 8, bit m % 8), checked one group at a time."""
    groups = n // 8
    nbytes = (groups + 7) // 8
    for m in range(groups):
        c = np.zeros((1, groups), np.uint8)
        c[0, m] = 1
        plane = oc.pack_cosets(c, nbytes)[0]
        assert plane.shape == (nbytes,)
        assert int.from_bytes(plane.tobytes(), "little") == 1 << m
    # quantize puts the coset of the group at coordinates 8m .. 8m+7 there:
    # x = H u / n (exact for these dyadic u) with a scale per 8-group; group m
    # of u is (2, 1/2, ..., 1/2) -> y = u -> half coset (squared distance
    # 1/4 against 11/4), every other group (2, 1/8, 0, ..., 0) -> integer
    # coset (5/8 against 15/8)
    cfg = oc.Codec(n, 2, 8)
    H = transform.hadamard_dense(n)
    for m in range(groups):
        u = np.zeros(n)
        u[0::8] = 2.0
        u[1::8] = 0.125
        u[8 * m + 1:8 * m + 8] = 0.5
        x = (H @ u / n)[None]
        q = oc.quantize(x, cfg)
        assert list(np.nonzero(q["c"][0])[0]) == [m]
        assert int.from_bytes(q["cosets"][0].tobytes(), "little") == 1 << m


def _exact_y_fp16(x16, L, G):
    """y of fp16 vectors without RoPE by exact integer arithmetic: u * 2^24 =
    H (x * 2^24) in Python integers, y = (L/2) u / a as an exact fraction,
    rounded once to fp64 by float()."""
    from fractions import Fraction
    n = x16.shape[-1]
    H = transform.hadamard_dense(n).astype(np.int64)
    xi = [int(v) for v in (x16.astype(np.float64) * 2.0 ** 24).astype(np.int64)]
    u = [sum(int(H[j, k]) * xi[k] for k in range(n)) for j in range(n)]
    out = []
    for g in range(n // G):
        grp = u[g * G:(g + 1) * G]
        a = max(Fraction(max(abs(v) for v in grp)), Fraction(1e-8 * math.sqrt(n)) * 2 ** 24)
        out += [float(Fraction(L, 2) * v / a) for v in grp]
    return np.array(out)


@pytest.mark.parametrize("n,bits,G", [(128, 2, 0), (64, 3, 32), (8, 2, 8)])
def test_y_is_the_exact_value_rounded_once(n, bits, G):
    """For fp16 inputs without RoPE the oracle's fp64 y equals the exact
    rational (L/2) u / a rounded once (u = H x exact), element for element.
    Pins the transform (a transposed or dropped term), the group maximum and
    the scale step of compute_y."""
    cfg = oc.Codec(n, bits, G)
    rng = np.random.default_rng(n + bits)
    x = rng.normal(size=(6, n)).astype(np.float16)
    x[1] = 0
    x[2, :] = 0
    x[2, 3] = np.float16(6e-8)      # fp16 subnormal: below the 1e-8 floor
    x[3] *= np.float16(1e-3)
    y, a = oc.compute_y(x, cfg)
    for r in range(x.shape[0]):
        assert np.array_equal(y[r], _exact_y_fp16(x[r], cfg.L, cfg.G)), r
    # the group maximum sits at +-L/2 exactly (nonzero groups)
    yg = np.abs(y[[0, 3, 4, 5]]).reshape(4, -1, cfg.G).max(-1)
    assert np.all(yg == cfg.L / 2)


def test_rope_key_y_against_dense_fp64():
    """Keys: y from an independent dense computation (rotation matrix of the
    inverse RoPE, dense Sylvester matrix) agrees with compute_y to fp64
    rounding."""
    d, theta = 96, 1e4
    cfg = oc.Codec(d, 2, 32, rope_theta=theta)
    x = _x((1, 1, 20, d), 31).astype(np.float64)
    pos = np.arange(20) + 1000
    y, _ = oc.compute_y(x, cfg, positions=pos, is_key=True)
    Hd = transform.hadamard_dense(128)
    h = d // 2
    for t in range(20):
        R = np.zeros((d, d))
        for i in range(h):
            ang = pos[t] * theta ** (-2.0 * i / d)
            c, s = math.cos(ang), math.sin(ang)
            R[i, i], R[i, i + h] = c, s           # x'_i = x_i c + x_{i+h} s
            R[i + h, i + h], R[i + h, i] = c, -s  # x'_{i+h} = x_{i+h} c - x_i s
        v = np.zeros(128)
        v[:d] = R @ x[0, 0, t]
        u = Hd @ v
        ref = np.concatenate([u[g * 32:(g + 1) * 32] * 2 / np.abs(u[g * 32:(g + 1) * 32]).max()
                              for g in range(4)])
        np.testing.assert_allclose(y[0, 0, t], ref, rtol=0, atol=1e-13)
