"""Pins of the oracle's lattice decoder against facts fixed by the pages and
by the mathematics (no GPU).  See tests/golden/e8_facts.json for the cited
values."""

import json
import os

import numpy as np
import pytest

from oracle import lattice

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "e8_facts.json")))


@pytest.fixture(scope="module")
def ball():
    return {s: lattice.enumerate_ball(9.0, s) for s in (True, False)}


def _norm2(p):
    return (np.asarray(p) ** 2).sum(-1)


def test_minimal_vectors_count(ball):
    b = ball[True]
    assert int(np.sum(_norm2(b) == 2.0)) == GOLD["kissing_number"]["value"]
    # relaxed adds the odd-sum (+-1/2)^8 vectors
    half = ball[False][np.all(np.abs(ball[False]) == 0.5, axis=1)]
    assert len(half) == GOLD["half_integer_shell_points"]["relaxed"]
    half_s = ball[True][np.all(np.abs(ball[True]) == 0.5, axis=1)]
    assert len(half_s) == GOLD["half_integer_shell_points"]["strict"]


def test_theta_series_shells(ball):
    # E8 theta series 1 + 240 q + 2160 q^2 + 6720 q^3 + 17520 q^4 (textbook)
    vals, counts = np.unique(_norm2(ball[True]), return_counts=True)
    assert list(vals) == [0, 2, 4, 6, 8]
    assert list(counts) == [1, 240, 2160, 6720, 17520]
    assert np.all(lattice.in_lattice(ball[True], True))
    assert np.all(lattice.in_lattice(ball[False], False))


@pytest.mark.parametrize("strict", [True, False])
def test_minimal_vectors_decode_to_themselves(ball, strict):
    mv = ball[strict][_norm2(ball[strict]) == 2.0]
    assert np.array_equal(lattice.decode_unconstrained(mv, strict), mv)
    # every minimal vector lies in the 2-bit cube codebook as well
    idx, c, p = lattice.decode(mv.astype(np.float32), 4, strict)
    assert np.array_equal(p, mv)


@pytest.mark.parametrize("strict", [True, False])
def test_unconstrained_matches_brute_force_in_ball(ball, strict):
    rng = np.random.default_rng(1)
    y = rng.normal(size=(3000, 8))
    y *= (rng.uniform(0, 2.0, size=(3000, 1)) / np.linalg.norm(y, axis=1, keepdims=True))
    p = lattice.decode_unconstrained(y, strict)
    best, _ = lattice.brute_force_nearest(y, ball[strict], chunk=32)
    d = _norm2(y - p)
    assert np.all(lattice.in_lattice(p, strict))
    np.testing.assert_allclose(d, best, rtol=0, atol=1e-12)


def test_argmin_variant_would_fail_brute_force(ball):
    """The brute-force pin detects the best-rounded-coordinate variant."""
    y = np.array(GOLD["worked_example"]["y"], dtype=np.float64)[None]
    r = np.round(y)
    gaps = np.abs(y - r)
    i = int(np.argmin(np.where(gaps == 0, np.inf, gaps)))  # best-rounded nonzero gap
    alt = r.copy()
    alt[0, i] += np.sign(y[0, i] - r[0, i]) or 1.0
    best, _ = lattice.brute_force_nearest(y, ball[True])
    assert _norm2(y - alt)[0] > best[0] + 0.5


def test_worked_example():
    ex = GOLD["worked_example"]
    y = np.array(ex["y"], dtype=np.float32)[None]
    for strict in (True, False):
        p = lattice.decode_unconstrained(y.astype(np.float64), strict)
        assert np.array_equal(p[0], np.array(ex["nearest"], dtype=np.float64))
        np.testing.assert_allclose(_norm2(y.astype(np.float64) - p)[0], ex["sqdist"], rtol=1e-6)
        _, _, pc = lattice.decode(y, 4, strict)
        assert np.array_equal(pc[0], np.array(ex["nearest"], dtype=np.float64))


@pytest.mark.parametrize("strict", [True, False])
def test_covering_bound_and_structure(strict):
    rng = np.random.default_rng(2)
    y = rng.uniform(-6, 6, size=(20000, 8))
    p = lattice.decode_unconstrained(y, strict)
    assert np.all(lattice.in_lattice(p, strict))
    assert np.max(_norm2(y - p)) <= GOLD["covering_radius_squared"]["value"] + 1e-12
    hole = np.zeros((1, 8))
    hole[0, 0] = 1.0
    assert _norm2(hole - lattice.decode_unconstrained(hole, True))[0] == 1.0


@pytest.mark.parametrize("strict", [True, False])
def test_perturbation_inside_packing_radius(ball, strict):
    rng = np.random.default_rng(3)
    pts = ball[strict][rng.integers(0, len(ball[strict]), 4000)]
    e = rng.normal(size=pts.shape)
    # E8 packing radius 1/sqrt(2) (pages); the relaxed set holds half-integer
    # points at distance 1 from each other, so its packing radius is 1/2.
    rho = np.sqrt(GOLD["packing_radius_squared"]["value"]) if strict else 0.5
    r = rho * rng.uniform(0, 0.999, (len(pts), 1))
    e *= r / np.linalg.norm(e, axis=1, keepdims=True)
    assert np.array_equal(lattice.decode_unconstrained(pts + e, strict), pts)


@pytest.mark.parametrize("strict", [True, False])
def test_cube_decoder_brute_force_2bit(strict):
    cb = lattice.enumerate_cube_codebook(4, strict)
    assert len(cb) == (36049 if strict else 68817)
    rng = np.random.default_rng(4)
    y = rng.uniform(-2.0, 2.0, size=(1500, 8)).astype(np.float32)
    # scaled groups always have one coordinate at +-L/2
    y[np.arange(500), rng.integers(0, 8, 500)] = np.float32(2.0)
    idx, c, p = lattice.decode(y, 4, strict)
    best, _ = lattice.brute_force_nearest(y.astype(np.float64), cb, chunk=16)
    np.testing.assert_allclose(_norm2(y.astype(np.float64) - p), best, rtol=0, atol=1e-12)
    assert np.all(lattice.in_lattice(p, strict))
    assert np.all(np.abs(p) <= 1.5)
    assert np.array_equal(lattice.codeword_points(idx, c, 4), p)


@pytest.mark.parametrize("strict", [True, False])
def test_cube_decoder_local_brute_force_3bit(strict):
    """3-bit codebook (11-20 M points): check against every codeword of the
    cube whose coordinates are within 2 of y (the answer always is)."""
    rng = np.random.default_rng(5)
    y = rng.uniform(-4.0, 4.0, size=(150, 8)).astype(np.float32)
    idx, c, p = lattice.decode(y, 8, strict)
    ints = np.arange(-3, 4, dtype=np.float64)
    halfs = np.arange(-3.5, 4.0, 1.0)
    for r in range(len(y)):
        yy = y[r].astype(np.float64)
        best = np.inf
        for vals, par in ((ints, True), (halfs, strict)):
            opts = [vals[np.abs(vals - t) <= 2.0] for t in yy]
            g = np.stack(np.meshgrid(*opts, indexing="ij"), -1).reshape(-1, 8)
            if par:
                g = g[np.mod(g.sum(-1), 2.0) == 0.0]
            if len(g):
                best = min(best, _norm2(yy - g).min())
        assert abs(_norm2(yy - p[r]) - best) <= 1e-12
    assert np.all(idx <= 7)


def test_tie_rules():
    # T1+T4: zero vector -> origin, integer coset, idx = L/2
    idx, c, p = lattice.decode(np.zeros((1, 8), np.float32), 4, True)
    assert c[0] == 0 and np.all(idx == 2) and np.all(p == 0)
    # T3: equal parity-step costs at coordinates 1 and 2 -> the lower index moves
    y = np.array([[0.8, 0.3, -0.3, 0, 0, 0, 0, 0]], np.float32)
    idx, c, p = lattice.decode(y, 4, False)
    assert c[0] == 0 and list(p[0]) == [1, 1, 0, 0, 0, 0, 0, 0]
    # T1 on the half coset: y = +0 -> +1/2, y = -0 -> -1/2
    y = np.array([[1.5, 1.5, 1.5, 1.5, 0.0, -0.0, 0.4, -0.4]], np.float32)
    _, c, p = lattice.decode(y, 4, False)
    assert c[0] == 1 and list(p[0]) == [1.5, 1.5, 1.5, 1.5, 0.5, -0.5, 0.5, -0.5]


@pytest.mark.parametrize("strict", [True, False])
@pytest.mark.parametrize("L", [4, 8])
def test_sign_symmetry_and_parity(strict, L):
    rng = np.random.default_rng(6)
    y = rng.uniform(-L / 2, L / 2, size=(5000, 8)).astype(np.float32)
    y[::7] = np.round(y[::7] * 2) / 2  # many exact ties
    i1, c1, p1 = lattice.decode(y, L, strict)
    i2, c2, p2 = lattice.decode(-y, L, strict)
    assert np.array_equal(p1, -p2) and np.array_equal(c1, c2)
    if strict:
        assert np.all(i1.astype(int).sum(-1) % 2 == 0)
    else:
        assert np.all(i1[c1 == 0].astype(int).sum(-1) % 2 == 0)


def test_fp64_near_ties_round_the_right_way():
    """Decisions are exact for fp64 inputs just below a rounding boundary,
    where |y| + 1/2 would round up to the boundary in fp64."""
    below = np.nextafter(0.5, 0.0)                  # 0.5 - 2^-54
    for strict in (True, False):
        y = np.array([[below, below, 0, 0, 0, 0, 0, 0]])
        idx, c, p = lattice.decode(y, 4, strict)
        assert c[0] == 0 and np.all(p == 0), p          # origin, not (1, 1, 0, ...)
        assert np.all(lattice.decode_unconstrained(y, strict) == 0)
        y = -y
        _, _, p = lattice.decode(y, 4, strict)
        assert np.all(p == 0)
    # just below 3/2 on the integer coset rounds to 1, and just above 1/2
    # rounds to 1
    above = np.nextafter(0.5, 1.0)
    y = np.array([[np.nextafter(1.5, 0.0), above, 0, 0, 0, 0, 0, 0]])
    _, c, p = lattice.decode(y, 4, False)
    assert c[0] == 0 and list(p[0]) == [1, 1, 0, 0, 0, 0, 0, 0]


def test_tiny_half_coset_parity_step_is_exact():
    """Strict half coset with an odd index sum: the step moves the coordinate
    with the largest |delta| = 1/2 - |y|, i.e. the smallest |y|; in fp64 the
    two |delta| below round to the same number, the exact path separates
    them (coordinate 1 moves, not coordinate 0)."""
    y = np.array([[1e-20, 1e-30, 1.5, 1.5, 1.5, 1.5, 1.5, 1.5]])
    _, c, p = lattice.decode(y, 4, True)
    cb = lattice.enumerate_cube_codebook(4, True)
    from fractions import Fraction
    dist = [sum((Fraction(float(a)) - Fraction(float(b))) ** 2 for a, b in zip(y[0], q))
            for q in cb]
    best = min(dist)
    winners = [cb[i] for i, dd in enumerate(dist) if dd == best]
    assert len(winners) == 1 and np.array_equal(p[0], winners[0]), (p, winners)


@pytest.mark.parametrize("strict", [True, False])
def test_cube_decoder_fp64_brute_force(strict):
    """fp64 inputs (not fp32-representable) against brute force over the
    whole 2-bit codebook."""
    cb = lattice.enumerate_cube_codebook(4, strict)
    rng = np.random.default_rng(14)
    y = rng.uniform(-2.0, 2.0, size=(1000, 8))
    y[::5] = np.round(y[::5] * 2) / 2 + rng.choice([-1, 1], size=(200, 8)) * 2.0 ** -50
    y = np.clip(y, -2.0, 2.0)
    idx, c, p = lattice.decode(y, 4, strict)
    best, _ = lattice.brute_force_nearest(y, cb, chunk=16)
    np.testing.assert_allclose(_norm2(y - p), best, rtol=0, atol=1e-12)
    assert np.all(lattice.in_lattice(p, strict))


def _exact_min_codewords(yq, cb):
    """All codewords at the exact minimum squared distance from the rational
    vector yq (fp64 prefilter, then exact arithmetic on the close ones)."""
    from fractions import Fraction
    yf = np.array([float(v) for v in yq])
    d = ((cb - yf) ** 2).sum(-1)
    cand = cb[d <= d.min() + 1e-9]
    ex = [sum((v - Fraction(float(q))) ** 2 for v, q in zip(yq, row)) for row in cand]
    m = min(ex)
    return [cand[i] for i, e in enumerate(ex) if e == m], m


@pytest.mark.parametrize("strict", [True, False])
def test_decisions_on_the_exact_quotient(strict):
    """y = (L/2) u / a is decided as the exact quotient: on small-integer u
    with non-power-of-two a (exact ties are common there), rows whose fp64
    rounding of y would tip a tie come out as an exact nearest codeword of
    the quotient, and on exact distance ties the integer coset (tie rule T4);
    checked against exact brute force over the 2-bit codebook."""
    from fractions import Fraction
    rng = np.random.default_rng(21 + strict)
    u = rng.integers(-6, 7, size=(20000, 8)).astype(np.float64)
    a = np.abs(u).max(-1, keepdims=True)
    a[a == 0] = 1.0
    u[:, 0] = np.where(rng.random(20000) < 0.5, a[:, 0], -a[:, 0])
    num, den = 2.0 * u, np.repeat(a, 8, axis=1)
    y = num / den
    _, c1, p1 = lattice.decode(y, 4, strict)
    _, c2, p2 = lattice.decode(y, 4, strict, exact=(num, den))
    rows = np.nonzero(np.any(p1 != p2, axis=1))[0]
    assert len(rows) > 0
    cb = lattice.enumerate_cube_codebook(4, strict)
    for r in rows[:25]:
        yq = [Fraction(int(nu)) / Fraction(int(de)) for nu, de in zip(num[r], den[r])]
        winners, m = _exact_min_codewords(yq, cb)
        assert any(np.array_equal(p2[r], w) for w in winners), (y[r], p2[r], winners)
        d1 = sum((v - Fraction(float(q))) ** 2 for v, q in zip(yq, p1[r]))
        assert d1 >= m
        if d1 == m and c1[r] != c2[r]:      # a coset tie the fp64 rounding tipped: T4
            assert c2[r] == 0
        elif d1 == m:                         # a parity-step tie: T3, the lower index moves
            i = int(np.nonzero(p1[r] != p2[r])[0][0])
            yi = yq[i]
            rnd = lattice._round_to_coset(np.array([float(yi)]), int(c2[r]))[0]
            assert p2[r][i] != rnd and p1[r][i] == rnd
