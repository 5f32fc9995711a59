"""E8 nearest-point decoding, written from the pages' definitions (oracle side).

Sources
-------
* NexusQuant blog, E8 walkthrough post, "The E8 Lattice, Briefly": E8 is the
  set of 8-vectors whose coordinates are all integers with even sum, or all
  half-integers.  The page says the half-integer sum may be odd; textbook E8
  (and the page's own "strict" variant, "The Relaxed Parity Discovery" in the
  same post and in the post "What Makes E8 Special") requires it even.
  ``strict=True`` is textbook E8 = D8 u (D8 + 1/2); ``strict=False`` is the
  relaxed set D8 u (Z^8 + 1/2).
* Same post, "The Conway-Sloane Nearest-Point Algorithm": round to each coset;
  when the parity is wrong, move the coordinate that was rounded worst by one
  step toward the input; keep the closer of the two coset candidates.  (The
  printed listing picks the *best*-rounded coordinate; the prose, and the
  exactness of the result, need the worst-rounded one.  This module follows
  the prose; the brute-force pins in ``tests/test_oracle_lattice.py`` fail for
  the other choice.)
* Same post, "Python Implementation": the quantizer clamps the lattice point
  to the range the code can hold.  The codec here restricts the decoder to
  the cube codebook  C(L) = lattice n [-(L-1)/2, (L-1)/2]^8  (integer coset:
  p in [-(L/2-1), L/2-1]; half coset: p in [-(L-1)/2, (L-1)/2]), i.e. every
  codeword whose coordinates fit in log2(L) bits, and returns the exact
  nearest codeword of that finite set.

Tie rules (several nearest points exist only on measure-zero sets; these make
the result unique and sign-symmetric, Q(-y) = -Q(y)):
  T1  per-coordinate rounding to a coset: ties go away from zero (for y = +-0
      the sign bit decides the half-integer choice +-1/2);
  T2  parity step direction when the rounding error is exactly 0: away from
      zero (sign bit of y);
  T3  parity step coordinate: lowest index among equal costs;
  T4  coset choice: the integer coset on equal distance.

Parity status: pinned (240 minimal vectors, shell counts of the radius-3
ball, brute force over the ball and over the whole cube codebook, covering
bound, hand-worked example) -- see tests/test_oracle_lattice.py.
"""

from __future__ import annotations

import math
from fractions import Fraction

import numpy as np

__all__ = [
    "decode",
    "decode_unconstrained",
    "codeword_points",
    "enumerate_cube_codebook",
    "enumerate_ball",
    "brute_force_nearest",
    "in_lattice",
]


def _round_to_coset(y: np.ndarray, c: int) -> np.ndarray:
    """Nearest integer (c=0) or half-integer (c=1) to each coordinate, T1 ties.

    Exact for any fp64 input: with f = floor(|y|), |y| - f is exact (f = 0,
    or f and |y| within a factor of two of each other), so the comparison
    with 1/2 is exact; the nearest half-integer is always f + 1/2.
    """
    a = np.abs(y)
    f = np.floor(a)
    if c == 0:
        m = f + (a - f >= 0.5)
    else:
        m = f + 0.5
    return np.copysign(m, y)


def _exact_sqdist(y_row, p_row) -> Fraction:
    return sum((Fraction(float(a)) - Fraction(float(b))) ** 2
               for a, b in zip(y_row, p_row))


def _coset_candidate(y: np.ndarray, c: int, pmax: float | None, parity: bool):
    """Nearest point of one coset (optionally limited to |p| <= pmax).

    Returns (p, d, fragile): p the candidate, d its fp64 squared distance,
    and a mask of rows whose parity step compared two costs closer than
    1e-12 (|delta| can round for half-integer candidates of tiny |y|); those
    rows are recomputed exactly by the caller.
    """
    p = _round_to_coset(y, c)
    if pmax is not None:
        p = np.clip(p, -pmax, pmax)
    fragile = np.zeros(y.shape[0], dtype=bool)
    if parity:
        # sum p is an integer on both cosets (8 half-integers sum to an integer)
        s = np.sum(p, axis=-1)
        odd = np.mod(s, 2.0) != 0.0
        if np.any(odd):
            yo, po = y[odd], p[odd]
            delta = yo - po
            # T2: toward y; when delta == 0, away from zero (sign bit of y)
            t = np.where(delta != 0.0, np.sign(delta), np.copysign(1.0, yo))
            toward = po + t
            if pmax is None:
                ok = np.ones_like(toward, dtype=bool)
            else:
                ok = np.abs(toward) <= pmax
            alt = np.where(ok, toward, po - t)
            # extra cost of moving coordinate i is 1 - 2|delta_i| toward y and
            # 1 + 2|delta_i| away from it, so minimising it maximises kappa:
            kappa = np.where(ok, np.abs(delta), -np.abs(delta))
            i_star = np.argmax(kappa, axis=-1)  # first index on ties (T3)
            rows = np.arange(po.shape[0])
            top = np.sort(kappa, axis=-1)
            near = (top[:, -1] - top[:, -2]) <= 1e-12
            fragile[np.nonzero(odd)[0][near]] = True
            po = po.copy()
            po[rows, i_star] = alt[rows, i_star]
            p = p.copy()
            p[odd] = po
    d = np.sum((y - p) ** 2, axis=-1)
    return p, d, fragile


def _exact_candidate(ys, neg, c: int, pmax, parity: bool):
    """One coset's candidate for one row in exact rational arithmetic (the
    same steps as _coset_candidate); ys exact values, neg their sign bits."""
    p = []
    for v, n in zip(ys, neg):
        a = abs(v)
        f = Fraction(math.floor(a))
        m = f + (1 if a - f >= Fraction(1, 2) else 0) if c == 0 else f + Fraction(1, 2)
        if pmax is not None:
            m = min(m, Fraction(pmax))
        p.append(-m if n else m)
    if parity and sum(p) % 2 != 0:
        best, i_best, alt_best = None, -1, None
        for i, (v, q, n) in enumerate(zip(ys, p, neg)):
            delta = v - q
            t = (1 if delta > 0 else -1) if delta != 0 else (-1 if n else 1)
            toward = q + t
            ok = pmax is None or abs(toward) <= Fraction(pmax)
            kappa = abs(delta) if ok else -abs(delta)
            if best is None or kappa > best:
                best, i_best, alt_best = kappa, i, (toward if ok else q - t)
        p[i_best] = alt_best
    d = sum((v - q) ** 2 for v, q in zip(ys, p))
    return p, d


def _decode_row_exact(ys, neg, L, strict: bool):
    """Exact (rational) two-coset decode of one row: (p as floats, c)."""
    pm0 = None if L is None else L / 2 - 1
    pm1 = None if L is None else (L - 1) / 2
    p0, d0 = _exact_candidate(ys, neg, 0, pm0, True)
    p1, d1 = _exact_candidate(ys, neg, 1, pm1, strict)
    if d1 < d0:
        return np.array([float(v) for v in p1]), 1
    return np.array([float(v) for v in p0]), 0


def _choose(p0, d0, p1, d1):
    """T4 coset choice in fp64; rows whose two distances lie within 1e-9
    (relative) of each other are returned for an exact re-decision."""
    pick1 = d1 < d0
    near = np.abs(d1 - d0) <= 1e-9 * np.maximum(1.0, np.maximum(d0, d1))
    p = np.where(pick1[:, None], p1, p0)
    return p, pick1.astype(np.uint8), near


def _near_boundary(y, L):
    """Rows with a coordinate within 1e-12 of a rounding boundary of either
    coset: a half-integer below L/2 - 1/2 for the integer coset, a nonzero
    integer below L/2 for the half coset (past those the cube clamps the
    rounding; at 0 the sign bit decides, and it is exact)."""
    a = np.abs(y)
    top0 = np.inf if L is None else L / 2 - 0.5
    top1 = np.inf if L is None else L / 2
    h = np.floor(a) + 0.5                      # nearest half-integer boundary below a + 1/2
    h = np.where(a - (h - 1) < h - a, h - 1, h)
    near0 = (np.abs(a - h) <= 1e-12) & (h < top0)
    k = np.round(a)                            # nearest integer
    near1 = (np.abs(a - k) <= 1e-12) & (k >= 1) & (k < top1)
    return np.any(near0 | near1, axis=-1)


def _decode(y, L, strict: bool, exact=None):
    """Shared body of decode / decode_unconstrained (L None: no cube).

    exact: None, or (num, den) arrays [N, 8] with y = num / den exactly; rows
    where fp64 cannot settle a decision are then decided on num / den instead
    of on the fp64 y."""
    pm0 = None if L is None else L / 2 - 1
    pm1 = None if L is None else (L - 1) / 2
    p0, d0, f0 = _coset_candidate(y, 0, pm0, True)
    p1, d1, f1 = _coset_candidate(y, 1, pm1, strict)
    p, c, near = _choose(p0, d0, p1, d1)
    redo = f0 | f1 | near
    if exact is not None:
        redo |= _near_boundary(y, L)
    for r in np.nonzero(redo)[0]:
        if exact is None:
            ys = [Fraction(float(v)) for v in y[r]]
        else:
            ys = [Fraction(float(nu)) / Fraction(float(de))
                  for nu, de in zip(exact[0][r], exact[1][r])]
        neg = [math.copysign(1.0, float(v)) < 0 for v in y[r]]
        p[r], c[r] = _decode_row_exact(ys, neg, L, strict)
    return p, c


def decode(y, L: int, strict: bool, exact=None):
    """Exact nearest codeword of the cube codebook C(L) for each 8-group.

    Parameters
    ----------
    y : array [N, 8] of fp64 (or narrower floats, widened exactly); the
        decision is exact for the value held: fp64 comparisons, and exact
        rational arithmetic wherever two compared costs lie within 1e-12
        (parity step) or 1e-9 relative (coset choice) of each other
    L : levels, 2**bits (4 for 2-bit, 8 for 3-bit)
    strict : textbook E8 parity on the half-integer coset too
    exact : optional (num, den), arrays [N, 8] of fp64 with y = num / den
        exactly (y itself then being that quotient rounded to fp64): rows
        where a decision is not settled in fp64 -- the costs above, or a
        coordinate within 1e-12 of a rounding boundary -- are decided on the
        exact quotient

    Returns
    -------
    idx : uint8 [N, 8], the per-coordinate code, idx = p + L/2 - c/2 in [0, L-1]
    c : uint8 [N], 1 for the half-integer coset
    p : float64 [N, 8], the codeword
    """
    y = np.asarray(y).astype(np.float64).reshape(-1, 8)
    if exact is not None:
        exact = (np.asarray(exact[0], np.float64).reshape(-1, 8),
                 np.asarray(exact[1], np.float64).reshape(-1, 8))
    p, c = _decode(y, L, strict, exact)
    idx = p + (L / 2) - c[:, None] * 0.5
    assert np.all(idx == np.round(idx)) and idx.min() >= 0 and idx.max() <= L - 1
    return idx.astype(np.uint8), c, p


def decode_unconstrained(y, strict: bool):
    """Exact nearest point of the whole lattice (no cube limit).  fp64 input."""
    y = np.asarray(y, dtype=np.float64).reshape(-1, 8)
    p, _ = _decode(y, None, strict)
    return p


def codeword_points(idx, c, L: int) -> np.ndarray:
    """p = idx - L/2 + c/2, the inverse of the code map."""
    idx = np.asarray(idx, dtype=np.float64).reshape(-1, 8)
    c = np.asarray(c, dtype=np.float64).reshape(-1)
    return idx - L / 2 + 0.5 * c[:, None]


def in_lattice(p, strict: bool) -> np.ndarray:
    """Membership test for E8 (strict) or D8 u (Z^8 + 1/2) (relaxed)."""
    p = np.asarray(p, dtype=np.float64).reshape(-1, 8)
    two = 2.0 * p
    if not np.all(two == np.round(two)):
        return np.zeros(p.shape[0], dtype=bool)
    frac = np.mod(two, 2.0)  # 0 for integers, 1 for half-integers
    all_int = np.all(frac == 0.0, axis=-1)
    all_half = np.all(frac == 1.0, axis=-1)
    even = np.mod(np.sum(p, axis=-1), 2.0) == 0.0
    return (all_int & even) | (all_half & (even | (not strict)))


def enumerate_cube_codebook(L: int, strict: bool) -> np.ndarray:
    """Every point of C(L), by direct enumeration of both cosets."""
    out = []
    ints = np.arange(-(L // 2 - 1), L // 2, dtype=np.float64)
    halfs = np.arange(-(L - 1) / 2, (L - 1) / 2 + 1, dtype=np.float64)
    for vals, parity in ((ints, True), (halfs, strict)):
        g = np.stack(np.meshgrid(*([vals] * 8), indexing="ij"), -1).reshape(-1, 8)
        if parity:
            g = g[np.mod(g.sum(-1), 2.0) == 0.0]
        out.append(g)
    return np.concatenate(out)


def enumerate_ball(r2: float, strict: bool) -> np.ndarray:
    """All lattice points with squared norm <= r2, by exhaustive enumeration
    of the integer and half-integer coordinate grids (pruned by norm)."""
    rmax = int(np.floor(np.sqrt(r2)))
    out = []
    ints = np.arange(-rmax, rmax + 1, dtype=np.float64)
    halfs = np.array([h + 0.5 for h in range(-rmax - 1, rmax + 1)
                      if (h + 0.5) ** 2 <= r2])
    for vals, parity in ((ints, True), (halfs, strict)):
        g = np.zeros((1, 0))
        for _ in range(8):
            g = np.concatenate([np.repeat(g, len(vals), 0),
                                np.tile(vals, g.shape[0])[:, None]], 1)
            g = g[(g * g).sum(-1) <= r2]
        if parity:
            g = g[np.mod(g.sum(-1), 2.0) == 0.0]
        out.append(g)
    return np.concatenate(out)


def brute_force_nearest(y, points: np.ndarray, chunk: int = 256):
    """Minimum squared distance from each y to a point set, and its arg."""
    y = np.asarray(y, dtype=np.float64).reshape(-1, 8)
    best = np.empty(y.shape[0])
    arg = np.empty(y.shape[0], dtype=np.int64)
    for s in range(0, y.shape[0], chunk):
        yy = y[s:s + chunk]
        d = ((yy[:, None, :] - points[None, :, :]) ** 2).sum(-1)
        arg[s:s + chunk] = np.argmin(d, axis=1)
        best[s:s + chunk] = d[np.arange(yy.shape[0]), arg[s:s + chunk]]
    return best, arg
