"""The codec end to end: quantize + pack, dequantize, packed-key scoring.

Sources
-------
* NexusQuant blog, E8 walkthrough post, "Python Implementation" (the
  quantizer): pad to a multiple of 8, split into 8-groups, amax per scale
  group floored at 1e-8, scale = amax / (levels / 2), nearest lattice point
  of the scaled group, rescale.  levels = 4 / 8 / 16 for 2 / 3 / 4 bits.
* Same post, "Why Per-Group Scaling?": one fp16 scale per 8 values, or
  ``quantize_perhead`` with one scale per 128-d head vector (0.125 bit/dim);
  the scale group G is a parameter here.
* Same post, "Bit Rate Accounting": b bits per coordinate (24 bits per
  8-group at 3 bits) plus a 16-bit scale; we add one coset bit per 8-group so
  that both cosets fit in b bits per coordinate.
* nexusquant-kv 0.5.1 README, "How it works" steps 3-5 (RoPE removal on keys,
  zero-padded Hadamard, E8 per 8-float group, K3V2 asymmetric bits) and
  "Results" (scale_bpe = 16/128 at G = 128).
* Same post, "What Makes This Hard in Practice" item 3: the compressed form
  has to stay on the device and be unpacked on the fly -> dequantize.
* Compact strict packing (our reading of "Bit Rate Accounting", which counts
  exactly b bits per coordinate, together with "The Relaxed Parity
  Discovery", where strict E8 keeps an even coordinate sum on both cosets):
  a strict codeword has an even index sum (sum idx = sum p + 4L - 4c), so
  the low bit of idx_7 equals the parity of the low bits of idx_0..idx_6 and
  need not be stored; that bit position carries the coset bit instead.  A
  group then takes exactly 8b bits and there is no coset plane.
* Nedelkoski et al., "E8 Lattice Key Quantization for Low-Bit KV-Cache
  Compression", Abstract and Table 3: attention scores computed from the
  packed keys without dequantizing them.  The oracle scores by
  dequantize-then-dot in fp64 (the kernel's table form is algebraically the
  same number; the oracle does not use that algebra).

Definitions (one head vector x of d values, n = next power of two >= d),
every step in fp64 from the exact input values:
  K only, theta > 0:  x' = RoPE^-1(x)       (transform.rope_inverse_f64)
  v = (x', 0, ..., 0) in R^n;  u = H_n v     (transform.fwht_f64)
  per scale group g of G coordinates:
      a_g  = max(max_j |u_j|, 1e-8 * sqrt(n))   (1e-8 in orthonormal units,
             z = u / sqrt(n))
      y_j  = (L/2) u_j / a_g                    -> max |y| = L/2 exactly
      sigma_g = a_g / ((L/2) sqrt(n)), stored as fp16 (RNE)
  each 8-group of y -> lattice.decode (exact nearest codeword of the quotient
  y, settled in exact arithmetic where fp64 cannot) -> idx in [0, L-1]^8,
  coset bit c
  Dequantize: p = idx - L/2 + c/2;  z^ = s16 * p;  x^ = (H_n z^ / sqrt(n))[:d];
  keys then get RoPE back (the README's re-application after quantization).
  D0 denotes dequantization without the RoPE step (the codec frame).

Packed planes, row-major over [S][H][T] vectors:
  codes : n*b/8 bytes per vector; coordinate j occupies bits [j*b, j*b+b) of
          the vector's little-endian bit stream
  cosets: ceil(n/64) bytes per vector; bit m = coset of 8-group m
  scales: n/G fp16 per vector

Parity status: pinned (scale range, zero vector, pack/unpack round trip,
plane sizes, strict parity of every group, lattice-point round trips,
score = dot with an independent dequantization, attend = one-hot rows, the
codec-frame form and linearity; compact packing: a bijection on all 36,049
strict 2-bit codewords, exactly 8b bits per group, same reconstruction as
the standard planes) -- tests/test_oracle_codec.py.
"""

from __future__ import annotations

import math
from dataclasses import dataclass

import numpy as np

from . import lattice, transform

__all__ = ["Codec", "quantize", "dequantize", "score", "attend", "pack_codes",
           "unpack_codes", "pack_cosets", "unpack_cosets", "fold_cosets",
           "unfold_cosets", "fp16_kv_bytes"]


@dataclass(frozen=True)
class Codec:
    head_dim: int
    bits: int
    scale_group: int = 0      # 0 -> n (one scale per vector)
    strict: bool = False
    rope_theta: float = 0.0   # > 0: keys have RoPE removed before quantizing
    rope_scaling: transform.RopeScaling | None = None   # frequency scaling
    compact: bool = False     # strict only: coset bit in idx_7's low bit

    def __post_init__(self):
        if self.compact and not self.strict:
            raise ValueError("compact packing needs strict parity")

    @property
    def n(self) -> int:
        return transform.next_pow2(self.head_dim)

    @property
    def L(self) -> int:
        return 1 << self.bits

    @property
    def G(self) -> int:
        return self.n if self.scale_group == 0 else self.scale_group

    @property
    def code_bytes(self) -> int:
        return self.n * self.bits // 8

    @property
    def coset_bytes(self) -> int:
        return 0 if self.compact else (self.n // 8 + 7) // 8

    @property
    def n_scales(self) -> int:
        return self.n // self.G

    @property
    def vector_bytes(self) -> int:
        return self.code_bytes + self.coset_bytes + 2 * self.n_scales


def fp16_kv_bytes(layers: int, kv_heads: int, head_dim: int, tokens: int = 1):
    """2 (K and V) x layers x heads x head_dim x tokens x 2 bytes (fp16).

    NexusQuant blog, post on the KV cache formula, "The formula"."""
    return 2 * layers * kv_heads * head_dim * tokens * 2


def compute_y(x, codec: Codec, positions=None, is_key: bool = False, with_u: bool = False):
    """y [.., n] and group maxima a [.., n/G], both fp64: the decision input
    (with_u: also u [.., n]).

    Every step in fp64 from the exact input values (fp16 / fp32 widened
    exactly): split-half RoPE removal with cos / sin of the fp64 angles
    (keys, theta > 0), zero padding, u = H v (fast transform, each sum one
    fp64 rounding; exact for fp16 inputs without RoPE, whose partial sums
    fit in 53 bits), a = max(max |u|, 1e-8 sqrt(n)) per group (the page's
    1e-8 floor in orthonormal units).  The decision input is the quotient
    y = (L/2) u / a of those fp64 numbers; the array returned holds it
    rounded once to fp64 (the group maximum maps to L/2 exactly), and the
    decoder settles close calls on the exact quotient.
    """
    x64 = np.asarray(x).astype(np.float64)
    d = codec.head_dim
    assert x64.shape[-1] == d
    if is_key and codec.rope_theta > 0:
        T = x64.shape[-2]
        pos = np.arange(T) if positions is None else np.asarray(positions)
        x64 = transform.rope_inverse_f64(x64, pos, codec.rope_theta, codec.rope_scaling)
    n = codec.n
    v = np.zeros(x64.shape[:-1] + (n,), dtype=np.float64)
    v[..., :d] = x64
    u = transform.fwht_f64(v)
    G = codec.G
    ug = u.reshape(u.shape[:-1] + (n // G, G))
    a = np.maximum(np.max(np.abs(ug), axis=-1), 1e-8 * math.sqrt(n))
    y = ((codec.L / 2) * ug / a[..., None]).reshape(u.shape)
    if with_u:
        return y, a, u
    return y, a


def compute_y_f32_stage_order(x, codec: Codec, positions=None, is_key: bool = False):
    """DIAGNOSTIC ONLY (not the decision input): the fp32 y of a butterfly
    implementation that rounds every step to fp32 in a fixed order -- RoPE
    removal as two rounded products and a rounded sum with fp32 cos / sin,
    Walsh-Hadamard stages h = 1, 2, ..., n/2 each rounded once, r = fp32
    ((L/2) / a), y = fp32(u r).  Tests use it to bound how far an fp32
    computation of y lies from the fp64 one."""
    x32 = np.asarray(x).astype(np.float32)
    d = codec.head_dim
    if is_key and codec.rope_theta > 0:
        T = x32.shape[-2]
        pos = np.arange(T) if positions is None else np.asarray(positions)
        c32, s32 = transform.rope_table_f32(pos, codec.rope_theta, d, codec.rope_scaling)
        x32 = transform.rope_inverse_f32(x32, c32, s32)
    n = codec.n
    v = np.zeros(x32.shape[:-1] + (n,), dtype=np.float32)
    v[..., :d] = x32
    u = transform.fwht_f32(v)
    G = codec.G
    ug = u.reshape(u.shape[:-1] + (n // G, G))
    a = np.maximum(np.max(np.abs(ug), axis=-1), np.float32(1e-8 * math.sqrt(n)))
    r = np.float32(codec.L / 2) / a
    y = (ug * r[..., None]).reshape(u.shape)
    return y.astype(np.float32), a.astype(np.float32)


def scales_from_maxima(a, codec: Codec) -> np.ndarray:
    """sigma = a / ((L/2) sqrt(n)) (orthonormal units), rounded once to fp16."""
    k = 1.0 / ((codec.L / 2) * math.sqrt(codec.n))
    return (np.asarray(a, dtype=np.float64) * k).astype(np.float16)


def pack_codes(idx, bits: int) -> np.ndarray:
    """[.., n] codes in [0, 2^b) -> [.., n*b/8] bytes, little-endian stream."""
    idx = np.asarray(idx, dtype=np.uint8)
    sh = idx.shape
    bitarr = ((idx[..., None] >> np.arange(bits, dtype=np.uint8)) & 1).astype(np.uint8)
    bitarr = bitarr.reshape(sh[:-1] + (sh[-1] * bits,))
    return np.packbits(bitarr, axis=-1, bitorder="little")


def unpack_codes(codes, bits: int, n: int) -> np.ndarray:
    codes = np.asarray(codes, dtype=np.uint8)
    bitarr = np.unpackbits(codes, axis=-1, bitorder="little")[..., :n * bits]
    bitarr = bitarr.reshape(codes.shape[:-1] + (n, bits)).astype(np.uint8)
    return (bitarr << np.arange(bits, dtype=np.uint8)).sum(-1).astype(np.uint8)


def pack_cosets(c, nbytes: int) -> np.ndarray:
    c = np.asarray(c, dtype=np.uint8)
    if nbytes == 0:                       # compact packing: no coset plane
        return np.zeros(c.shape[:-1] + (0,), np.uint8)
    pad = nbytes * 8 - c.shape[-1]
    if pad:
        c = np.concatenate([c, np.zeros(c.shape[:-1] + (pad,), np.uint8)], -1)
    return np.packbits(c, axis=-1, bitorder="little")


def unpack_cosets(cs, groups: int) -> np.ndarray:
    return np.unpackbits(np.asarray(cs, np.uint8), axis=-1,
                         bitorder="little")[..., :groups]


def fold_cosets(idx, c) -> np.ndarray:
    """Compact form of strict codewords: idx [.., 8] with an even sum, c [..]
    -> idx with the low bit of idx_7 replaced by c."""
    idx = np.array(idx, dtype=np.uint8, copy=True)
    idx[..., 7] = (idx[..., 7] & 0xFE) | (np.asarray(c, dtype=np.uint8) & 1)
    return idx


def unfold_cosets(idx_c):
    """Inverse of fold_cosets: c is the stored bit; the low bit of idx_7 is
    the parity of idx_0 .. idx_6 (the index sum is even)."""
    idx = np.array(idx_c, dtype=np.uint8, copy=True)
    c = (idx[..., 7] & 1).astype(np.uint8)
    low = (idx[..., :7].astype(np.int64).sum(-1) & 1).astype(np.uint8)
    idx[..., 7] = (idx[..., 7] & 0xFE) | low
    return idx, c


def quantize(x, codec: Codec, positions=None, is_key: bool = False):
    """Quantize vectors x [.., d] -> dict of planes plus the decision data."""
    y, a, u = compute_y(x, codec, positions, is_key, with_u=True)
    lead = y.shape[:-1]
    # exact quotient of every coordinate: (L/2) u (exact: L/2 is a power of
    # two) over its group's maximum
    den = np.repeat(a, codec.G, axis=-1)
    idx, c, _ = lattice.decode(y.reshape(-1, 8), codec.L, codec.strict,
                               exact=((codec.L / 2) * u, den))
    ng = codec.n // 8
    stored = fold_cosets(idx, c) if codec.compact else idx
    idx = idx.reshape(lead + (codec.n,))
    c = c.reshape(lead + (ng,))
    return {
        "codes": pack_codes(stored.reshape(lead + (codec.n,)), codec.bits),
        "cosets": pack_cosets(c, codec.coset_bytes),
        "scales": scales_from_maxima(a, codec),
        "idx": idx, "c": c, "y": y, "a": a,
    }


def dequantize(codes, cosets, scales, codec: Codec, positions=None,
               is_key: bool = False, apply_rope: bool = True) -> np.ndarray:
    """fp64 reconstruction [.., d] of packed vectors."""
    n, d, G = codec.n, codec.head_dim, codec.G
    if codec.compact:
        u = unpack_codes(codes, codec.bits, n)
        idx8, c8 = unfold_cosets(u.reshape(u.shape[:-1] + (n // 8, 8)))
        idx = idx8.reshape(u.shape).astype(np.float64)
        c = c8.astype(np.float64)
    else:
        idx = unpack_codes(codes, codec.bits, n).astype(np.float64)
        c = unpack_cosets(cosets, n // 8).astype(np.float64)
    p = idx - codec.L / 2 + 0.5 * np.repeat(c, 8, axis=-1)
    s = np.repeat(np.asarray(scales, np.float16).astype(np.float64), G, axis=-1)
    z = s * p
    x = transform.fwht_f64(z)[..., :d] / math.sqrt(n)
    if is_key and apply_rope and codec.rope_theta > 0:
        T = x.shape[-2]
        pos = np.arange(T) if positions is None else np.asarray(positions)
        x = transform.rope_forward_f64(x, pos, codec.rope_theta, codec.rope_scaling)
    return x


def score(q, codes, cosets, scales, codec: Codec) -> np.ndarray:
    """S[s][h][t] = q[s][h] . D0(K)[s][h // (Hq/H)][t]   (fp64).

    q: [S, Hq, d]; planes: [S, H, T, .]."""
    q = np.asarray(q).astype(np.float64)
    k = dequantize(codes, cosets, scales, codec, apply_rope=False)  # [S,H,T,d]
    S, Hq, _ = q.shape
    H = k.shape[1]
    grp = Hq // H
    out = np.empty((S, Hq, k.shape[2]))
    for h in range(Hq):
        out[:, h, :] = np.einsum("sd,std->st", q[:, h, :], k[:, h // grp])
    return out


def attend(weights, codes, cosets, scales, codec: Codec) -> np.ndarray:
    """out[s][h] = sum_t weights[s][h][t] * D(V)[s][h // (Hq/H)][t]   (fp64).

    The value half of decode attention on the packed cache (the packed form
    is kept on the device and unpacked on the fly: NexusQuant blog, E8
    walkthrough post, "What Makes This Hard in Practice", item 3; scores from
    the same cache: Nedelkoski et al., Abstract).  Values carry no RoPE.
    weights: [S, Hq, T]; planes: [S, H, T, .] -> [S, Hq, d]."""
    w = np.asarray(weights, dtype=np.float64)
    v = dequantize(codes, cosets, scales, codec, is_key=False)    # [S,H,T,d]
    S, Hq, _ = w.shape
    H = v.shape[1]
    grp = Hq // H
    out = np.empty((S, Hq, v.shape[-1]))
    for h in range(Hq):
        out[:, h, :] = np.einsum("st,std->sd", w[:, h, :], v[:, h // grp])
    return out
