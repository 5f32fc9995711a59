"""Rotations of the head vector: RoPE removal / re-application and Hadamard.

Sources
-------
* nexusquant-kv 0.5.1 README, "How it works", steps 3-4: undo the rotary
  embedding on keys, then a Hadamard rotation; non-power-of-2 head dims are
  zero-padded.  The README's "Supported models" names split-half RoPE
  (Llama / Mistral / Qwen / Phi), i.e. coordinate i pairs with i + d/2.
* NexusQuant blog, post "The E8 lattice quantizes 8 numbers at once",
  "Handling outliers": the head vector is multiplied by the transpose of a
  128 x 128 Hadamard matrix, an orthogonal rotation.  We take the Sylvester
  matrix H[j][k] = (-1)^popcount(j & k), which is symmetric, so the product
  with its transpose is H v; the orthonormal rotation is H / sqrt(n).
* RoPE frequencies omega_i = theta^(-2i/d), the form HF models use with
  ``rope_theta`` from the config (README "API reference", ``rope_base``).
* Frequency scaling: README "API reference" lets the caller hand over the
  model config's ``rope_scaling`` dict, for Llama-3.1-style models; README
  "Limitations" names linear scaling and Llama-3.1 beyond its original
  context.  The pages print no formula; we take the published
  definitions of the two HF types that phrase points at: "linear" divides
  every frequency by the factor; "llama3" keeps the high-frequency band
  (wavelength below C / high_freq_factor), divides the low-frequency band
  (wavelength above C / low_freq_factor) by the factor and interpolates
  linearly in C / wavelength between them (C = original context length).

fp64 functions define every value the codec computes, the decision input y
included.  The fp32 functions (``rope_table_f32``, ``rope_inverse_f32``,
``fwht_f32``) are diagnostics: each operation is one IEEE fp32 operation in a
stated order (products and sums rounded separately, FWHT stages in the order
h = 1, 2, 4, ..., n/2), and tests use them to bound the error of an fp32
computation against the fp64 one.

Parity status: pinned (H H^T = nI, fast transform equals the dense product,
norm preservation, inverse-after-forward RoPE is the identity, position 0 is
the identity, the rotation direction by a hand-computed value (e_0 at
position 1 becomes cos(1) e_0 + sin(1) e_{d/2}); scaling: factor 1 is the identity, linear scaling equals
unscaled RoPE at position p / factor, llama3 frequencies lie between w/f and
w, fall monotonically, keep / divide the outer bands and are continuous at
the band edges) -- see tests/test_oracle_transform.py.
"""

from __future__ import annotations

import math
from dataclasses import dataclass

import numpy as np

__all__ = [
    "RopeScaling",
    "scale_freqs",
    "next_pow2",
    "rope_freqs",
    "rope_angles",
    "rope_table_f32",
    "rope_inverse_f32",
    "rope_forward_f64",
    "rope_inverse_f64",
    "hadamard_dense",
    "fwht_f32",
    "fwht_f64",
]


def next_pow2(d: int) -> int:
    n = 8
    while n < d:
        n *= 2
    return n


@dataclass(frozen=True)
class RopeScaling:
    """A model config's rope_scaling: kind "linear" or "llama3"."""
    kind: str
    factor: float
    low_freq_factor: float = 1.0
    high_freq_factor: float = 4.0
    original_max: int = 8192


def scale_freqs(omega, scaling: RopeScaling | None) -> np.ndarray:
    """Scaled frequencies, one fp64 operation at a time in the written order.

    linear: w / f.  llama3, with wavelength l = 2 pi / w and C the original
    context: w if l < C / high; w / f if l > C / low; otherwise
    (1 - a) w / f + a w with a = (C / l - low) / (high - low)."""
    omega = np.asarray(omega, dtype=np.float64)
    if scaling is None:
        return omega.copy()
    f = float(scaling.factor)
    if scaling.kind == "linear":
        return np.array([w / f for w in omega.tolist()])
    assert scaling.kind == "llama3", scaling.kind
    C = float(scaling.original_max)
    lo, hi = float(scaling.low_freq_factor), float(scaling.high_freq_factor)
    out = []
    for w in omega.tolist():
        wavelen = 2.0 * math.pi / w
        if wavelen < C / hi:
            out.append(w)
        elif wavelen > C / lo:
            out.append(w / f)
        else:
            a = (C / wavelen - lo) / (hi - lo)
            out.append((1.0 - a) * w / f + a * w)
    return np.array(out, dtype=np.float64)


def rope_freqs(theta: float, d: int, scaling: RopeScaling | None = None) -> np.ndarray:
    """omega_i = theta ** (-(2 i) / d), i in [0, d/2), each by C pow(), then
    the frequency scaling."""
    w = np.array([math.pow(theta, -(2.0 * i) / d) for i in range(d // 2)],
                 dtype=np.float64)
    return scale_freqs(w, scaling)


def rope_angles(positions, theta: float, d: int, scaling=None) -> np.ndarray:
    """[T, d/2] fp64 angles position * omega_i (one rounded product each)."""
    pos = np.asarray(positions, dtype=np.float64).reshape(-1, 1)
    return pos * rope_freqs(theta, d, scaling)[None, :]


def rope_table_f32(positions, theta: float, d: int, scaling=None):
    """cos and sin of the fp64 angles, each rounded once to fp32."""
    a = rope_angles(positions, theta, d, scaling)
    return np.cos(a).astype(np.float32), np.sin(a).astype(np.float32)


def rope_inverse_f32(x32: np.ndarray, cos32: np.ndarray, sin32: np.ndarray):
    """Remove split-half RoPE in fp32.  x32: [..., T, d]; tables [T, d/2].

    x'_i     = x_i c_i + x_{i+h} s_i
    x'_{i+h} = x_{i+h} c_i - x_i s_i          (h = d/2)
    Each product and each sum is rounded to fp32 separately.
    """
    x32 = np.asarray(x32, dtype=np.float32)
    h = x32.shape[-1] // 2
    lo, hi = x32[..., :h], x32[..., h:]
    out = np.empty_like(x32)
    out[..., :h] = (lo * cos32) + (hi * sin32)
    out[..., h:] = (hi * cos32) - (lo * sin32)
    return out


def rope_forward_f64(x: np.ndarray, positions, theta: float, scaling=None):
    """Apply split-half RoPE in fp64: y_i = x_i c - x_{i+h} s,
    y_{i+h} = x_{i+h} c + x_i s."""
    x = np.asarray(x, dtype=np.float64)
    d = x.shape[-1]
    a = rope_angles(positions, theta, d, scaling)
    c, s = np.cos(a), np.sin(a)
    h = d // 2
    lo, hi = x[..., :h], x[..., h:]
    return np.concatenate([lo * c - hi * s, hi * c + lo * s], axis=-1)


def rope_inverse_f64(x: np.ndarray, positions, theta: float, scaling=None):
    x = np.asarray(x, dtype=np.float64)
    d = x.shape[-1]
    a = rope_angles(positions, theta, d, scaling)
    c, s = np.cos(a), np.sin(a)
    h = d // 2
    lo, hi = x[..., :h], x[..., h:]
    return np.concatenate([lo * c + hi * s, hi * c - lo * s], axis=-1)


def hadamard_dense(n: int) -> np.ndarray:
    """Sylvester Hadamard matrix, H[j][k] = (-1)^popcount(j & k), fp64."""
    j = np.arange(n)
    bits = np.bitwise_and(j[:, None], j[None, :])
    pc = np.zeros_like(bits)
    while np.any(bits):
        pc += bits & 1
        bits = bits >> 1
    return np.where(pc % 2 == 0, 1.0, -1.0)


def _fwht(v: np.ndarray, dtype) -> np.ndarray:
    v = np.array(v, dtype=dtype, copy=True)
    n = v.shape[-1]
    h = 1
    while h < n:
        w = v.reshape(v.shape[:-1] + (n // (2 * h), 2, h))
        a = w[..., 0, :].copy()
        b = w[..., 1, :].copy()
        w[..., 0, :] = a + b
        w[..., 1, :] = a - b
        v = w.reshape(v.shape)
        h *= 2
    return v


def fwht_f32(v: np.ndarray) -> np.ndarray:
    """Unnormalised Walsh-Hadamard transform H v in fp32, stages h = 1..n/2.

    Stage h pairs coordinates j and j + h (bit h of j clear) and writes
    (a + b, a - b); every sum is one fp32 rounding.
    """
    return _fwht(v, np.float32)


def fwht_f64(v: np.ndarray) -> np.ndarray:
    return _fwht(v, np.float64)
