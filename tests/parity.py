"""Comparison helpers for GPU-vs-oracle parity tests.

Acceptance (codes): packed code and coset bytes equal per 8-group, except
groups where the GPU's codeword is a valid codeword whose squared distance to
the oracle's fp64 y exceeds the oracle's own by less than 1e-6 (y in lattice
units); such exempt groups must number at most 1e-6 of all groups, counted
over a pool (every check_codes call of the session adds its groups and its
exempt groups to POOL; tests/test_gpu_parity.py asserts the pooled budget
last, and the whole-cache tests assert it per cache).  Scales: equal bits,
or one fp16 step where the oracle's sigma lies within 1e-6 relative of an
fp16 rounding midpoint.  Dequantized vectors: |x_gpu - x_ref| <= 1e-3
|x_ref| per vector (plus 1e-6 absolute for near-zero vectors).  Scores: |S_gpu - S_ref| <= 1e-3 |q| |D0 k|.
"""

import math

import numpy as np

from oracle import codec as oc
from oracle import lattice, transform

REGRET_TOL = 1e-6
EXEMPT_FRAC = 1e-6

# groups checked and exempt groups found in this session
POOL = {"groups": 0, "exempt": 0, "cases": 0}


def pooled_budget_ok():
    return POOL["exempt"] <= math.floor(EXEMPT_FRAC * POOL["groups"])


def oracle_scaling(cfg):
    """The oracle's RopeScaling for an nq.Config (None when unscaled)."""
    if cfg.rope_scaling == 1:
        return transform.RopeScaling("linear", cfg.rope_factor)
    if cfg.rope_scaling == 2:
        return transform.RopeScaling("llama3", cfg.rope_factor, cfg.rope_low_freq_factor,
                                     cfg.rope_high_freq_factor, cfg.rope_original_max)
    return None


def oracle_codec(cfg, is_value: bool) -> oc.Codec:
    return oc.Codec(cfg.head_dim, cfg.bits_v if is_value else cfg.bits_k,
                    cfg.scale_group, cfg.parity == 0,
                    0.0 if is_value else cfg.rope_theta,
                    None if is_value else oracle_scaling(cfg),
                    compact=cfg.packing == 1)


def unpack_planes(codes, cosets, codec: oc.Codec):
    """(idx [groups, 8], c [groups]) of packed planes, either packing."""
    idx = oc.unpack_codes(codes.reshape(-1, codec.code_bytes), codec.bits, codec.n).reshape(-1, 8)
    if codec.compact:
        return oc.unfold_cosets(idx)
    return idx, oc.unpack_cosets(cosets.reshape(-1, codec.coset_bytes), codec.n // 8).reshape(-1)


def to_np(packed):
    return (packed.codes.cpu().numpy(), packed.cosets.cpu().numpy(),
            packed.scales.cpu().numpy())


def check_codes(codes, cosets, scales, ref, codec: oc.Codec, label=""):
    """Compare GPU planes (numpy, [..., bytes]) with oracle.quantize output."""
    n, L = codec.n, codec.L
    codes = codes.reshape(-1, codec.code_bytes)
    cosets = cosets.reshape(codes.shape[0], codec.coset_bytes)
    scales = scales.reshape(-1, codec.n_scales)
    rc = ref["codes"].reshape(-1, codec.code_bytes)
    rs = ref["cosets"].reshape(rc.shape[0], codec.coset_bytes)
    rsc = ref["scales"].reshape(-1, codec.n_scales)
    assert codes.shape == rc.shape, (label, codes.shape, rc.shape)
    # scales: equal bits (both sides round a * (1/((L/2) sqrt n)) once to
    # fp16), except one fp16 step where the oracle's a * k lies within 1e-6
    # relative of the midpoint of the two fp16 numbers: there the fp32 group
    # maximum of the kernels (a few fp32 ulps from the fp64 one) rounds it the
    # other way
    sg, sr = scales.view(np.uint16), rsc.view(np.uint16)
    bad_sc = np.nonzero(sg != sr)
    if len(bad_sc[0]):
        k = 1.0 / ((L / 2) * math.sqrt(n))
        a = np.asarray(ref["a"], np.float64).reshape(sr.shape)[bad_sc]
        g16, r16 = sg[bad_sc], sr[bad_sc]
        step = np.abs(g16.astype(np.int64) - r16.astype(np.int64)) == 1
        mid = (g16.view(np.float16).astype(np.float64) + r16.view(np.float16).astype(np.float64)) / 2
        near = np.abs(a * k - mid) <= 1e-6 * np.abs(a * k)
        assert (step & near).all(), \
            f"{label}: {int((~(step & near)).sum())} scale mismatches away from an fp16 midpoint"
    stats_sc = int(len(bad_sc[0]))
    idx_g, c_g = unpack_planes(codes, cosets, codec)
    idx_r = ref["idx"].reshape(-1, 8)
    c_r = ref["c"].reshape(-1)
    mism = np.any(idx_g != idx_r, axis=1) | (c_g != c_r)
    n_groups = idx_r.shape[0]
    n_bad = int(mism.sum())
    stats = {"groups": n_groups, "exempt": n_bad, "max_regret": 0.0, "scale_steps": stats_sc}
    if n_bad:
        y = ref["y"].reshape(-1, 8)[mism].astype(np.float64)
        pg = lattice.codeword_points(idx_g[mism], c_g[mism], L)
        pr = lattice.codeword_points(idx_r[mism], c_r[mism], L)
        valid = lattice.in_lattice(pg, codec.strict)
        regret = ((y - pg) ** 2).sum(-1) - ((y - pr) ** 2).sum(-1)
        stats["max_regret"] = float(regret.max())
        assert valid.all(), f"{label}: GPU emitted non-codewords"
        assert (regret < REGRET_TOL).all(), f"{label}: regret {regret.max()} in {n_bad} groups"
    POOL["groups"] += n_groups
    POOL["exempt"] += n_bad
    POOL["cases"] += 1
    if n_bad:
        print(f"[exempt] {label}: {n_bad} of {n_groups} groups, max regret "
              f"{stats['max_regret']:.3e}", flush=True)
    # every byte of groups that agree is equal (also the unused coset bits)
    vec_bad = mism.reshape(codes.shape[0], -1).any(axis=1)
    assert np.array_equal(codes[~vec_bad], rc[~vec_bad]), label
    assert np.array_equal(cosets[~vec_bad], rs[~vec_bad]), label
    return stats


def check_dequant(x_gpu, x_ref, label=""):
    x_gpu = np.asarray(x_gpu, dtype=np.float64).reshape(-1, x_ref.shape[-1])
    x_ref = np.asarray(x_ref, dtype=np.float64).reshape(x_gpu.shape)
    err = np.linalg.norm(x_gpu - x_ref, axis=1)
    lim = 1e-3 * np.linalg.norm(x_ref, axis=1) + 1e-6
    bad = np.nonzero(err > lim)[0]
    assert len(bad) == 0, f"{label}: {len(bad)} vectors off, worst rel {np.max(err / lim)}"
    return float(np.max(err / lim))


def check_scores(s_gpu, s_ref, qnorm, knorm, label=""):
    s_gpu = np.asarray(s_gpu, dtype=np.float64)
    lim = 1e-3 * qnorm * knorm + 1e-9
    err = np.abs(s_gpu - s_ref)
    bad = err > lim
    assert not bad.any(), f"{label}: {int(bad.sum())} scores off, worst {np.max(err / lim)}"
    return float(np.max(err / lim))
