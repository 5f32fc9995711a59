"""Whole-cache comparison of packed planes with the oracle, chunk by chunk in
worker processes (the CPU side of tests/test_gpu_exemptions.py).

The parent puts the input tensor and the three packed planes in shared
memory; each worker maps them, runs the oracle's quantize on a (slab, heads)
chunk from the exact input bytes, and counts: groups, groups whose code or
coset bit differs, the largest regret among those (fp64 squared distance to
the oracle's y of the device codeword minus that of the oracle's codeword),
non-codewords, scales that differ by more than one fp16 step or away from a
rounding midpoint.  Workers import numpy and the oracle only.
"""

import math
from multiprocessing import shared_memory

import numpy as np

from oracle import codec as oc
from oracle import lattice

_OPEN = {}


def _view(spec):
    name, shape, dtype = spec
    shm = _OPEN.get(name)
    if shm is None:
        shm = _OPEN[name] = shared_memory.SharedMemory(name=name)
    return np.ndarray(shape, dtype=np.dtype(dtype), buffer=shm.buf)


def check_chunk(job):
    specs, codec_kw, is_key, s, h0, h1 = job
    x = _view(specs["x"])[s, h0:h1]
    codes = _view(specs["codes"])[s, h0:h1]
    cosets = _view(specs["cosets"])[s, h0:h1]
    scales = _view(specs["scales"])[s, h0:h1]
    codec = oc.Codec(**codec_kw)
    L, n = codec.L, codec.n
    ref = oc.quantize(x, codec, is_key=is_key)
    out = {"groups": 0, "exempt": 0, "max_regret": 0.0, "bad_regret": 0, "invalid": 0,
           "scale_steps": 0, "scale_bad": 0}
    # scales
    sg = scales.reshape(-1, codec.n_scales).view(np.uint16)
    sr = ref["scales"].reshape(-1, codec.n_scales).view(np.uint16)
    bad = np.nonzero(sg != sr)
    if len(bad[0]):
        k = 1.0 / ((L / 2) * math.sqrt(n))
        a = ref["a"].reshape(sr.shape)[bad]
        g16, r16 = sg[bad], sr[bad]
        step = np.abs(g16.astype(np.int64) - r16.astype(np.int64)) == 1
        mid = (g16.view(np.float16).astype(np.float64) + r16.view(np.float16).astype(np.float64)) / 2
        near = np.abs(a * k - mid) <= 1e-6 * np.abs(a * k)
        out["scale_steps"] = int(len(bad[0]))
        out["scale_bad"] = int((~(step & near)).sum())
    # codes and coset bits per group
    idx_g = oc.unpack_codes(codes.reshape(-1, codec.code_bytes), codec.bits, n).reshape(-1, 8)
    if codec.compact:
        idx_g, c_g = oc.unfold_cosets(idx_g)
    else:
        c_g = oc.unpack_cosets(cosets.reshape(-1, codec.coset_bytes), n // 8).reshape(-1)
    idx_r = ref["idx"].reshape(-1, 8)
    c_r = ref["c"].reshape(-1)
    mism = np.any(idx_g != idx_r, axis=1) | (c_g != c_r)
    out["groups"] = int(idx_r.shape[0])
    out["exempt"] = int(mism.sum())
    if out["exempt"]:
        y = ref["y"].reshape(-1, 8)[mism]
        pg = lattice.codeword_points(idx_g[mism], c_g[mism], L)
        pr = lattice.codeword_points(idx_r[mism], c_r[mism], L)
        regret = ((y - pg) ** 2).sum(-1) - ((y - pr) ** 2).sum(-1)
        out["max_regret"] = float(regret.max())
        out["bad_regret"] = int((regret >= 1e-6).sum())
        out["invalid"] = int((~lattice.in_lattice(pg, codec.strict)).sum())
    return out
