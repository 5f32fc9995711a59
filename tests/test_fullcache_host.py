"""The whole-cache checker (tests/fullcache.py) on the CPU: the oracle's own
planes give no exemptions; a planted one-step code change is counted, with
its regret; a changed scale is flagged (no GPU)."""

import uuid
from multiprocessing import shared_memory

import numpy as np

import fullcache
from oracle import codec as oc


def _shm(a, keep):
    shm = shared_memory.SharedMemory(create=True, size=max(a.nbytes, 1),
                                     name=f"nqt_{uuid.uuid4().hex[:12]}")
    keep.append(shm)
    np.ndarray(a.shape, a.dtype, buffer=shm.buf)[...] = a
    return (shm.name, a.shape, a.dtype.str)


def test_checker_counts_planted_changes():
    rng = np.random.default_rng(0)
    S, H, T, d = 2, 2, 50, 128
    x = (rng.normal(size=(S, H, T, d)) * np.where(rng.random(d) < 0.03, 8, 1)).astype(np.float16)
    codec = oc.Codec(d, 2, 0, strict=False, rope_theta=5e5)
    kw = dict(head_dim=d, bits=2, scale_group=0, strict=False, rope_theta=5e5, compact=False)
    ref = oc.quantize(x, codec, is_key=True)
    codes = ref["codes"].copy()
    keep = []
    try:
        specs = {"x": _shm(x, keep), "codes": _shm(codes, keep),
                 "cosets": _shm(ref["cosets"], keep), "scales": _shm(ref["scales"], keep)}
        jobs = [(specs, kw, True, s, h, h + 1) for s in range(S) for h in range(H)]
        res = [fullcache.check_chunk(j) for j in jobs]
        assert sum(r["groups"] for r in res) == S * H * T * 16
        assert sum(r["exempt"] + r["scale_steps"] for r in res) == 0
        # plant: coordinate 0 of vector (1, 0, 7) moves one code step; the
        # group is still counted as exempt, with a regret far above 1e-6
        c2 = codes.copy()
        i0 = int(c2[1, 0, 7, 0]) & 3
        c2[1, 0, 7, 0] = (int(c2[1, 0, 7, 0]) & 0xFC) | (i0 ^ 1)
        specs2 = dict(specs, codes=_shm(c2, keep))
        r = fullcache.check_chunk((specs2, kw, True, 1, 0, 1))
        assert r["exempt"] == 1 and r["bad_regret"] == 1 and r["max_regret"] > 1e-3
        # plant: a scale two fp16 steps away
        sc = ref["scales"].copy()
        sc.view(np.uint16)[0, 1, 3, 0] += 2
        specs3 = dict(specs, scales=_shm(sc, keep))
        r = fullcache.check_chunk((specs3, kw, True, 0, 1, 2))
        assert r["scale_steps"] == 1 and r["scale_bad"] == 1
    finally:
        for shm in keep:
            shm.close()
            shm.unlink()
