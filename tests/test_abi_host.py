"""Host-side checks of libnq: it loads, exports every symbol include/nq.h
declares, and rejects bad arguments before touching the GPU (no GPU)."""

import ctypes
import os
import re

import pytest

from e8_lattice_vector_amd import nq

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared():
    src = open(os.path.join(ROOT, "include", "nq.h")).read()
    return sorted(set(re.findall(r"^\s*(?:int|size_t|const char\*)\s+(nq_\w+)\s*\(", src, re.M)))


def test_exports_every_declared_symbol():
    lib = nq.load()
    names = _declared()
    assert set(names) == set(nq.EXPORTED)
    for name in names:
        assert hasattr(lib, name), name


def test_plane_sizes_and_workspace():
    c = nq.Config(128, 2, 2, 0, nq.PARITY_RELAXED, nq.DTYPE_F16, 5e5)
    assert [nq.packed_bytes(c, 0, 10, p) for p in range(3)] == [320, 20, 20]
    c3 = nq.Config(128, 3, 2, 64, nq.PARITY_RELAXED, nq.DTYPE_F16, 1e6)
    assert [nq.packed_bytes(c3, 0, 1, p) for p in range(3)] == [48, 2, 4]
    assert [nq.packed_bytes(c3, 1, 1, p) for p in range(3)] == [32, 2, 4]
    c96 = nq.Config(96, 2, 2, 0, nq.PARITY_STRICT, nq.DTYPE_F16, 1e4)
    assert [nq.packed_bytes(c96, 0, 1, p) for p in range(3)] == [32, 2, 2]
    c8 = nq.Config(8, 2, 2, 8, nq.PARITY_STRICT, nq.DTYPE_F32, 0.0)
    assert [nq.packed_bytes(c8, 0, 64, p) for p in range(3)] == [128, 64, 128]
    # fp32 and fp64 RoPE tables (keys with theta > 0), 256 bytes of counters,
    # two queues of min(n, max(1024, n / 32)) 8-byte entries, each part
    # rounded up to 256 bytes
    def r(b):
        return (b + 255) // 256 * 256

    def ws(cfg, S, H, T, rope):
        n = S * H * T
        cap = min(n, max(1024, n // 32))
        th = T * cfg.head_dim // 2
        return (r(th * 8) + r(cfg.head_dim // 2 * 8) if rope else 0) + 256 + 2 * r(cap * 8)

    assert nq.workspace_bytes(c, 1, 1, 32768) == ws(c, 1, 1, 32768, True) == \
        32768 * 64 * 8 + 512 + 256 + 2 * 8192
    assert nq.workspace_bytes(c, 32, 8, 32768) == 32768 * 64 * 8 + 512 + 256 + 2 * (1 << 21)
    assert nq.workspace_bytes(c, 1, 1, 3) == 1536 + 512 + 256 + 512
    c8r = nq.Config(8, 2, 2, 8, 0, 0, 1e4)
    assert nq.workspace_bytes(c8r, 1, 1, 3) == ws(c8r, 1, 1, 3, True) == 1280
    assert nq.workspace_bytes(c8, 1, 1, 64) == ws(c8, 1, 1, 64, False) == 1280
    assert nq.workspace_bytes(c, 0, 1, 3) == 0 and nq.workspace_bytes(c, 1, 1, 0) == 0
    assert nq.packed_bytes(c, 0, 1, 7) == 0
    assert nq.packed_bytes(nq.Config(exact=2), 0, 1, 0) == 0      # exact must be 0 or 1


@pytest.mark.parametrize("kw", [dict(head_dim=7), dict(head_dim=264), dict(bits_k=4),
                                dict(bits_v=1), dict(scale_group=24), dict(scale_group=256),
                                dict(head_dim=40, rope_theta=1e4)])
def test_unsupported_configs(kw):
    base = dict(head_dim=128, bits_k=2, bits_v=2, scale_group=0, parity=1, in_dtype=0,
                rope_theta=0.0)
    base.update(kw)
    c = nq.Config(**base)
    assert nq.packed_bytes(c, 0, 1, 0) == 0
    cc = c.c()
    pk = nq._Packed(0x1000, 0x2000, 0x3000)
    st = nq.load().nq_quantize_kv(ctypes.byref(cc), 0x10000, None, 1, 1, 4, None,
                                  ctypes.byref(pk), None, None, 0, None)
    assert st == nq.NQ_ERR_UNSUPPORTED


def test_invalid_arguments_rejected_before_launch():
    lib = nq.load()
    c = nq.Config(128, 2, 2, 0, nq.PARITY_RELAXED, nq.DTYPE_F16, 5e5).c()
    pk = nq._Packed(0x1000, 0x2000, 0x3000)
    bad = nq._Packed(0x1008, 0x2000, 0x3000)
    q = lambda *a: lib.nq_quantize_kv(*a)  # noqa: E731
    # null config, no tensors, bad shape, misaligned input / plane / positions
    assert q(None, 0x10000, None, 1, 1, 4, None, ctypes.byref(pk), None, None, 0, None) == -1
    assert q(ctypes.byref(c), None, None, 1, 1, 4, None, None, None, None, 0, None) == -1
    assert q(ctypes.byref(c), 0x10000, None, 0, 1, 4, None, ctypes.byref(pk), None, None, 0, None) == -1
    assert q(ctypes.byref(c), 0x10004, None, 1, 1, 4, None, ctypes.byref(pk), None, None, 0, None) == -1
    assert q(ctypes.byref(c), 0x10000, None, 1, 1, 4, None, ctypes.byref(bad), None, None, 0, None) == -1
    assert q(ctypes.byref(c), 0x10000, None, 1, 1, 4, 0x5004, ctypes.byref(pk), None, None, 0, None) == -1
    assert q(ctypes.byref(c), 0x10000, None, 1, 1, 4, None, None, None, None, 0, None) == -1
    # keys with RoPE need the workspace table
    assert q(ctypes.byref(c), 0x10000, None, 1, 1, 4, None, ctypes.byref(pk), None, None, 0, None) == -3
    assert q(ctypes.byref(c), 0x10000, None, 1, 1, 4, None, ctypes.byref(pk), None, 0x8000, 128, None) == -3
    # values need the workspace too (the queue of the fp64 pass); a misaligned
    # workspace is rejected
    nb = nq.workspace_bytes(nq.Config(128, 2, 2, 0, 1, 0, 5e5), 1, 1, 4)
    assert q(ctypes.byref(c), None, 0x10000, 1, 1, 4, None, None, ctypes.byref(pk), None, 0, None) == -3
    assert q(ctypes.byref(c), None, 0x10000, 1, 1, 4, None, None, ctypes.byref(pk), 0x8000, nb - 1,
             None) == -3
    assert q(ctypes.byref(c), None, 0x10000, 1, 1, 4, None, None, ctypes.byref(pk), 0x8008, nb,
             None) == -1
    dq = lib.nq_dequantize_kv
    assert dq(ctypes.byref(c), ctypes.byref(pk), None, 1, 1, 4, None, None, None, None, 0, None) == -1
    assert dq(ctypes.byref(c), ctypes.byref(pk), None, 1, 1, 4, None, 0x10000, None, None, 0, None) == -3
    sc = lib.nq_score_packed_keys
    assert sc(ctypes.byref(c), ctypes.byref(pk), 1, 3, 4, 8, 0x10000, 0x20000, None, 0, None) == -1
    assert sc(ctypes.byref(c), ctypes.byref(pk), 1, 2, 4, 8, 0x10000, 0x20008, None, 0, None) == -1
    at = lib.nq_attend_packed_values
    assert at(ctypes.byref(c), ctypes.byref(pk), 1, 3, 4, 8, 0x10000, 0x20000, None) == -1
    assert at(ctypes.byref(c), ctypes.byref(pk), 1, 2, 4, 8, 0x10004, 0x20000, None) == -1
    assert at(ctypes.byref(c), None, 1, 2, 4, 8, 0x10000, 0x20000, None) == -1
    assert at(ctypes.byref(c), ctypes.byref(pk), 0, 2, 4, 8, 0x10000, 0x20000, None) == -1
    dd = lib.nq_e8_decode_debug
    assert dd(0x1000, 10, 4, 0, 1, 0x2000, 0x3000, None) == -2
    assert dd(0x1000, 0, 2, 0, 1, 0x2000, 0x3000, None) == -1
    assert dd(0x1000, 10, 2, 5, 1, 0x2000, 0x3000, None) == -1
    assert dd(0x1000, 10, 2, 0, 2, 0x2000, 0x3000, None) == -1
    for s in (0, -1, -2, -3, -4, 9):
        assert isinstance(nq.status_string(s), str)


@pytest.mark.parametrize("kw", [
    dict(rope_scaling=3),
    dict(rope_scaling=-1),
    dict(rope_scaling=nq.ROPE_SCALING_LINEAR, rope_factor=0.0),
    dict(rope_scaling=nq.ROPE_SCALING_LINEAR, rope_factor=float("inf")),
    dict(rope_scaling=nq.ROPE_SCALING_LLAMA3, rope_factor=8.0, rope_original_max=0),
    dict(rope_scaling=nq.ROPE_SCALING_LLAMA3, rope_factor=8.0, rope_original_max=8192,
         rope_low_freq_factor=4.0, rope_high_freq_factor=1.0),
    dict(rope_scaling=nq.ROPE_SCALING_LLAMA3, rope_factor=8.0, rope_original_max=8192,
         rope_low_freq_factor=0.0),
])
def test_invalid_rope_scaling_rejected(kw):
    c = nq.Config(128, 2, 2, 0, nq.PARITY_RELAXED, nq.DTYPE_F16, 5e5, **kw)
    assert nq.packed_bytes(c, 0, 1, 0) == 0
    pk = nq._Packed(0x1000, 0x2000, 0x3000)
    cc = c.c()
    st = nq.load().nq_quantize_kv(ctypes.byref(cc), 0x10000, None, 1, 1, 4, None,
                                  ctypes.byref(pk), None, 0x8000, 1 << 20, None)
    assert st == nq.NQ_ERR_INVALID_ARG


def test_rope_scaling_from_hf_dict():
    f = nq.Config.scaling_from_hf({"rope_type": "llama3", "factor": 8.0, "low_freq_factor": 1.0,
                                   "high_freq_factor": 4.0,
                                   "original_max_position_embeddings": 8192})
    c = nq.Config(128, 2, 2, 0, 1, 0, 5e5, **f)
    assert (c.rope_scaling, c.rope_original_max, c.rope_factor) == (nq.ROPE_SCALING_LLAMA3, 8192, 8.0)
    assert nq.packed_bytes(c, 0, 1, 0) == 32
    assert nq.Config.scaling_from_hf(None) == {"rope_scaling": nq.ROPE_SCALING_NONE}
    assert nq.Config.scaling_from_hf({"type": "linear", "factor": 2.0})["rope_factor"] == 2.0
    with pytest.raises(ValueError):
        nq.Config.scaling_from_hf({"rope_type": "yarn", "factor": 4.0})


def test_token_window_checked_before_launch():
    lib = nq.load()
    c = nq.Config(128, 2, 2, 0, nq.PARITY_RELAXED, nq.DTYPE_F16, 0.0).c()
    q = lambda pk: lib.nq_quantize_kv(ctypes.byref(c), 0x10000, None, 1, 1, 4, None,  # noqa: E731
                                      ctypes.byref(pk), None, None, 0, None)
    # window past the capacity, negative offset or capacity
    assert q(nq._Packed(0x1000, 0x2000, 0x3000, 10, 7)) == nq.NQ_ERR_INVALID_ARG
    assert q(nq._Packed(0x1000, 0x2000, 0x3000, 0, -1)) == nq.NQ_ERR_INVALID_ARG
    assert q(nq._Packed(0x1000, 0x2000, 0x3000, -5, 0)) == nq.NQ_ERR_INVALID_ARG
    assert q(nq._Packed(0x1000, 0x2000, 0x3000, 3, 0)) == nq.NQ_ERR_INVALID_ARG
    # the same checks guard the reading entry points
    pk = nq._Packed(0x1000, 0x2000, 0x3000, 10, 7)
    assert lib.nq_dequantize_kv(ctypes.byref(c), ctypes.byref(pk), None, 1, 1, 4, None,
                                0x10000, None, None, 0, None) == nq.NQ_ERR_INVALID_ARG
    assert lib.nq_score_packed_keys(ctypes.byref(c), ctypes.byref(pk), 1, 1, 2, 4, 0x10000,
                                    0x20000, None, 0, None) == nq.NQ_ERR_INVALID_ARG
    assert lib.nq_attend_packed_values(ctypes.byref(c), ctypes.byref(pk), 1, 1, 2, 4, 0x10000,
                                       0x20000, None) == nq.NQ_ERR_INVALID_ARG


def test_compact_packing_host_checks():
    lib = nq.load()
    ok = nq.Config(128, 2, 2, 0, nq.PARITY_STRICT, nq.DTYPE_F16, 0.0, packing=nq.PACKING_COMPACT)
    bad = nq.Config(128, 2, 2, 0, nq.PARITY_RELAXED, nq.DTYPE_F16, 0.0, packing=nq.PACKING_COMPACT)
    assert nq.packed_bytes(ok, 0, 10, nq.PLANE_CODES) == 320
    assert nq.packed_bytes(ok, 0, 10, nq.PLANE_COSETS) == 0
    assert nq.packed_bytes(bad, 0, 10, nq.PLANE_CODES) == 0
    assert nq.packed_bytes(nq.Config(128, 2, 2, 0, 0, 0, 0.0, packing=7), 0, 10, 0) == 0
    cc, cb = ok.c(), bad.c()
    nocs = nq._Packed(0x1000, None, 0x3000)
    q = lib.nq_quantize_kv
    # relaxed + compact is rejected; compact accepts a NULL coset plane, standard does not
    assert q(ctypes.byref(cb), 0x10000, None, 1, 1, 4, None, ctypes.byref(nocs), None, None, 0,
             None) == nq.NQ_ERR_INVALID_ARG
    std = nq.Config(128, 2, 2, 0, nq.PARITY_STRICT, nq.DTYPE_F16, 0.0).c()
    assert q(ctypes.byref(std), 0x10000, None, 1, 1, 4, None, ctypes.byref(nocs), None, None, 0,
             None) == nq.NQ_ERR_INVALID_ARG
    # (a valid compact call would launch; only its argument checks run here)
    assert q(ctypes.byref(cc), 0x10004, None, 1, 1, 4, None, ctypes.byref(nocs), None, None, 0,
             None) == nq.NQ_ERR_INVALID_ARG


def test_build_spill_check_parses_remarks():
    from e8_lattice_vector_amd import build
    txt = ("x.hip:2:1: remark: Function Name: _Z1kv [-Rpass-analysis=kernel-resource-usage]\n"
           "x.hip:2:1: remark:     ScratchSize [bytes/lane]: 0 [-Rpass-analysis=kernel-resource-usage]\n"
           "x.hip:9:1: remark: Function Name: _Z2k2v [-Rpass-analysis=kernel-resource-usage]\n"
           "x.hip:9:1: remark:     ScratchSize [bytes/lane]: 12 [-Rpass-analysis=kernel-resource-usage]\n")
    assert build.spilling_kernels(txt) == [("_Z2k2v", 12)]


def test_no_alloc_checks_before_launch():
    """nq_quantize_kv_noalloc refuses, on the host and before anything is
    enqueued, calls whose workspace exceeds its 32 MiB array, and reports
    config errors like nq_quantize_kv (no GPU needed)."""
    lib = nq.load()
    c = nq.Config(128, 2, 2, 0, nq.PARITY_RELAXED, nq.DTYPE_F16, 5e5)
    cc = c.c()
    pk = nq._Packed(0x1000, 0x2000, 0x3000)
    f = lib.nq_quantize_kv_noalloc
    assert nq.workspace_bytes(c, 1, 1, 131072) > 32 << 20
    assert f(ctypes.byref(cc), 0x10000, None, 1, 1, 131072, None, ctypes.byref(pk), None,
             None) == nq.NQ_ERR_WORKSPACE
    bad = nq.Config(128, 4, 2, 0, nq.PARITY_RELAXED, nq.DTYPE_F16, 5e5).c()
    assert f(ctypes.byref(bad), 0x10000, None, 1, 1, 4, None, ctypes.byref(pk), None,
             None) == nq.NQ_ERR_UNSUPPORTED
    assert f(ctypes.byref(cc), 0x10000, None, 0, 1, 4, None, ctypes.byref(pk), None,
             None) == nq.NQ_ERR_INVALID_ARG
