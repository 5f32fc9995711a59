"""ctypes binding of libnq (include/nq.h).  Argument marshalling only: every
step of quantize / dequantize / score runs in the HIP kernels of libnq.so.

Tensors are torch tensors in device memory; torch supplies allocation and
the current stream.  The library itself allocates nothing.
"""

from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libnq.so")

NQ_OK = 0
NQ_ERR_INVALID_ARG = -1
NQ_ERR_UNSUPPORTED = -2
NQ_ERR_WORKSPACE = -3
NQ_ERR_HIP = -4
PARITY_STRICT = 0
PARITY_RELAXED = 1
DTYPE_F16 = 0
DTYPE_F32 = 1
PLANE_CODES, PLANE_COSETS, PLANE_SCALES = 0, 1, 2
ROPE_SCALING_NONE, ROPE_SCALING_LINEAR, ROPE_SCALING_LLAMA3 = 0, 1, 2
PACKING_STANDARD, PACKING_COMPACT = 0, 1

EXPORTED = ("nq_packed_bytes", "nq_workspace_bytes", "nq_status_string",
            "nq_quantize_kv", "nq_dequantize_kv", "nq_score_packed_keys",
            "nq_attend_packed_values", "nq_e8_decode_debug", "nq_quantize_kv_noalloc")


class _Config(ctypes.Structure):
    _fields_ = [("head_dim", ctypes.c_int32), ("bits_k", ctypes.c_int32),
                ("bits_v", ctypes.c_int32), ("scale_group", ctypes.c_int32),
                ("parity", ctypes.c_int32), ("in_dtype", ctypes.c_int32),
                ("rope_theta", ctypes.c_double),
                ("rope_scaling", ctypes.c_int32), ("rope_original_max", ctypes.c_int32),
                ("rope_factor", ctypes.c_double), ("rope_low_freq_factor", ctypes.c_double),
                ("rope_high_freq_factor", ctypes.c_double), ("packing", ctypes.c_int32),
                ("exact", ctypes.c_int32)]


class _Packed(ctypes.Structure):
    _fields_ = [("codes", ctypes.c_void_p), ("cosets", ctypes.c_void_p),
                ("scales", ctypes.c_void_p), ("token_capacity", ctypes.c_int64),
                ("token_offset", ctypes.c_int64)]


class NQError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__(f"{what}: {status_string(status)} ({status})")


_lib = None


def load(path: str = LIB_PATH):
    """Load libnq.so; raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise ImportError(f"libnq.so not built at {path}; run "
                          "`python -m e8_lattice_vector_amd.build`")
    lib = ctypes.CDLL(path)
    vp, i32, i64, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
    cfgp, pkp = ctypes.POINTER(_Config), ctypes.POINTER(_Packed)
    lib.nq_packed_bytes.argtypes = [cfgp, ctypes.c_int, i64, ctypes.c_int]
    lib.nq_packed_bytes.restype = sz
    lib.nq_workspace_bytes.argtypes = [cfgp, i64, i32, i64]
    lib.nq_workspace_bytes.restype = sz
    lib.nq_status_string.argtypes = [ctypes.c_int]
    lib.nq_status_string.restype = ctypes.c_char_p
    lib.nq_quantize_kv.argtypes = [cfgp, vp, vp, i64, i32, i64, vp, pkp, pkp, vp, sz, vp]
    lib.nq_quantize_kv.restype = ctypes.c_int
    lib.nq_quantize_kv_noalloc.argtypes = [cfgp, vp, vp, i64, i32, i64, vp, pkp, pkp, vp]
    lib.nq_quantize_kv_noalloc.restype = ctypes.c_int
    lib.nq_dequantize_kv.argtypes = [cfgp, pkp, pkp, i64, i32, i64, vp, vp, vp, vp, sz, vp]
    lib.nq_dequantize_kv.restype = ctypes.c_int
    lib.nq_score_packed_keys.argtypes = [cfgp, pkp, i64, i32, i32, i64, vp, vp, vp, sz, vp]
    lib.nq_score_packed_keys.restype = ctypes.c_int
    lib.nq_attend_packed_values.argtypes = [cfgp, pkp, i64, i32, i32, i64, vp, vp, vp]
    lib.nq_attend_packed_values.restype = ctypes.c_int
    lib.nq_e8_decode_debug.argtypes = [vp, i64, i32, i32, i32, vp, vp, vp]
    lib.nq_e8_decode_debug.restype = ctypes.c_int
    _lib = lib
    return lib


def status_string(status: int) -> str:
    return load().nq_status_string(int(status)).decode()


@dataclass(frozen=True)
class Config:
    """Mirror of nq_config."""
    head_dim: int = 128
    bits_k: int = 2
    bits_v: int = 2
    scale_group: int = 0
    parity: int = PARITY_RELAXED
    in_dtype: int = DTYPE_F16
    rope_theta: float = 0.0
    rope_scaling: int = ROPE_SCALING_NONE
    rope_original_max: int = 0
    rope_factor: float = 1.0
    rope_low_freq_factor: float = 1.0
    rope_high_freq_factor: float = 4.0
    packing: int = PACKING_STANDARD
    exact: int = 0

    def c(self) -> _Config:
        return _Config(self.head_dim, self.bits_k, self.bits_v, self.scale_group,
                       self.parity, self.in_dtype, float(self.rope_theta),
                       self.rope_scaling, self.rope_original_max, float(self.rope_factor),
                       float(self.rope_low_freq_factor), float(self.rope_high_freq_factor),
                       self.packing, self.exact)

    @staticmethod
    def scaling_from_hf(rope_scaling) -> dict:
        """Config fields for a model config's ``rope_scaling`` dict (None,
        {"rope_type": "linear", "factor": f} or {"rope_type": "llama3",
        "factor", "low_freq_factor", "high_freq_factor",
        "original_max_position_embeddings"})."""
        if not rope_scaling:
            return {"rope_scaling": ROPE_SCALING_NONE}
        kind = rope_scaling.get("rope_type", rope_scaling.get("type"))
        if kind == "linear":
            return {"rope_scaling": ROPE_SCALING_LINEAR,
                    "rope_factor": float(rope_scaling["factor"])}
        if kind == "llama3":
            return {"rope_scaling": ROPE_SCALING_LLAMA3,
                    "rope_factor": float(rope_scaling["factor"]),
                    "rope_low_freq_factor": float(rope_scaling["low_freq_factor"]),
                    "rope_high_freq_factor": float(rope_scaling["high_freq_factor"]),
                    "rope_original_max": int(rope_scaling["original_max_position_embeddings"])}
        raise ValueError(f"unsupported rope_scaling type {kind!r}")

    @property
    def n(self) -> int:
        n = 8
        while n < self.head_dim:
            n *= 2
        return n

    @property
    def torch_dtype(self):
        return torch.float16 if self.in_dtype == DTYPE_F16 else torch.float32


@dataclass
class Packed:
    """Three planes shaped [S][H][capacity][bytes]; a call covers the token
    window [token_offset, token_offset + T) of every (slab, head) plane."""
    codes: torch.Tensor
    cosets: torch.Tensor
    scales: torch.Tensor

    @property
    def capacity(self) -> int:
        return self.codes.shape[2]

    def c(self, token_offset: int = 0) -> _Packed:
        return _Packed(self.codes.data_ptr(), self.cosets.data_ptr(),
                       self.scales.data_ptr(), self.capacity, int(token_offset))

    def nbytes(self) -> int:
        return sum(t.numel() * t.element_size() for t in (self.codes, self.cosets, self.scales))


def _ptr(t):
    return None if t is None else t.data_ptr()


def _stream(stream):
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    return getattr(stream, "cuda_stream", stream)


def _check(status: int, what: str):
    if status != NQ_OK:
        raise NQError(status, what)


def _bad(what: str):
    raise NQError(NQ_ERR_INVALID_ARG, what)


def _check_tensor(t, dtype, shape, what: str):
    """A caller-supplied device tensor must have this dtype and shape and be
    contiguous (the library writes it as a dense row-major array)."""
    if (t.dtype != dtype or not t.is_contiguous() or tuple(t.shape) != tuple(shape)
            or t.device.type != "cuda"):
        _bad(f"{what}: need a contiguous {dtype} device tensor of shape {tuple(shape)}, "
             f"got {t.dtype} {tuple(t.shape)} on {t.device}")


def _check_positions(positions, T: int, what: str):
    if positions is not None and (positions.dtype != torch.int32 or positions.numel() != T
                                  or not positions.is_contiguous()):
        _bad(f"{what} positions: need {T} contiguous int32 values")


def _check_packed(cfg: Config, p: Packed, is_value: bool, S: int, H: int, T: int,
                  token_offset: int, what: str):
    """Planes [S][H][capacity][bytes per vector] with the config's byte counts
    and room for tokens [token_offset, token_offset + T)."""
    if token_offset < 0 or p.codes.dim() != 4:
        _bad(f"{what}: planes must be [S][H][capacity][bytes]")
    cap = p.capacity
    if cap < token_offset + T:
        _bad(f"{what}: capacity {cap} < token window end {token_offset + T}")
    nb = [packed_bytes(cfg, is_value, 1, pl) for pl in (PLANE_CODES, PLANE_COSETS, PLANE_SCALES)]
    for t, dt, per, name in ((p.codes, torch.uint8, nb[0], "codes"),
                             (p.cosets, torch.uint8, nb[1], "cosets"),
                             (p.scales, torch.float16, nb[2] // 2, "scales")):
        if t.dtype != dt or not t.is_contiguous() or tuple(t.shape) != (S, H, cap, per):
            _bad(f"{what} {name}: need a contiguous {dt} tensor of shape {(S, H, cap, per)}, "
                 f"got {t.dtype} {tuple(t.shape)}")


def packed_bytes(cfg: Config, is_value: bool, n_vectors: int, plane: int) -> int:
    cc = cfg.c()
    return int(load().nq_packed_bytes(ctypes.byref(cc), int(is_value), int(n_vectors), plane))


def workspace_bytes(cfg: Config, S: int, H: int, T: int) -> int:
    cc = cfg.c()
    return int(load().nq_workspace_bytes(ctypes.byref(cc), int(S), int(H), int(T)))


def alloc_packed(cfg: Config, is_value: bool, S: int, H: int, T: int, device) -> Packed:
    """Caller-side allocation of the three planes (torch owns the memory)."""
    nv = S * H * T
    planes = []
    for plane in (PLANE_CODES, PLANE_COSETS, PLANE_SCALES):
        nb = packed_bytes(cfg, is_value, nv, plane)
        # the coset plane is empty with compact packing
        if nb == 0 and not (plane == PLANE_COSETS and cfg.packing == PACKING_COMPACT):
            raise NQError(NQ_ERR_INVALID_ARG, "packed_bytes")
        planes.append(torch.empty(nb, dtype=torch.uint8, device=device))
    codes, cosets, scales = planes
    return Packed(codes.view(S, H, T, -1), cosets.view(S, H, T, cosets.numel() // max(nv, 1)),
                  scales.view(torch.float16).view(S, H, T, -1))


def alloc_workspace(cfg: Config, S: int, H: int, T: int, device):
    """Workspace for quantize (and dequantize) calls on S x H x T vectors."""
    nb = workspace_bytes(cfg, S, H, T)
    if nb == 0:
        raise NQError(NQ_ERR_INVALID_ARG, "workspace_bytes")
    return torch.empty(nb, dtype=torch.uint8, device=device)


def quantize_kv(cfg: Config, k, v, positions=None, pk: Packed | None = None,
                pv: Packed | None = None, workspace=None, stream=None, token_offset: int = 0):
    """Quantize + pack K and/or V ([S][H][T][d] device tensors) into tokens
    [token_offset, token_offset + T) of the packed planes."""
    ref = k if k is not None else v
    S, H, T, d = ref.shape
    if d != cfg.head_dim:
        raise NQError(NQ_ERR_INVALID_ARG, "quantize_kv head_dim")
    for t in (k, v):
        if t is not None and (t.dtype != cfg.torch_dtype or not t.is_contiguous()
                              or tuple(t.shape) != (S, H, T, d)):
            raise NQError(NQ_ERR_INVALID_ARG, "quantize_kv tensor")
    if k is not None and pk is None:
        pk = alloc_packed(cfg, False, S, H, token_offset + T, k.device)
    if v is not None and pv is None:
        pv = alloc_packed(cfg, True, S, H, token_offset + T, v.device)
    if k is not None:
        _check_packed(cfg, pk, False, S, H, T, token_offset, "quantize_kv pk")
    if v is not None:
        _check_packed(cfg, pv, True, S, H, T, token_offset, "quantize_kv pv")
    if workspace is None:
        workspace = alloc_workspace(cfg, S, H, T, ref.device)
    _check_positions(positions, T, "quantize_kv")
    cc = cfg.c()
    ck = pk.c(token_offset) if k is not None else None
    cv = pv.c(token_offset) if v is not None else None
    st = load().nq_quantize_kv(
        ctypes.byref(cc), _ptr(k), _ptr(v), S, H, T, _ptr(positions),
        ctypes.byref(ck) if ck is not None else None,
        ctypes.byref(cv) if cv is not None else None,
        _ptr(workspace), 0 if workspace is None else workspace.numel(), _stream(stream))
    _check(st, "nq_quantize_kv")
    return pk, pv


def quantize_kv_noalloc(cfg: Config, k, v, pk: Packed | None, pv: Packed | None,
                        positions=None, stream=None, token_offset: int = 0):
    """quantize_kv through nq_quantize_kv_noalloc: the library's own static
    workspace; the caller supplies the packed planes (nothing is allocated)."""
    ref = k if k is not None else v
    S, H, T, d = ref.shape
    if d != cfg.head_dim:
        _bad("quantize_kv_noalloc head_dim")
    for t, p, is_v in ((k, pk, False), (v, pv, True)):
        if t is None:
            continue
        if t.dtype != cfg.torch_dtype or not t.is_contiguous() or tuple(t.shape) != (S, H, T, d):
            _bad("quantize_kv_noalloc tensor")
        if p is None:
            _bad("quantize_kv_noalloc needs the packed planes")
        _check_packed(cfg, p, is_v, S, H, T, token_offset, "quantize_kv_noalloc")
    _check_positions(positions, T, "quantize_kv_noalloc")
    cc = cfg.c()
    ck = pk.c(token_offset) if k is not None else None
    cv = pv.c(token_offset) if v is not None else None
    st = load().nq_quantize_kv_noalloc(
        ctypes.byref(cc), _ptr(k), _ptr(v), S, H, T, _ptr(positions),
        ctypes.byref(ck) if ck is not None else None,
        ctypes.byref(cv) if cv is not None else None, _stream(stream))
    _check(st, "nq_quantize_kv_noalloc")
    return pk, pv


def dequantize_kv(cfg: Config, pk: Packed | None, pv: Packed | None, S: int, H: int,
                  T: int, positions=None, k_out=None, v_out=None, workspace=None,
                  stream=None, token_offset: int = 0):
    """Dequantize tokens [token_offset, token_offset + T) -> [S][H][T][d]."""
    if pk is None and pv is None:
        _bad("dequantize_kv: neither pk nor pv")
    dev = (pk if pk is not None else pv).codes.device
    shape = (S, H, T, cfg.head_dim)
    if pk is not None:
        _check_packed(cfg, pk, False, S, H, T, token_offset, "dequantize_kv pk")
        if k_out is None:
            k_out = torch.empty(shape, dtype=cfg.torch_dtype, device=dev)
        _check_tensor(k_out, cfg.torch_dtype, shape, "dequantize_kv k_out")
    if pv is not None:
        _check_packed(cfg, pv, True, S, H, T, token_offset, "dequantize_kv pv")
        if v_out is None:
            v_out = torch.empty(shape, dtype=cfg.torch_dtype, device=dev)
        _check_tensor(v_out, cfg.torch_dtype, shape, "dequantize_kv v_out")
    _check_positions(positions, T, "dequantize_kv")
    if workspace is None and pk is not None and cfg.rope_theta > 0:
        workspace = alloc_workspace(cfg, S, H, T, dev)
    cc = cfg.c()
    ck = pk.c(token_offset) if pk is not None else None
    cv = pv.c(token_offset) if pv is not None else None
    st = load().nq_dequantize_kv(
        ctypes.byref(cc), ctypes.byref(ck) if ck is not None else None,
        ctypes.byref(cv) if cv is not None else None, S, H, T, _ptr(positions),
        _ptr(k_out if pk is not None else None), _ptr(v_out if pv is not None else None),
        _ptr(workspace), 0 if workspace is None else workspace.numel(), _stream(stream))
    _check(st, "nq_dequantize_kv")
    return (k_out if pk is not None else None), (v_out if pv is not None else None)


def score_packed_keys(cfg: Config, pk: Packed, q, S: int, H: int, T: int,
                      scores=None, stream=None, token_offset: int = 0):
    """q: [S][Hq][d] device tensor -> fp32 scores [S][Hq][T] against keys
    [token_offset, token_offset + T)."""
    Hq = q.shape[1]
    if q.dtype != cfg.torch_dtype or not q.is_contiguous() or q.shape != (S, Hq, cfg.head_dim):
        raise NQError(NQ_ERR_INVALID_ARG, "score_packed_keys q")
    _check_packed(cfg, pk, False, S, H, T, token_offset, "score_packed_keys pk")
    if scores is None:
        scores = torch.empty((S, Hq, T), dtype=torch.float32, device=q.device)
    _check_tensor(scores, torch.float32, (S, Hq, T), "score_packed_keys scores")
    cc = cfg.c()
    ck = pk.c(token_offset)
    st = load().nq_score_packed_keys(ctypes.byref(cc), ctypes.byref(ck), S, H, Hq, T,
                                     q.data_ptr(), scores.data_ptr(), None, 0,
                                     _stream(stream))
    _check(st, "nq_score_packed_keys")
    return scores


def attend_packed_values(cfg: Config, pv: Packed, weights, S: int, H: int, T: int,
                         out=None, stream=None, token_offset: int = 0):
    """weights: fp32 [S][Hq][T] device tensor -> fp32 [S][Hq][d] sum_t w_t * V_t
    over values [token_offset, token_offset + T)."""
    Hq = weights.shape[1]
    if (weights.dtype != torch.float32 or not weights.is_contiguous()
            or tuple(weights.shape) != (S, Hq, T)):
        raise NQError(NQ_ERR_INVALID_ARG, "attend_packed_values weights")
    _check_packed(cfg, pv, True, S, H, T, token_offset, "attend_packed_values pv")
    if out is None:
        out = torch.empty((S, Hq, cfg.head_dim), dtype=torch.float32, device=weights.device)
    _check_tensor(out, torch.float32, (S, Hq, cfg.head_dim), "attend_packed_values out")
    cc = cfg.c()
    cv = pv.c(token_offset)
    st = load().nq_attend_packed_values(ctypes.byref(cc), ctypes.byref(cv), S, H, Hq, T,
                                        weights.data_ptr(), out.data_ptr(), _stream(stream))
    _check(st, "nq_attend_packed_values")
    return out


def e8_decode_debug(y, bits: int, parity: int, stream=None, constrained: bool = True):
    """y: device fp32 [N, 8] -> (idx uint8 [N, 8], coset uint8 [N]); with
    constrained=False the unconstrained decoder, idx as int8 in the uint8."""
    if y.dtype != torch.float32 or y.dim() != 2 or y.shape[1] != 8 or not y.is_contiguous():
        raise NQError(NQ_ERR_INVALID_ARG, "e8_decode_debug y")
    n = y.shape[0]
    idx = torch.empty((n, 8), dtype=torch.uint8, device=y.device)
    cos = torch.empty((n,), dtype=torch.uint8, device=y.device)
    st = load().nq_e8_decode_debug(y.data_ptr(), n, bits, parity, int(constrained), idx.data_ptr(),
                                   cos.data_ptr(), _stream(stream))
    _check(st, "nq_e8_decode_debug")
    return idx, cos
