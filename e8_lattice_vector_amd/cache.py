"""Decode-time append on the packed cache.

The behaviour of the pages' quantized cache (nexusquant-kv README,
"HuggingFace ecosystem"): the prefill KV is E8-quantized, and recent
single-token decode writes are kept in fp16 (a KIVI-style residual) until
they are quantized in turn.  Here the residual holds fewer than `block` tokens;
once it fills, the block is quantized into the packed planes at the cache's
end.

Buffer management only: every quantization, score and dequantization runs in
libnq, on a token window of planes allocated for `capacity` tokens
(nq_packed.token_capacity / token_offset).  Keys are rotated at positions
0, 1, 2, ... in the order they arrive, so each block gets RoPE positions
n_packed + t.
"""

from __future__ import annotations

import torch

from . import nq


class PackedKVCache:
    """K/V of S slabs x H KV heads with room for `capacity` tokens."""

    def __init__(self, cfg: nq.Config, S: int, H: int, capacity: int, block: int = 64,
                 device="cuda"):
        if block <= 0 or capacity <= 0:
            raise ValueError("block and capacity must be positive")
        self.cfg, self.S, self.H = cfg, S, H
        self.capacity, self.block = capacity, block
        self.pk = nq.alloc_packed(cfg, False, S, H, capacity, device)
        self.pv = nq.alloc_packed(cfg, True, S, H, capacity, device)
        shape = (S, H, block, cfg.head_dim)
        self.rk = torch.empty(shape, dtype=cfg.torch_dtype, device=device)
        self.rv = torch.empty(shape, dtype=cfg.torch_dtype, device=device)
        # sized for the larger of a decode block and nothing else: a prefill
        # allocates its own workspace
        self.ws = nq.alloc_workspace(cfg, S, H, block, device)
        self.n_packed = 0   # tokens 0 .. n_packed - 1 are in the packed planes
        self.n_res = 0      # the next n_res tokens wait in the fp16 residual

    @property
    def n_tokens(self) -> int:
        return self.n_packed + self.n_res

    def _room(self, t: int):
        if self.n_tokens + t > self.capacity:
            raise ValueError(f"cache full: {self.n_tokens} + {t} > {self.capacity}")

    def prefill(self, k, v, stream=None):
        """Quantize a prefill chunk [S][H][T][d] straight into the planes."""
        if self.n_res:
            raise ValueError("prefill after decode-time appends")
        T = k.shape[2]
        self._room(T)
        nq.quantize_kv(self.cfg, k, v, pk=self.pk, pv=self.pv, stream=stream,
                       token_offset=self.n_packed)
        self.n_packed += T

    def append(self, k, v, stream=None):
        """Append decode tokens [S][H][t][d]: they join the fp16 residual, and
        every full block of it is quantized into the planes."""
        t = k.shape[2]
        self._room(t)
        # the residual copies run on the same stream as the quantization that
        # reads them, so they are ordered before it
        if stream is None:
            ts = torch.cuda.current_stream()
        elif isinstance(stream, torch.cuda.Stream):
            ts = stream
        else:   # a raw hipStream_t handle
            ts = torch.cuda.ExternalStream(int(stream))
        i = 0
        while i < t:
            n = min(self.block - self.n_res, t - i)
            with torch.cuda.stream(ts):
                self.rk[:, :, self.n_res:self.n_res + n].copy_(k[:, :, i:i + n])
                self.rv[:, :, self.n_res:self.n_res + n].copy_(v[:, :, i:i + n])
            self.n_res += n
            i += n
            if self.n_res == self.block:
                nq.quantize_kv(self.cfg, self.rk, self.rv, pk=self.pk, pv=self.pv,
                               workspace=self.ws, stream=stream,
                               token_offset=self.n_packed)
                self.n_packed += self.block
                self.n_res = 0

    def residual(self):
        """fp16 K and V of the tokens not yet quantized, [S][H][n_res][d]."""
        return self.rk[:, :, :self.n_res], self.rv[:, :, :self.n_res]

    def score(self, q, stream=None):
        """Packed-key scores of q [S][Hq][d] against tokens 0 .. n_packed - 1."""
        return nq.score_packed_keys(self.cfg, self.pk, q, self.S, self.H, self.n_packed,
                                    stream=stream)

    def attend(self, weights, stream=None):
        """sum_t weights[s][h][t] V_t over the packed tokens."""
        return nq.attend_packed_values(self.cfg, self.pv, weights, self.S, self.H,
                                       self.n_packed, stream=stream)

    def dequantize(self, start: int = 0, count: int | None = None, stream=None):
        """fp16 K and V of packed tokens [start, start + count)."""
        count = self.n_packed - start if count is None else count
        return nq.dequantize_kv(self.cfg, self.pk, self.pv, self.S, self.H, count,
                                stream=stream, token_offset=start)
