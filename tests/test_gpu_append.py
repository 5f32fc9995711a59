"""Decode-time append (token windows of the packed planes) through the C ABI.

A cache filled by a prefill chunk, single-token appends and a multi-token
chunk, quantized block by block at the cache's end, must hold the same bytes
as one quantization of the whole prefix, and those bytes match the oracle.
Reads of a window (score, attend, dequantize) equal reads of a dense copy
(dequantized keys within one fp16 step).
"""

import numpy as np
import pytest
import torch

from e8_lattice_vector_amd import nq, synth
from e8_lattice_vector_amd.cache import PackedKVCache
from oracle import codec as oc

from parity import check_codes, check_dequant, oracle_codec, to_np

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]

DEV = "cuda"


def log(msg):
    print(msg, flush=True)


@pytest.mark.parametrize("cfg,block", [
    (nq.Config(128, 2, 2, 0, nq.PARITY_RELAXED, nq.DTYPE_F16, 5e5), 32),
    (nq.Config(96, 3, 2, 32, nq.PARITY_STRICT, nq.DTYPE_F16, 1e4), 16),
])
def test_append_matches_one_shot(cfg, block):
    S, H, T0, n_dec, cap = 2, 3, 301, 157, 520
    log(f"[append] d={cfg.head_dim} bits={cfg.bits_k}/{cfg.bits_v} block={block}")
    T = T0 + n_dec
    k = synth.kv("k", S, H, T, cfg.head_dim, cfg.rope_theta, 4, DEV)
    v = synth.kv("v", S, H, T, cfg.head_dim, 0.0, 4, DEV)
    cache = PackedKVCache(cfg, S, H, cap, block, DEV)
    cache.prefill(k[:, :, :T0].contiguous(), v[:, :, :T0].contiguous())
    t = T0
    for _ in range(45):                                   # single-token decode writes
        cache.append(k[:, :, t:t + 1], v[:, :, t:t + 1])
        t += 1
    cache.append(k[:, :, t:T], v[:, :, t:T])             # one multi-token chunk
    torch.cuda.synchronize()
    n = cache.n_packed
    assert n == T0 + (n_dec // block) * block and cache.n_res == n_dec % block
    rk, rv = cache.residual()
    assert torch.equal(rk, k[:, :, n:T]) and torch.equal(rv, v[:, :, n:T])
    # one quantization of the whole packed prefix
    kp, vp = k[:, :, :n].contiguous(), v[:, :, :n].contiguous()
    pk1, pv1 = nq.quantize_kv(cfg, kp, vp)
    torch.cuda.synchronize()
    for a, b in ((cache.pk, pk1), (cache.pv, pv1)):
        for x, y in ((a.codes, b.codes), (a.cosets, b.cosets), (a.scales, b.scales)):
            assert torch.equal(x[:, :, :n].view(torch.uint8), y.view(torch.uint8))
    # and the oracle on the same bytes
    for is_v, x, p in ((False, kp, cache.pk), (True, vp, cache.pv)):
        codec = oracle_codec(cfg, is_v)
        ref = oc.quantize(x.cpu().numpy(), codec, positions=np.arange(n), is_key=not is_v)
        codes, cosets, scales = (t_[:, :, :n].cpu().numpy() for t_ in (p.codes, p.cosets, p.scales))
        check_codes(codes, cosets, scales, ref, codec, f"append/{'V' if is_v else 'K'}")
    # window reads against dense copies of the same planes
    q = synth.queries(S, 2 * H, cfg.head_dim, 4, DEV)
    s_win = cache.score(q)
    s_ref = nq.score_packed_keys(cfg, pk1, q, S, H, n)
    w = torch.softmax(s_ref, dim=-1).contiguous()
    o_win = cache.attend(w)
    o_ref = nq.attend_packed_values(cfg, pv1, w, S, H, n)
    kd_win, vd_win = cache.dequantize(100, 150)
    pos = torch.arange(100, 250, dtype=torch.int32, device=DEV)
    sub = nq.Packed(*(t_[:, :, 100:250].contiguous() for t_ in (pk1.codes, pk1.cosets, pk1.scales)))
    subv = nq.Packed(*(t_[:, :, 100:250].contiguous() for t_ in (pv1.codes, pv1.cosets, pv1.scales)))
    kd_ref, vd_ref = nq.dequantize_kv(cfg, sub, subv, S, H, 150, positions=pos)
    torch.cuda.synchronize()
    assert torch.equal(s_win, s_ref)
    assert torch.equal(o_win, o_ref)
    assert torch.equal(vd_win, vd_ref)
    # keys: the window (positions 100 + t) takes the token-walking kernel,
    # whose cos / sin are rotated from tile to tile; the dense copy with
    # explicit positions forms them directly: within one fp16 step
    kw, kr = kd_win.float(), kd_ref.float()
    assert ((kw - kr).abs() <= kr.abs() * 2.0 ** -10 + 2.0 ** -24).all()
    # the dequantized window against the oracle (RoPE at positions 100..249)
    codec = oracle_codec(cfg, False)
    codes, cosets, scales = to_np(sub)
    xr = oc.dequantize(codes, cosets, scales, codec, positions=np.arange(100, 250), is_key=True)
    check_dequant(kd_win.float().cpu().numpy(), xr, "append/deqK")


def test_quantize_into_window_leaves_the_rest():
    """A quantize call on a window writes only that window of each plane."""
    cfg = nq.Config(64, 2, 2, 0, nq.PARITY_RELAXED, nq.DTYPE_F16, 1e4)
    S, H, cap, t0, T = 2, 2, 90, 37, 21
    log("[window] quantize into tokens 37..57 of 90")
    pk = nq.alloc_packed(cfg, False, S, H, cap, DEV)
    for t_ in (pk.codes, pk.cosets, pk.scales):
        t_.view(torch.uint8).fill_(0xA5)
    k = synth.kv("k", S, H, T, cfg.head_dim, cfg.rope_theta, 9, DEV)
    nq.quantize_kv(cfg, k, None, pk=pk, token_offset=t0)
    ref, _ = nq.quantize_kv(cfg, k, None, positions=torch.arange(t0, t0 + T, dtype=torch.int32,
                                                                  device=DEV))
    torch.cuda.synchronize()
    for a, b in ((pk.codes, ref.codes), (pk.cosets, ref.cosets), (pk.scales, ref.scales)):
        a8 = a.view(torch.uint8)
        assert torch.equal(a8[:, :, t0:t0 + T], b.view(torch.uint8))
        assert bool((a8[:, :, :t0] == 0xA5).all()) and bool((a8[:, :, t0 + T:] == 0xA5).all())
