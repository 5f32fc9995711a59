"""Benchmark of the E8 KV-cache hot path on one MI355X.

One step = the whole path over the Llama-3.1-8B 32K-token cache (32 layers x
8 KV heads x 32768 tokens x head_dim 128, fp16 K and V, k2v2 relaxed, one
scale per head vector):
  1. quantize + pack K (RoPE removed, theta 5e5) and V      nq_quantize_kv
  2. dequantize K (RoPE re-applied) and V                   nq_dequantize_kv
  3. score one decode query per query head (32 heads, GQA 4) against the
     packed keys                                            nq_score_packed_keys
Inputs are synthetic (e8_lattice_vector_amd.synth) and resident in HBM
before timing starts.  Prints one JSON line.

  python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]
"""

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0  # MI355X HBM3E, vendor figure


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-decode-shape", action="store_true",
                    help="skip the scoring run at the Qwen2.5-14B decode shape")
    ap.add_argument("--cpu-sample-tokens", type=int, default=32768,
                    help="tokens per slab (all 8 heads, K and V) the oracle runs on")
    ap.add_argument("--cpu-sample-slabs", type=int, default=2,
                    help="slabs of the cache the oracle runs on")
    return ap.parse_args()


def profiled_traffic(profiles):
    """HBM bytes per launch from committed rocprofv3 summaries (FETCH_SIZE and
    WRITE_SIZE, each scaled by the copy-kernel calibration), averaged over the
    summaries (one per launch of the step), or None when any is missing or the
    kernel source has changed since its counters were taken."""
    import hashlib
    import re

    src = os.path.join(ROOT, "e8_lattice_vector_amd", "csrc", "nq_kernels.hip")
    vals = []
    for profile in profiles:
        try:
            text = open(os.path.join(ROOT, "profiles", profile)).read()
            sha = hashlib.sha256(open(src, "rb").read()).hexdigest()
        except OSError:
            return None
        m_sha = re.search(r"nq_kernels.hip sha256: ([0-9a-f]{64})", text)
        m_tr = re.search(r"traffic_bytes_per_launch: (\d+)", text)
        if not m_sha or not m_tr or m_sha.group(1) != sha:
            return None
        vals.append(int(m_tr.group(1)))
    return round(sum(vals) / len(vals)) if vals else None


def cpu_baseline(w, tokens, slabs):
    """The oracle, as it stands, on a bounded sample of the same workload."""
    import numpy as np  # noqa: F401

    from e8_lattice_vector_amd import synth
    from oracle import codec as oc

    k = synth.kv("k", slabs, w.H, tokens, w.d, w.theta, 0).numpy()
    v = synth.kv("v", slabs, w.H, tokens, w.d, 0.0, 0).numpy()
    q = synth.queries(slabs, 32, w.d, 0).numpy()
    ck = oc.Codec(w.d, w.bits_k, w.G, w.strict, w.theta)
    cv = oc.Codec(w.d, w.bits_v, w.G, w.strict, 0.0)
    from threadpoolctl import threadpool_limits

    # one thread, so that "cores" is what the run used (numpy's BLAS would
    # otherwise spread the scoring products over the host's cores)
    with threadpool_limits(limits=1):
        t0 = time.perf_counter()
        rk = oc.quantize(k, ck, is_key=True)
        rv = oc.quantize(v, cv)
        oc.dequantize(rk["codes"], rk["cosets"], rk["scales"], ck, is_key=True)
        oc.dequantize(rv["codes"], rv["cosets"], rv["scales"], cv)
        oc.score(q, rk["codes"], rk["cosets"], rk["scales"], ck)
        dt = time.perf_counter() - t0
    cache_tokens = tokens * slabs / w.S  # slabs of S
    return {
        "value": cache_tokens / dt,
        "unit": "tokens/s",
        "cores": 1,
        "kind": "oracle",
        "sample": f"{slabs} of {w.S} slabs x {w.H} heads x {tokens} tokens, K+V quantize, "
                  f"dequantize and 32-query scoring ({dt:.1f} s single-threaded numpy)",
    }


def qwen_decode_scores(steps, warmup, dev, stream):
    """Packed-key scoring at the decode shape of the scoring row: 768 slabs
    (16 sequences x 48 layers) x 8 KV heads x 16384 keys, 40 query heads (GQA
    5). Keys come from the Llama generator and are quantized in slab batches,
    so only the packed keys (3.6 GB) stay resident; scores are 2.0 GB."""
    import torch

    from e8_lattice_vector_amd import nq, synth, workloads

    w = workloads.QWEN_DECODE
    cfg = nq.Config(w.d, w.bits_k, w.bits_v, w.G,
                    nq.PARITY_STRICT if w.strict else nq.PARITY_RELAXED, nq.DTYPE_F16, w.theta)
    pk = nq.alloc_packed(cfg, False, w.S, w.H, w.T, dev)
    batch = 32
    ws = nq.alloc_workspace(cfg, batch, w.H, w.T, dev)
    for s0 in range(0, w.S, batch):
        k = synth.kv("k", batch, w.H, w.T, w.d, w.theta, 0, dev, torch.float16, slab0=s0)
        sub = nq.Packed(pk.codes[s0:s0 + batch], pk.cosets[s0:s0 + batch],
                        pk.scales[s0:s0 + batch])
        nq.quantize_kv(cfg, k, None, pk=sub, workspace=ws)
        del k
    q = synth.queries(w.S, w.Hq, w.d, 0, dev)
    sc = torch.empty((w.S, w.Hq, w.T), dtype=torch.float32, device=dev)
    for _ in range(warmup):
        nq.score_packed_keys(cfg, pk, q, w.S, w.H, w.T, scores=sc)
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    torch.cuda.synchronize()
    ev[0].record(stream)
    for _ in range(steps):
        nq.score_packed_keys(cfg, pk, q, w.S, w.H, w.T, scores=sc)
    ev[1].record(stream)
    torch.cuda.synchronize()
    ms = ev[0].elapsed_time(ev[1]) / steps
    keys = w.S * w.H * w.T
    nbytes = pk.nbytes() + q.numel() * 2 + sc.numel() * 4
    del pk, ws, q, sc
    return {
        "workload": w.name,
        "ms": ms,
        "keys_per_s": keys / (ms * 1e-3),
        "GBps": nbytes / (ms * 1e-3) / 1e9,
        "pct_hbm_peak": 100 * nbytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBPS,
        "bytes": nbytes,
        "what": "scores of 40 fp16 decode queries per slab against 768 x 8 x 16384 packed keys "
                "(36 B/key read, 20 B/key written)",
    }


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (got --gpus {args.gpus}); the path has "
              "no cross-GPU step to measure.", file=sys.stderr)
        sys.exit(2)

    import torch

    from e8_lattice_vector_amd import nq, synth, workloads

    w = workloads.LLAMA
    dev = "cuda:0"
    torch.cuda.set_device(0)
    cfg = nq.Config(w.d, w.bits_k, w.bits_v, w.G,
                    nq.PARITY_STRICT if w.strict else nq.PARITY_RELAXED,
                    nq.DTYPE_F16, w.theta)
    Hq = 32
    k, v = synth.workload_inputs(w, seed=0, device=dev)
    q = synth.queries(w.S, Hq, w.d, 0, dev)
    pk = nq.alloc_packed(cfg, False, w.S, w.H, w.T, dev)
    pv = nq.alloc_packed(cfg, True, w.S, w.H, w.T, dev)
    ws = nq.alloc_workspace(cfg, w.S, w.H, w.T, dev)
    kd = torch.empty_like(k)
    vd = torch.empty_like(v)
    scores = torch.empty((w.S, Hq, w.T), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream()

    def step(ev=None):
        if ev is not None:
            ev[0].record(stream)
        nq.quantize_kv(cfg, k, None, pk=pk, workspace=ws)
        if ev is not None:
            ev[1].record(stream)
        nq.quantize_kv(cfg, None, v, pv=pv, workspace=ws)
        if ev is not None:
            ev[2].record(stream)
        nq.dequantize_kv(cfg, pk, pv, w.S, w.H, w.T, k_out=kd, v_out=vd, workspace=ws)
        if ev is not None:
            ev[3].record(stream)
        nq.score_packed_keys(cfg, pk, q, w.S, w.H, w.T, scores=scores)
        if ev is not None:
            ev[4].record(stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    events = [[torch.cuda.Event(enable_timing=True) for _ in range(5)]
              for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(events[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    seg = [[e[j].elapsed_time(e[j + 1]) for j in range(4)] for e in events]
    tk = sum(s[0] for s in seg) / args.steps
    tv = sum(s[1] for s in seg) / args.steps
    tdq = sum(s[2] for s in seg) / args.steps
    tsc = sum(s[3] for s in seg) / args.steps
    ms_step = wall * 1e3 / args.steps

    nv = w.S * w.H * w.T
    fp16_bytes = nv * w.d * 2
    vec_bytes = pk.nbytes() // nv
    packed = nv * vec_bytes
    table = w.T * (w.d // 2) * 8
    q_bytes = (fp16_bytes + packed) * 2 + table           # K and V, + RoPE table read
    dq_bytes = q_bytes
    sc_bytes = packed + w.S * Hq * w.d * 2 + w.S * Hq * w.T * 4
    tq = tk + tv
    q_gbps = q_bytes / (tq * 1e-3) / 1e9

    # next row: value half of decode attention on the packed V, weights =
    # softmax of the step's scores (timed on its own, not part of the step)
    wts = torch.softmax(scores, dim=-1).contiguous()
    att = torch.empty((w.S, Hq, w.d), dtype=torch.float32, device=dev)
    for _ in range(args.warmup):
        nq.attend_packed_values(cfg, pv, wts, w.S, w.H, w.T, out=att)
    ea = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    torch.cuda.synchronize()
    ea[0].record(stream)
    for _ in range(args.steps):
        nq.attend_packed_values(cfg, pv, wts, w.S, w.H, w.T, out=att)
    ea[1].record(stream)
    torch.cuda.synchronize()
    tat = ea[0].elapsed_time(ea[1]) / args.steps
    at_bytes = packed + w.S * Hq * w.T * 4 + w.S * Hq * w.d * 4
    del wts, att

    # plain device copy of 4 GiB for context
    src = torch.empty(1 << 31, dtype=torch.float16, device=dev)
    dst = torch.empty_like(src)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    dst.copy_(src)
    e0.record(stream)
    for _ in range(5):
        dst.copy_(src)
    e1.record(stream)
    torch.cuda.synchronize()
    copy_gbps = 2 * src.numel() * 2 * 5 / (e0.elapsed_time(e1) * 1e-3) / 1e9
    del src, dst

    out = {
        "metric": "KV quantize+pack tokens/s and HBM GB/s (% of peak), Llama-3.1-8B shape, 1 GPU",
        "value": w.T / (ms_step * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {
            "workload": w.name,
            "slabs": w.S, "kv_heads": w.H, "tokens": w.T, "head_dim": w.d,
            "codec": f"k{w.bits_k}v{w.bits_v} {'strict' if w.strict else 'relaxed'} "
                     f"scale per {w.G or w.d} coords, rope_theta {w.theta:g}",
            "step": "quantize+pack K,V -> dequantize K,V -> score 32 decode queries",
            "storage": "fp16 in/out, 36 B per packed vector",
        },
        "quantize": {
            "tokens_per_s": w.T / (tq * 1e-3),
            "ms": tq,
            "hbm_GBps": q_gbps,
            "fp16_kv_GBps": 2 * fp16_bytes / (tq * 1e-3) / 1e9,
            "pct_hbm_peak": 100 * q_gbps / HBM_PEAK_GBPS,
            "pct_copy_bw": 100 * q_gbps / copy_gbps,
        },
        "kernels_ms": {"quantize_k(+rope table)": tk, "quantize_v": tv,
                       "dequantize_kv(+rope table)": tdq, "score": tsc},
        "dequantize_GBps": dq_bytes / (tdq * 1e-3) / 1e9,
        "score_GBps": sc_bytes / (tsc * 1e-3) / 1e9,
        "copy_GBps": copy_gbps,
        "next_rows": {
            "attend_packed_values": {
                "ms": tat,
                "GBps": at_bytes / (tat * 1e-3) / 1e9,
                "what": "sum_t softmax(scores)_t * V_t over the packed V, 32 query heads",
            },
        },
        "roofline": {
            "bound": "hbm",
            "achieved": q_gbps,
            "peak": HBM_PEAK_GBPS,
            "unit": "GB/s",
            "frac": q_gbps / HBM_PEAK_GBPS,
            "traffic": profiled_traffic(["quantize_fast_kernel-llama-3.1-8b-32k.md",
                                         "quantize_mfma_kernel-llama-3.1-8b-32k.md"]),
            "traffic_unit": "bytes per launch (rocprofv3 FETCH_SIZE/WRITE_SIZE, copy-calibrated)",
            "kernel": "quantize: K launch quantize_fast_kernel (butterfly Hadamard, incl. "
                      "RoPE-table build), V launch quantize_mfma_kernel (matrix-core Hadamard)",
            "avg_launch_ms": tq / 2,
        },
    }
    if not args.no_decode_shape:
        out["score_decode_shape"] = qwen_decode_scores(args.steps, args.warmup, dev, stream)
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(w, args.cpu_sample_tokens, args.cpu_sample_slabs)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
