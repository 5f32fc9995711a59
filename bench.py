"""Benchmark of the E8 KV-cache hot path on one MI355X.

Headline (the metric): quantize + pack of the Llama-3.1-8B 32K-token cache
(32 layers x 8 KV heads x 32768 tokens x head_dim 128, fp16 K and V, k2v2
relaxed, one scale per head vector); `value` = tokens of the cache / median
time of one quantize call on K and V (HIP events on the kernels' stream).

One step = the whole path over that cache:
  1. quantize + pack K (RoPE removed, theta 5e5) and V      nq_quantize_kv
  2. dequantize K (RoPE re-applied) and V                   nq_dequantize_kv
  3. score one decode query per query head (32 heads, GQA 4) against the
     packed keys                                            nq_score_packed_keys
Also timed on their own: packed-value attention, the Mistral-7B (K3V2) and
Phi-3-mini (d = 96, strict) caches, scoring at the Qwen2.5-14B decode shape,
and the CPU oracle on a sample (cpu_baseline).  Inputs are synthetic
(e8_lattice_vector_amd.synth) and resident in HBM before timing starts.
Prints one JSON line.

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
    ap.add_argument("--steps", type=int, default=20)
    # the GPU's clocks settle over the first ~25 ms of sustained work: the
    # default warm-up (about 50 ms of steps) keeps the timed steps past that
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-decode-shape", action="store_true",
                    help="skip the scoring run at the Qwen2.5-14B decode shape")
    ap.add_argument("--no-other-shapes", action="store_true",
                    help="skip the Mistral-7B and Phi-3-mini caches")
    ap.add_argument("--cpu-sample-slabs", type=int, default=2,
                    help="slabs of the cache (all heads and tokens, K and V) the oracle runs on")
    return ap.parse_args()


SOURCES = ("nq_kernels.hip", "nq_device.h", "nq_exact.hip")


def source_sha() -> str:
    """sha256 of the quantize kernels' sources (the files whose code the
    committed counters measured), concatenated in a fixed order."""
    import hashlib

    h = hashlib.sha256()
    for f in SOURCES:
        with open(os.path.join(ROOT, "e8_lattice_vector_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def profiled_traffic(profiles):
    """HBM bytes per launch from committed rocprofv3 summaries (FETCH_SIZE and
    WRITE_SIZE, each scaled by the copy-kernel calibration), averaged over the
    summaries (one per launch of the step), or None when any is missing or the
    kernel sources have changed since its counters were taken."""
    import re

    vals = []
    for profile in profiles:
        try:
            text = open(os.path.join(ROOT, "profiles", profile)).read()
            sha = source_sha()
        except OSError:
            return None
        m_sha = re.search(r"kernel sources sha256: ([0-9a-f]{64})", text)
        m_tr = re.search(r"traffic_bytes_per_launch: (\d+)", text)
        if not m_sha or not m_tr or m_sha.group(1) != sha:
            return None
        vals.append(int(m_tr.group(1)))
    return round(sum(vals) / len(vals)) if vals else None


def median(xs):
    xs = sorted(xs)
    n = len(xs)
    return xs[n // 2] if n % 2 else 0.5 * (xs[n // 2 - 1] + xs[n // 2])


def _cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.lower().startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_job(job):
    """Worker: the oracle's quantize + pack of heads [h0, h1) of one slab of
    the cache (K with RoPE removal, or V), single-threaded; returns the
    oracle's seconds (input generation excluded)."""
    kind, w, slab, h0, h1 = job
    import torch
    from threadpoolctl import threadpool_limits

    from e8_lattice_vector_amd import synth
    from oracle import codec as oc

    torch.set_num_threads(1)
    x = synth.kv(kind, 1, w.H, w.T, w.d, w.theta if kind == "k" else 0.0, 0,
                 slab0=slab).numpy()[:, h0:h1]
    cdc = oc.Codec(w.d, w.bits_k if kind == "k" else w.bits_v, w.G, w.strict,
                   w.theta if kind == "k" else 0.0)
    with threadpool_limits(limits=1):
        t0 = time.perf_counter()
        oc.quantize(x, cdc, is_key=kind == "k")
        return time.perf_counter() - t0


def cpu_baseline(w, slabs, heads_per_job=1, max_procs=16):
    """The oracle, as it stands, on a bounded sample of the same workload:
    quantize + pack of K and V of `slabs` slabs (all heads, all tokens), in
    single-threaded worker processes over the host's cores (at most
    max_procs, the CPU share of one GPU)."""
    import multiprocessing as mp

    jobs = [(kind, w, s, h0, min(w.H, h0 + heads_per_job))
            for kind in ("k", "v") for s in range(slabs) for h0 in range(0, w.H, heads_per_job)]
    # no more processes than jobs: an idle process is not a core at work
    nproc = max(1, min(max_procs, os.cpu_count() or 1, len(jobs)))
    t0 = time.perf_counter()
    with mp.get_context("spawn").Pool(nproc) as pool:
        secs = pool.map(cpu_job, jobs, chunksize=1)
    wall = time.perf_counter() - t0
    busy = sum(secs)
    cache_tokens = w.T * slabs / w.S          # the sample is slabs / S of the cache
    return {
        "value": cache_tokens / (busy / nproc),
        "unit": "tokens/s",
        "cores": nproc,
        "kind": "oracle",
        "cpu_model": _cpu_model(),
        "nproc": os.cpu_count(),
        "sample": f"{slabs} of {w.S} slabs x {w.H} heads x {w.T} tokens, K and V quantize+pack "
                  f"(fp64 oracle), {len(jobs)} jobs on {nproc} single-threaded processes: "
                  f"{busy:.1f} s of oracle time ({wall:.1f} s wall incl. input generation); "
                  f"tokens/s = sampled tokens / (oracle seconds / processes)",
    }


def timed(fn, steps, warmup, stream, min_warm_s=0.05):
    """Median milliseconds of `fn` over `steps` calls (HIP events on the
    stream the kernels run on), after `warmup` calls and at least
    `min_warm_s` seconds of untimed calls: after a change of workload the
    GPU's clocks settle over tens of milliseconds (a memory-bound kernel
    timed after 20 short calls ran up to 40 % slower than after 50 ms)."""
    import torch

    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < min_warm_s:
        for _ in range(4):
            fn()
        torch.cuda.synchronize()
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(steps)]
    torch.cuda.synchronize()
    for e in ev:
        e[0].record(stream)
        fn()
        e[1].record(stream)
    torch.cuda.synchronize()
    return median([e[0].elapsed_time(e[1]) for e in ev])


def other_workload(wname, steps, warmup, dev, stream, Hq):
    """Quantize + pack, dequantize and (Hq > 0) packed-key scoring of one of
    the other caches of the pages' models, each timed on its own."""
    import torch

    from e8_lattice_vector_amd import nq, synth, workloads

    w = workloads.ALL[wname]
    cfg = nq.Config(w.d, w.bits_k, w.bits_v, w.G,
                    nq.PARITY_STRICT if w.strict else nq.PARITY_RELAXED, nq.DTYPE_F16, w.theta)
    k, v = synth.workload_inputs(w, seed=0, device=dev)
    pk = nq.alloc_packed(cfg, False, w.S, w.H, w.T, dev)
    pv = nq.alloc_packed(cfg, True, w.S, w.H, w.T, dev)
    ws = nq.alloc_workspace(cfg, w.S, w.H, w.T, dev)
    kd, vd = torch.empty_like(k), torch.empty_like(v)
    tq = timed(lambda: nq.quantize_kv(cfg, k, v, pk=pk, pv=pv, workspace=ws), steps, warmup,
               stream)
    tdq = timed(lambda: nq.dequantize_kv(cfg, pk, pv, w.S, w.H, w.T, k_out=kd, v_out=vd,
                                         workspace=ws), steps, warmup, stream)
    nv = w.S * w.H * w.T
    fp16 = 2 * nv * w.d * 2
    packed = pk.nbytes() + pv.nbytes()
    table = w.T * (w.d // 2) * 8 if w.theta > 0 else 0
    qb = fp16 + packed + table
    out = {
        "shape": f"{w.S} slabs x {w.H} KV heads x {w.T} tokens x d {w.d}",
        "codec": f"k{w.bits_k}v{w.bits_v} {'strict' if w.strict else 'relaxed'}, scale per "
                 f"{w.G or 'head vector'}, rope_theta {w.theta:g}",
        "quantize": {"ms": tq, "tokens_per_s": w.T / (tq * 1e-3),
                     "hbm_GBps": qb / (tq * 1e-3) / 1e9,
                     "frac_hbm_peak": qb / (tq * 1e-3) / 1e9 / HBM_PEAK_GBPS, "bytes": qb},
        "dequantize": {"ms": tdq, "tokens_per_s": w.T / (tdq * 1e-3),
                       "hbm_GBps": qb / (tdq * 1e-3) / 1e9,
                       "frac_hbm_peak": qb / (tdq * 1e-3) / 1e9 / HBM_PEAK_GBPS},
    }
    if Hq:
        q = synth.queries(w.S, Hq, w.d, 0, dev)
        sc = torch.empty((w.S, Hq, w.T), dtype=torch.float32, device=dev)
        tsc = timed(lambda: nq.score_packed_keys(cfg, pk, q, w.S, w.H, w.T, scores=sc), steps,
                    warmup, stream)
        sb = pk.nbytes() + q.numel() * 2 + sc.numel() * 4
        out["score"] = {"ms": tsc, "query_heads": Hq, "keys_per_s": nv / (tsc * 1e-3),
                        "hbm_GBps": sb / (tsc * 1e-3) / 1e9,
                        "frac_hbm_peak": sb / (tsc * 1e-3) / 1e9 / HBM_PEAK_GBPS}
    del k, v, pk, pv, ws, kd, vd
    torch.cuda.empty_cache()
    return out


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
    ms = timed(lambda: nq.score_packed_keys(cfg, pk, q, w.S, w.H, w.T, scores=sc), steps,
               warmup, stream)
    keys = w.S * w.H * w.T
    nbytes = pk.nbytes() + q.numel() * 2 + sc.numel() * 4
    del pk, ws, q, sc
    return {
        "workload": w.name,
        "ms": ms,
        "keys_per_s": keys / (ms * 1e-3),
        "GBps": nbytes / (ms * 1e-3) / 1e9,
        "frac_hbm_peak": nbytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBPS,
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
        nq.quantize_kv(cfg, k, v, pk=pk, pv=pv, workspace=ws)
        if ev is not None:
            ev[1].record(stream)
        nq.dequantize_kv(cfg, pk, pv, w.S, w.H, w.T, k_out=kd, v_out=vd, workspace=ws)
        if ev is not None:
            ev[2].record(stream)
        nq.score_packed_keys(cfg, pk, q, w.S, w.H, w.T, scores=scores)
        if ev is not None:
            ev[3].record(stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    events = [[torch.cuda.Event(enable_timing=True) for _ in range(4)]
              for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(events[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    seg = [[e[j].elapsed_time(e[j + 1]) for j in range(3)] for e in events]
    tq, tdq, tsc = (median([s_[j] for s_ in seg]) for j in range(3))
    tstep = median([e[0].elapsed_time(e[3]) for e in events])
    ms_step = wall * 1e3 / args.steps
    # the two tensors' launches, each in a call of its own
    tk = timed(lambda: nq.quantize_kv(cfg, k, None, pk=pk, workspace=ws), args.steps,
               args.warmup, stream)
    tv = timed(lambda: nq.quantize_kv(cfg, None, v, pv=pv, workspace=ws), args.steps,
               args.warmup, stream)
    # scoring back to back: inside the step it follows dequantize, whose
    # 4.2 GB of output are still being written back from the caches
    tsa = timed(lambda: nq.score_packed_keys(cfg, pk, q, w.S, w.H, w.T, scores=scores),
                args.steps, args.warmup, stream)

    nv = w.S * w.H * w.T
    fp16_bytes = nv * w.d * 2
    vec_bytes = pk.nbytes() // nv
    packed = nv * vec_bytes
    table = w.T * (w.d // 2) * 8
    k_bytes = fp16_bytes + packed + table                 # K launch, + RoPE table read
    v_bytes = fp16_bytes + packed
    q_bytes = k_bytes + v_bytes
    dq_bytes = q_bytes
    sc_bytes = packed + w.S * Hq * w.d * 2 + w.S * Hq * w.T * 4
    q_gbps = q_bytes / (tq * 1e-3) / 1e9

    # next row: value half of decode attention on the packed V, weights =
    # softmax of the step's scores (timed on its own, not part of the step)
    wts = torch.softmax(scores, dim=-1).contiguous()
    att = torch.empty((w.S, Hq, w.d), dtype=torch.float32, device=dev)
    tat = timed(lambda: nq.attend_packed_values(cfg, pv, wts, w.S, w.H, w.T, out=att),
                args.steps, args.warmup, stream)
    at_bytes = packed + w.S * Hq * w.T * 4 + w.S * Hq * w.d * 4
    del wts, att

    # plain device copy of 4 GiB (context only, not a ceiling)
    src = torch.empty(1 << 31, dtype=torch.float16, device=dev)
    dst = torch.empty_like(src)
    tcp = timed(lambda: dst.copy_(src), 5, 1, stream)
    copy_gbps = 2 * src.numel() * 2 / (tcp * 1e-3) / 1e9
    del src, dst, k, v, kd, vd, pk, pv, ws, q, scores
    torch.cuda.empty_cache()

    out = {
        "metric": "KV quantize+pack tokens/s and HBM GB/s (% of peak), Llama-3.1-8B shape, 1 GPU",
        "value": w.T / (tq * 1e-3),
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
            "value": "tokens of the 32K cache / median time of one nq_quantize_kv call on K "
                     "and V (RoPE table, fp32 kernels, fp64 near-tie passes)",
            "storage": "fp16 in/out, 36 B per packed vector",
            "arithmetic": "fp32 (fp64 for near-tie vectors); scoring and attention multiply on "
                          "bf16 matrix cores with exact code values and the fp32 query / "
                          "weight split into two bf16 parts (hi + lo), fp32 accumulation",
        },
        "quantize": {
            "tokens_per_s": w.T / (tq * 1e-3),
            "ms": tq,
            "hbm_GBps": q_gbps,
            "fp16_kv_GBps": 2 * fp16_bytes / (tq * 1e-3) / 1e9,
            "frac_hbm_peak": q_gbps / HBM_PEAK_GBPS,
            "bytes": q_bytes,
        },
        "step": {
            "ms_median_events": tstep,
            "ms_wall": ms_step,
            "tokens_per_s": w.T / (tstep * 1e-3),
        },
        "kernels_ms_median": {"quantize_kv (K and V in one call)": tq,
                              "quantize_k alone (rope table, fp32 kernel, fp64 pass)": tk,
                              "quantize_v alone (counter clear, fp32 kernel, fp64 pass)": tv,
                              "dequantize_kv (K, V)": tdq,
                              "score (in the step, after dequantize)": tsc,
                              "score alone (back to back)": tsa},
        "frac_hbm_peak": {"quantize_k": k_bytes / (tk * 1e-3) / 1e9 / HBM_PEAK_GBPS,
                          "quantize_v": v_bytes / (tv * 1e-3) / 1e9 / HBM_PEAK_GBPS,
                          "dequantize_kv": dq_bytes / (tdq * 1e-3) / 1e9 / HBM_PEAK_GBPS,
                          "score_in_step": sc_bytes / (tsc * 1e-3) / 1e9 / HBM_PEAK_GBPS,
                          "score_alone": sc_bytes / (tsa * 1e-3) / 1e9 / HBM_PEAK_GBPS},
        "dequantize_GBps": dq_bytes / (tdq * 1e-3) / 1e9,
        "score_GBps": sc_bytes / (tsa * 1e-3) / 1e9,
        "copy_GBps_context": copy_gbps,
        "next_rows": {
            "attend_packed_values": {
                "ms": tat,
                "GBps": at_bytes / (tat * 1e-3) / 1e9,
                "frac_hbm_peak": at_bytes / (tat * 1e-3) / 1e9 / HBM_PEAK_GBPS,
                "what": "sum_t softmax(scores)_t * V_t over the packed V, 32 query heads",
            },
        },
        "roofline": {
            "bound": "hbm",
            "achieved": q_gbps,
            "peak": HBM_PEAK_GBPS,
            "unit": "GB/s",
            "frac": q_gbps / HBM_PEAK_GBPS,
            "traffic": profiled_traffic(["quantize_pair_kernel-llama-3.1-8b-32k.md",
                                         "quantize_mfma_kernel-llama-3.1-8b-32k.md"]),
            "traffic_unit": "bytes per launch (rocprofv3 FETCH_SIZE/WRITE_SIZE, copy-calibrated)",
            "kernel": "quantize (one call on K and V): RoPE-table build, K launch "
                      "quantize_pair_kernel (RoPE removal fused with the stride-64 butterfly, "
                      "DPP butterflies), V launch quantize_mfma_kernel (matrix-core Hadamard), "
                      "the fp64 near-tie pass after each",
            "algorithmic_bytes_per_launch": {"K": k_bytes, "V": v_bytes},
            "avg_launch_ms": tq / 2,
        },
    }
    if not args.no_other_shapes:
        out["other_workloads"] = {
            "mistral-7b": other_workload("mistral-7b", args.steps, args.warmup, dev, stream, 32),
            "phi-3-mini": other_workload("phi-3-mini", args.steps, args.warmup, dev, stream, 0),
        }
    if not args.no_decode_shape:
        out["score_decode_shape"] = qwen_decode_scores(args.steps, args.warmup, dev, stream)
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(w, args.cpu_sample_slabs)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
