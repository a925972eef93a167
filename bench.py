"""Benchmark of the KV-cache transform-and-quantize hot path on one MI355X.

One step = one pass of the whole path over the long-context decode workload, inputs
resident in HBM: quantize (fp16 K cache [64 x 32768, 8, 128], randomized Hadamard 128,
nsep+pchan INT4, B = 128) -> dequantize (back to fp16) -> decode scores from the packed
cache (fp16 queries [64, 32, 128], GQA 4, fp32 scores [64, 32, 32768]).

Prints one JSON line.  value = algorithmic bytes of a step / step time (GB/s); the
roofline entry is the dominant kernel (quantize) timed with HIP events on the stream it
runs on; cpu_baseline is the fp64 oracle on a bounded sample on the host cores.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, ~8 TB/s
WORKLOAD = "long_context_decode"


def percentile(sorted_vals, p):
    """Linear-interpolated percentile of an ascending list."""
    if not sorted_vals:
        return float("nan")
    k = (len(sorted_vals) - 1) * p / 100.0
    i = int(k)
    j = min(i + 1, len(sorted_vals) - 1)
    return sorted_vals[i] + (sorted_vals[j] - sorted_vals[i]) * (k - i)


def time_calls(torch, fn, stream, steps, warmup, before=None):
    """Median, p10 and p90 (us) of `steps` calls of fn, each bracketed by HIP events on `stream`
    after `warmup` untimed calls; before() (a cache flush) runs ahead of each timed call, outside
    the events."""
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    for e0, e1 in ev:
        if before is not None:
            before()
        e0.record(stream)
        fn()
        e1.record(stream)
    torch.cuda.synchronize()
    t = sorted(e0.elapsed_time(e1) * 1e3 for e0, e1 in ev)
    return {"us": round(percentile(t, 50), 2), "us_p10": round(percentile(t, 10), 2), "us_p90": round(percentile(t, 90), 2)}


def algorithmic_bytes(w, q_heads):
    """Every input read once and every output written once (bytes per kernel launch)."""
    n = w.seqs * w.tokens * w.heads * w.head_dim            # K elements
    tok = w.seqs * w.tokens * w.heads                        # (token, head) vectors
    codes = n // 2
    norms = 2 * tok
    scales = 2 * (w.seqs * w.tokens // w.block_tokens) * w.heads * w.head_dim
    signs = w.heads * w.head_dim
    x = 2 * n
    q = 2 * w.seqs * q_heads * w.head_dim
    scores = 4 * w.seqs * q_heads * w.tokens
    out = 4 * w.seqs * q_heads * w.head_dim
    return {"quantize": x + signs + codes + norms + scales,
            "dequantize": codes + norms + scales + signs + x,
            "score_decode": q + signs + codes + norms + scales + scores,
            # fused decode attention (a "next" row, outside the step): K and V caches in, fp32 out
            "attention_decode": q + 2 * (signs + codes + norms + scales) + out,
            # the NSN variant: s1 and s2 per token, offsets shaped like the per-channel scales
            "quantize_nsn": x + signs + codes + 2 * norms + 2 * scales,
            "dequantize_nsn": codes + 2 * norms + 2 * scales + signs + x,
            "score_decode_nsn": q + signs + codes + 2 * norms + 2 * scales + scores,
            "elements": n,
            # the kernels' inputs alone (the "input GB/s" figure)
            "inputs": {"quantize": x + signs, "dequantize": codes + norms + scales + signs,
                       "score_decode": q + signs + codes + norms + scales}}


TRAFFIC_FILE = os.path.join(ROOT, "profiles", "long_context_hbm_traffic.md")


def source_digest(sources: str):
    """SHA-256 over the listed source files (comma-separated, repo-relative, in order), or None if
    one is missing."""
    import hashlib
    h = hashlib.sha256()
    for rel in sources.split(","):
        path = os.path.join(ROOT, rel)
        if not os.path.exists(path):
            return None
        h.update(open(path, "rb").read())
    return h.hexdigest()


def measured_traffic(kernel: str):
    """HBM bytes per launch of `kernel` from the committed rocprofv3 FETCH_SIZE / WRITE_SIZE summary,
    or None when there is none or a source of the kernel (its file and the headers it includes) has
    changed since it was taken."""
    if not os.path.exists(TRAFFIC_FILE):
        return None
    for line in open(TRAFFIC_FILE):
        f = line.split()
        if len(f) == 5 and f[0] == "traffic" and f[1] == kernel:
            kv = dict(x.split("=", 1) for x in f[2:])
            if source_digest(kv["source"]) == kv["sha256"]:
                return int(kv["bytes_per_launch"])
    return None


def _oracle_inputs(w, s):
    from activation_quantization_amd import synth
    return (synth.make_x(w, seq_range=(s, s + 1)).double().numpy(),
            synth.make_q(w, seq_range=(s, s + 1)).double().numpy())


def _oracle_run(w, signs, x, q):
    """One sequence of the long-context workload through the fp64 oracle: quantize, dequantize,
    decode scores (one thread)."""
    import oracle
    sp = oracle.Spec(1, w.tokens, w.heads, w.head_dim, 4, "nsep_pchan", w.block_tokens, w.hadamard)
    r = oracle.quantize(x, sp, signs)
    kh = oracle.dequantize(r.packed, r.norms16, r.scales16, sp, signs)
    oracle.score_decode(q, kh, sp)


def _oracle_worker(name, seq_ids, barrier, results):
    """A process of the all-core leg: generate its sequences, wait for every worker, then run the
    oracle on them and report the seconds that took."""
    import threadpoolctl
    from activation_quantization_amd import synth
    w = synth.WORKLOADS[name]
    signs = synth.make_signs(w).numpy()
    inputs = [_oracle_inputs(w, s) for s in seq_ids]
    with threadpoolctl.threadpool_limits(1):
        barrier.wait()
        t0 = time.perf_counter()
        for x, q in inputs:
            _oracle_run(w, signs, x, q)
        results.put(time.perf_counter() - t0)


def _host_info():
    model = "unknown"
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    return {"nproc": os.cpu_count(), "cpu_model": model}


def cpu_baseline(w, seqs_one: int, seqs_all: int, workers: int):
    """The fp64 oracle (as it stands) on a bounded sample of the workload's sequences: seqs_one
    sequences on one thread, then seqs_all sequences split over `workers` single-threaded processes
    (the host's cores; sequences are independent).  Only the oracle's work is timed (inputs are
    generated first).  GB/s counts the step's algorithmic bytes."""
    import multiprocessing as mp
    import threadpoolctl
    from activation_quantization_amd import synth
    b = algorithmic_bytes(synth.scaled(w, seqs=1), w.q_heads)
    seq_bytes = b["quantize"] + b["dequantize"] + b["score_decode"]
    signs = synth.make_signs(w).numpy()
    t_one = 0.0
    with threadpoolctl.threadpool_limits(1):
        for s in range(seqs_one):
            x, q = _oracle_inputs(w, s)
            t0 = time.perf_counter()
            _oracle_run(w, signs, x, q)
            t_one += time.perf_counter() - t0
    out = {"value": round(seqs_one * seq_bytes / t_one / 1e9, 4), "unit": "GB/s", "cores": 1, "kind": "oracle",
           **_host_info(),
           "one_thread": {"GB/s": round(seqs_one * seq_bytes / t_one / 1e9, 4), "seqs": seqs_one, "s": round(t_one, 1)}}
    if workers > 1 and seqs_all >= workers:
        ctx = mp.get_context("spawn")          # fresh interpreters: nothing of this process's GPU state
        barrier, results = ctx.Barrier(workers + 1), ctx.Queue()
        procs = [ctx.Process(target=_oracle_worker, args=(WORKLOAD, list(range(i, seqs_all, workers)), barrier, results))
                 for i in range(workers)]
        for p in procs:
            p.start()
        barrier.wait()
        t0 = time.perf_counter()
        busy = sum(results.get() for _ in procs)
        wall = time.perf_counter() - t0
        for p in procs:
            p.join()
        out["all_cores"] = {"GB/s": round(seqs_all * seq_bytes / wall / 1e9, 4), "seqs": seqs_all,
                            "workers": workers, "s": round(wall, 1), "busy_cores": round(busy / wall, 1)}
        out["value"] = out["all_cores"]["GB/s"]
        out["cores"] = workers
    out["sample"] = (f"{seqs_one} sequence(s) on one thread, then {seqs_all} split over {workers} single-threaded "
                     f"processes, of {w.seqs} sequences ({w.tokens * w.heads * w.head_dim} K elements each), "
                     "quantize+dequantize+score, fp64 numpy, oracle time only; value = the all-core figure")
    return out


def config_bytes(w, bits_mode):
    """Algorithmic bytes of quantize / dequantize for workload w (input dtype 2 bytes)."""
    n = w.seqs * w.tokens * w.heads * w.head_dim
    tok = w.seqs * w.tokens * w.heads
    per_channel = "pchan" in w.mode
    nsep = w.mode in ("nsep", "nsep_pchan")
    scales = 2 * ((w.seqs * w.tokens // w.block_tokens) * w.heads * w.head_dim if per_channel else tok)
    norms = 2 * tok if nsep else 0
    signs = w.heads * w.head_dim if w.hadamard else 0
    q = 2 * n + signs + n // 2 + norms + scales
    return q, q


def stream_decode(torch, kvq, d, w, q, k_cache, v_cache, signs, att_out, ws, stream, dev, steps, warmup):
    """The decode loop's streaming append and attention over the streamed cache.

    Every sequence of the K and V caches starts at T - B cached tokens (whole blocks); one decode
    step appends one new token per sequence to each cache (one kvq_append_kv call), so a cycle of B steps fills the
    full-precision residual and flushes it (the B-th append quantizes it into the cache).  Then
    decode attention over T - 1 tokens: T - B from the packed caches and B - 1 from the residuals.
    New tokens are seeded N(0, 1) fp16 (the append's cost does not depend on their values)."""
    B, T, S = w.block_tokens, w.tokens, w.seqs
    gen = torch.Generator(device="cpu").manual_seed(7)
    xk = torch.randn((S, B, w.heads, w.head_dim), generator=gen).half().to(dev)
    xv = torch.randn((S, B, w.heads, w.head_dim), generator=gen).half().to(dev)
    steps_k = [xk[:, i:i + 1].contiguous() for i in range(B)]
    steps_v = [xv[:, i:i + 1].contiguous() for i in range(B)]
    rk, rv = kvq.alloc_residual(d, dev), kvq.alloc_residual(d, dev)

    def cycle():
        n = T - B
        for i in range(B):
            n = kvq.append_kv(d, n, steps_k[i], steps_v[i], rk, rv, k_cache, v_cache, signs, signs, stream=stream)
        return n

    cycle()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    cycle()
    e1.record(stream)
    torch.cuda.synchronize()
    cycle_us = e0.elapsed_time(e1) * 1e3
    tok_bytes = S * w.heads * w.head_dim * 2                     # one new token per sequence, fp16
    blk_bytes = S * B * w.heads * w.head_dim * 2                 # a full residual
    packed = S * B * w.heads * (w.head_dim // 2 + 2) + S * w.heads * w.head_dim * 2
    cycle_bytes = 2 * (B * 2 * tok_bytes + blk_bytes + packed)   # K and V: copies in/out, one flush
    rows = {"append_decode_step": {"us_per_step": round(cycle_us / B, 2), "appends_per_step": 2, "calls_per_step": 1,
                                   "tokens_per_append": S, "cycle_steps": B, "cycle_us": round(cycle_us, 1),
                                   "cycle_bytes": cycle_bytes,
                                   "GB/s": round(cycle_bytes / (cycle_us * 1e-6) / 1e9, 1)}}
    n = T - 1
    t = time_calls(torch, lambda: kvq.attention_decode_stream(d, n, q, k_cache, rk, v_cache, rv, signs, signs,
                                                              out=att_out, workspace=ws, stream=stream),
                   stream, steps, warmup)
    nb = algorithmic_bytes(w, w.q_heads)["attention_decode"]
    gbs = nb / (t["us"] * 1e-6) / 1e9
    rows["attention_decode_stream"] = {**t, "tokens_cached": n, "residual_tokens": B - 1, "GB/s": round(gbs, 1),
                                       "frac_hbm": round(gbs / HBM_PEAK_GBS, 4)}
    return rows


NSN_KERNELS = ("quantize_nsn", "dequantize_nsn", "score_decode_nsn")


def nsn_kernels(torch, kvq, w, x, q, signs, y, stream, dev, steps, warmup, only=None):
    """The NSN variant (normalize, shift, normalize before the per-channel quantizer) on the same
    cache: quantize, dequantize to fp16, decode score, each timed with HIP events on the stream
    (`only`: just that one, after an untimed quantize that fills the cache it reads)."""
    d = kvq.Desc(w.seqs, w.tokens, w.heads, w.head_dim, 4, "nsn_pchan", w.block_tokens, w.hadamard, torch.float16)
    out = kvq.alloc_nsn(d, dev)
    scores = torch.empty((w.seqs, w.q_heads, w.tokens), dtype=torch.float32, device=dev)
    nbytes = algorithmic_bytes(w, w.q_heads)
    calls = {"quantize_nsn": lambda: kvq.quantize_nsn(d, x, signs, out=out, stream=stream),
             "dequantize_nsn": lambda: kvq.dequantize_nsn(d, *out, signs, out=y, stream=stream),
             "score_decode_nsn": lambda: kvq.score_decode_nsn(d, q, *out, signs, out=scores, stream=stream)}
    rows = {}
    if only is not None:
        calls["quantize_nsn"]()
        calls = {only: calls[only]}
    for name, fn in calls.items():
        t = time_calls(torch, fn, stream, steps, warmup)
        gbs = nbytes[name] / (t["us"] * 1e-6) / 1e9
        rows[name] = {**t, "bytes": nbytes[name], "GB/s": round(gbs, 1), "frac_hbm": round(gbs / HBM_PEAK_GBS, 4),
                      "in_step": False}
    del out, scores
    return rows


RRS_KERNELS = ("rrs_smooth_scales", "rrs_quantize_act", "rrs_quantize_weights", "rrs_gemm")
INT8_MFMA_PEAK_TOPS = 5000.0     # MI355X dense int8 matrix throughput, TOP/s


def rrs_kernels(torch, kvq, synth, dev, steps, warmup, only=None):
    """The RRS activation path into an INT4 GEMM on the activation workload: X [8192, 4096] bf16
    (the activation generator) times synthetic weights W [4096, 4096] bf16, Hadamard 128 with the
    workload's signs, INT4.  Each kernel timed with HIP events on the stream; the GEMM against the
    int8 matrix-core peak (2 N M K integer operations), the others against HBM."""
    wa = synth.WORKLOADS["activation_4096"]
    n, k = wa.tokens, wa.head_dim
    m = 4096
    x = synth.make_x(wa).reshape(n, k).to(dev)
    w = synth.make_weights(m, k, seed=11, dtype="bf16").to(dev)
    sg = synth.make_signs(wa).reshape(k).to(dev)
    stream = torch.cuda.current_stream()
    s = kvq.rrs_smooth_scales(x, sg, 128, stream=stream)
    xq = kvq.rrs_quantize_act(x, sg, 128, s, 4, stream=stream)
    wq = kvq.rrs_quantize_weights(w, sg, 128, 4, stream=stream)
    y = kvq.rrs_gemm(*xq, *wq, s, stream=stream)
    calls = {"rrs_smooth_scales": lambda: kvq.rrs_smooth_scales(x, sg, 128, out=s, stream=stream),
             "rrs_quantize_act": lambda: kvq.rrs_quantize_act(x, sg, 128, s, 4, out=xq, stream=stream),
             "rrs_quantize_weights": lambda: kvq.rrs_quantize_weights(w, sg, 128, 4, out=wq, stream=stream),
             "rrs_gemm": lambda: kvq.rrs_gemm(*xq, *wq, s, out=y, stream=stream)}
    nbytes = {"rrs_smooth_scales": 2 * n * k + k + 4 * (k // 128),
              "rrs_quantize_act": 2 * n * k + k + 4 * (k // 128) + n * k // 2 + 2 * n,
              "rrs_quantize_weights": 2 * m * k + k + m * k // 2 + 2 * m,
              "rrs_gemm": n * k // 2 + 2 * n + m * k // 2 + 2 * m + 4 * (k // 128) + 4 * n * m}
    if only is not None:
        calls = {only: calls[only]}
    rows = {}
    for name, fn in calls.items():
        t = time_calls(torch, fn, stream, steps, warmup)
        us = t["us"]
        gbs = nbytes[name] / (us * 1e-6) / 1e9
        row = {**t, "bytes": nbytes[name], "GB/s": round(gbs, 1), "frac_hbm": round(gbs / HBM_PEAK_GBS, 4),
               "shape": [n, m, k], "in_step": False}
        if name == "rrs_gemm":
            tops = 2.0 * n * m * k / (us * 1e-6) / 1e12
            row.update({"TOP/s": round(tops, 1), "frac_int8_mfma": round(tops / INT8_MFMA_PEAK_TOPS, 4)})
        rows[name] = row
    del x, w, y, xq, wq, s
    return rows


def other_configs(torch, kvq, synth, dev, steps, warmup, only=None):
    """Quantize and dequantize of the other workloads at every bit width they name (K and V for the
    Qwen-like layer), each call after a 512 MiB read that evicts L2 and the MALL (the events bracket
    the kernel only).  A read, not a write: a written flush buffer leaves dirty lines whose
    write-back would land inside the timed kernel."""
    flush = torch.ones(128 << 20, dtype=torch.int32, device=dev)
    stream = torch.cuda.current_stream()
    rows = []
    names = ("qwen_kv_layer", "batched_hadamard", "activation_4096")
    if only is not None:                                   # "<workload>/<kernel>"
        names = (only.split("/")[0],)
    for name in names:
        w = synth.WORKLOADS[name]
        dt = synth.torch_dtype(w)
        sg = synth.make_signs(w).to(dev) if w.hadamard else None
        for tensor_id in range(w.tensors):
            x = synth.make_x(w, tensor_id=tensor_id).to(dev)
            y = torch.empty_like(x)
            for bits in w.bits:
                d = kvq.Desc(w.seqs, w.tokens, w.heads, w.head_dim, bits, w.mode, w.block_tokens, w.hadamard, dt)
                out = kvq.alloc_outputs(d, dev)
                qb, db = config_bytes(w, w.mode)
                for kname, fn, nbytes in (("quantize", lambda: kvq.quantize(d, x, sg, out=out, stream=stream), qb),
                                          ("dequantize", lambda: kvq.dequantize(d, *out, sg, out_dtype=dt, out=y,
                                                                                 stream=stream), db)):
                    if only is not None and only.split("/")[1] != kname:
                        if kname == "quantize":
                            fn()                           # the codes the dequantize reads
                        continue
                    t = time_calls(torch, fn, stream, steps, warmup, before=flush.sum)
                    gbs = nbytes / (t["us"] * 1e-6) / 1e9
                    rows.append({"workload": name, "tensor": "KV"[tensor_id] if w.tensors == 2 else "x", "kernel": kname,
                                 "shape": [w.seqs, w.tokens, w.heads, w.head_dim], "mode": w.mode, "bits": bits,
                                 "hadamard": w.hadamard, "dtype": w.dtype, **t, "bytes": nbytes, "GB/s": round(gbs, 1),
                                 "frac_hbm": round(gbs / HBM_PEAK_GBS, 4)})
                del out
            del x, y
    return rows


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--cpu-seqs", type=int, default=2,
                    help="sequences the oracle baseline times on one thread (0 = skip the baseline)")
    ap.add_argument("--cpu-seqs-all", type=int, default=16,
                    help="sequences the oracle baseline times over all host cores")
    ap.add_argument("--cpu-workers", type=int, default=0,
                    help="processes for the all-core leg (0 = the host's cores, at most 16)")
    ap.add_argument("--only", choices=("quantize", "dequantize", "score_decode", "attention_decode") + NSN_KERNELS
                    + RRS_KERNELS,
                    default=None,
                    help="run just this kernel in each step (for profiler runs; no cpu baseline)")
    ap.add_argument("--config-only", default=None,
                    help="time just <workload>/<kernel> of the other workloads (e.g. activation_4096/quantize; "
                         "for profiler runs) and exit")
    ap.add_argument("--other-configs", type=int, default=1,
                    help="also time quantize / dequantize of the other workloads (1 = yes), after an L2/MALL flush")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="time a plain device-to-device copy of the fp16 input (the reference kernel "
                         "for scaling rocprofv3 FETCH_SIZE / WRITE_SIZE) and exit")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py runs on one GPU only: the quantize / dequantize / decode-score path has no "
              "cross-GPU step (sharding by sequence or KV head needs no exchange); use --gpus 1.",
              file=sys.stderr)
        sys.exit(2)

    import torch
    from activation_quantization_amd import kvq, synth

    w = synth.WORKLOADS[WORKLOAD]
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.config_only:
        rows = other_configs(torch, kvq, synth, dev, args.steps, args.warmup, only=args.config_only)
        print(json.dumps({"profile_only": args.config_only, "rotation": os.environ.get("KVQ_ROTATION", "mfma"),
                          "rows": rows}), flush=True)
        return
    d = kvq.Desc(w.seqs, w.tokens, w.heads, w.head_dim, 4, "nsep_pchan", w.block_tokens, w.hadamard, torch.float16)
    print(f"[bench] generating {WORKLOAD} x {w.seqs}x{w.tokens}x{w.heads}x{w.head_dim} fp16", file=sys.stderr, flush=True)
    t0 = time.time()
    x = synth.make_x(w, pin=True).to(dev, non_blocking=True)
    signs = synth.make_signs(w).to(dev)
    q = synth.make_q(w).to(dev)
    codes, norms, scales = kvq.alloc_outputs(d, dev)
    y = torch.empty_like(x)
    scores = torch.empty((w.seqs, w.q_heads, w.tokens), dtype=torch.float32, device=dev)
    torch.cuda.synchronize()
    print(f"[bench] inputs resident in HBM after {time.time() - t0:.1f} s", file=sys.stderr, flush=True)

    stream = torch.cuda.current_stream()
    if args.only in RRS_KERNELS:
        kernels = rrs_kernels(torch, kvq, synth, dev, args.steps, args.warmup, only=args.only)
        print(json.dumps({"profile_only": args.only, "kernels": kernels, "steps": args.steps}), flush=True)
        return
    if args.only in NSN_KERNELS:
        kernels = nsn_kernels(torch, kvq, w, x, q, signs, y, stream, dev, args.steps, args.warmup, only=args.only)
        print(json.dumps({"profile_only": args.only, "kernels": kernels, "steps": args.steps}), flush=True)
        return
    if args.calibrate_copy:
        del y
        y = torch.empty_like(x)
        for _ in range(args.warmup):
            y.copy_(x)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(args.steps):
            y.copy_(x)
        e1.record(stream)
        torch.cuda.synchronize()
        us = e0.elapsed_time(e1) * 1e3 / args.steps
        nbytes = x.numel() * x.element_size()
        print(json.dumps({"calibrate_copy": {"bytes_read": nbytes, "bytes_written": nbytes, "us": round(us, 2),
                                             "GB/s": round(2 * nbytes / (us * 1e-6) / 1e9, 1)}}), flush=True)
        return
    names = ("quantize", "dequantize", "score_decode")
    run = {n: args.only in (None, n) for n in names}
    run_attn = args.only in (None, "attention_decode")
    if args.only == "attention_decode":
        run = {n: False for n in names}

    if args.only not in (None, "quantize"):
        kvq.quantize(d, x, signs, out=(codes, norms, scales), stream=stream)   # the cache it reads

    def step(ev=None):
        if ev: ev[0].record(stream)
        if run["quantize"]:
            kvq.quantize(d, x, signs, out=(codes, norms, scales), stream=stream)
        if ev: ev[1].record(stream)
        if run["dequantize"]:
            kvq.dequantize(d, codes, norms, scales, signs, out=y, stream=stream)
        if ev: ev[2].record(stream)
        if run["score_decode"]:
            kvq.score_decode(d, q, codes, norms, scales, signs, out=scores, stream=stream)
        if ev: ev[3].record(stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    events = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(args.steps)]
    t_start = time.perf_counter()
    for i in range(args.steps):
        step(events[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_start
    # per kernel: median, p10 and p90 over the timed steps (HIP events on the stream the kernels run on)
    samples = {n: sorted(e[k].elapsed_time(e[k + 1]) for e in events) for k, n in enumerate(names)}
    per_kernel_ms = {n: percentile(v, 50) for n, v in samples.items()}
    gpu_step_ms = percentile(sorted(events[i][0].elapsed_time(events[i][3]) for i in range(args.steps)), 50)
    ms_per_step = wall * 1e3 / args.steps

    b = algorithmic_bytes(w, w.q_heads)
    step_bytes = sum(b[n] for n in names if run[n])

    # fused decode attention over a K cache and a V cache of the same statistics (timed apart from
    # the step: it is a "next" row, not one of the step's kernels)
    attn_us = None
    if run_attn:
        if not run["quantize"]:
            kvq.quantize(d, x, signs, out=(codes, norms, scales), stream=stream)
        xv = synth.make_x(w, tensor_id=1, pin=True).to(dev, non_blocking=True)
        vcache = kvq.alloc_outputs(d, dev)
        kvq.quantize(d, xv, signs, out=vcache, stream=stream)
        del xv
        att_out = torch.empty((w.seqs, w.q_heads, w.head_dim), dtype=torch.float32, device=dev)
        ws = torch.empty(kvq.attention_workspace_bytes(d, w.q_heads) // 4, dtype=torch.float32, device=dev)
        kc = (codes, norms, scales)
        attn_t = time_calls(torch, lambda: kvq.attention_decode(d, q, kc, vcache, signs, signs, out=att_out,
                                                                 workspace=ws, stream=stream),
                            stream, args.steps, args.warmup)
        attn_us = attn_t["us"]
    kernels = {}
    for n in names:
        if not run[n]:
            continue
        gbs = b[n] / (per_kernel_ms[n] * 1e-3) / 1e9
        kernels[n] = {"us": round(per_kernel_ms[n] * 1e3, 2), "us_p10": round(percentile(samples[n], 10) * 1e3, 2),
                      "us_p90": round(percentile(samples[n], 90) * 1e3, 2), "bytes": b[n], "GB/s": round(gbs, 1),
                      "frac_hbm": round(gbs / HBM_PEAK_GBS, 4),
                      "input_GB/s": round(b["inputs"][n] / (per_kernel_ms[n] * 1e-3) / 1e9, 1)}
    traffic = measured_traffic("quantize")
    if attn_us is not None:
        gbs = b["attention_decode"] / (attn_us * 1e-6) / 1e9
        kernels["attention_decode"] = {**attn_t, "bytes": b["attention_decode"], "GB/s": round(gbs, 1),
                                       "frac_hbm": round(gbs / HBM_PEAK_GBS, 4), "in_step": False}
    if attn_us is not None and not args.only:
        kernels.update(stream_decode(torch, kvq, d, w, q, kc, vcache, signs, att_out, ws, stream, dev,
                                     args.steps, args.warmup))
        kernels.update(nsn_kernels(torch, kvq, w, x, q, signs, y, stream, dev, min(args.steps, 10),
                                   min(args.warmup, 2)))
    if args.only:
        print(json.dumps({"profile_only": args.only, "kernels": kernels, "steps": args.steps}), flush=True)
        return
    # the attainable ceiling: a device-to-device copy of the 4 GiB fp16 cache (as many bytes read as
    # written), timed like the kernels; each long-context kernel's rate is also given against it
    copy_t = time_calls(torch, lambda: y.copy_(x), stream, min(args.steps, 10), min(args.warmup, 2))
    copy_bytes = 2 * x.numel() * x.element_size()
    copy_gbs = copy_bytes / (copy_t["us"] * 1e-6) / 1e9
    for n, k in kernels.items():
        if "GB/s" in k and "us" in k and "shape" not in k:
            k["frac_copy"] = round(k["GB/s"] / copy_gbs, 4)
    qa = kernels["quantize"]["GB/s"]
    out = {
        "metric": "quantize/dequant/decode-score GB/s and % of HBM peak, 1x MI355X",
        "value": round(step_bytes / (ms_per_step * 1e-3) / 1e9, 2),
        "unit": "GB/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic (seeded; Qwen2-7B-like KV statistics: 8 outlier channels per head at 100-167, token norm swing <= 4.7x)",
        "config": {"workload": WORKLOAD, "seqs": w.seqs, "tokens_per_seq": w.tokens, "kv_heads": w.heads,
                   "head_dim": w.head_dim, "q_heads": w.q_heads, "mode": "nsep_pchan", "bits": 4,
                   "block_tokens": w.block_tokens, "hadamard": w.hadamard, "step": "quantize+dequantize+score_decode",
                   "step_bytes": step_bytes, "gpu_step_ms": round(gpu_step_ms, 4)},
        "kernels": kernels,
        "roofline": {"bound": "hbm", "kernel": "quantize", "achieved": qa, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(qa / HBM_PEAK_GBS, 4), "traffic": traffic},
        "copy_ceiling": {**copy_t, "bytes": copy_bytes, "GB/s": round(copy_gbs, 1),
                         "frac_hbm": round(copy_gbs / HBM_PEAK_GBS, 4), "what": "torch device-to-device copy of the fp16 cache"},
        "cpu_baseline": None,
    }
    if args.other_configs:
        del y
        out["other_configs"] = other_configs(torch, kvq, synth, dev, min(args.steps, 10), min(args.warmup, 2))
        y = None
    # the RRS activation path into an INT4 GEMM (a "next" row, outside the step)
    out["kernels"].update(rrs_kernels(torch, kvq, synth, dev, min(args.steps, 10), min(args.warmup, 2)))
    if args.cpu_seqs > 0:
        del x, y
        print("[bench] timing the fp64 oracle on the host", file=sys.stderr, flush=True)
        workers = args.cpu_workers or min(16, os.cpu_count() or 1)
        out["cpu_baseline"] = cpu_baseline(w, args.cpu_seqs, args.cpu_seqs_all, workers)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
