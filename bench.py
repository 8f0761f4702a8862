"""Benchmark of the fused FP8 MLA decode (libfp8mla.so) on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--config 2] [--replicas R]
    python bench.py --config 3 [--layers 78]     (the pages' cast-path comparison)
    python bench.py --write                      (the BF16 -> FP8 write path)
    python bench.py --extend {spec4,chunk1k,prefill4k_h64}   (extend / prefill attention)
    python bench.py --serving-step {bf16,fp8_cast,fp8_fused} [--layers L] [--trace T.json]
                                                 (one decode step over L layers: KV write +
                                                  attention, for the paired-trace ledger)

A step is one fused decode call over one batch: mla_decode_fp8 on the batch-40
workload (B=40 requests, 16 query heads sharing one 576-wide FP8 KV head,
context U[1024, 8192], page size 1, pool 495,552 slots, per-tensor scale
U[0.5, 2]) -- page-table resolution, FP8 row gather, in-kernel dequantisation,
score MFMA, online softmax, P.V MFMA and the split-K combine.  Inputs are
resident in HBM before timing.  R independent replicas (>= 1 GB together)
are cycled call by call so reads come from HBM, not from the 256 MB
Infinity Cache.

Prints ONE JSON line: useful KV GB/s (576 B per attended token / call time),
the roofline of the decode kernels against MI355X's 8 TB/s HBM peak, and the
CPU oracle timed on the host on a bounded sample.
"""
import argparse
import ctypes
import hashlib
import json
import math
import os
import re
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "useful KV GB/s (% of HBM peak) + µs/call, FP8 MLA decode, batch 40, 4k ctx"
HBM_PEAK_GBPS = 8000.0
COUNTERS_FILE = os.path.join(ROOT, "profiles", "mla_decode_batch40_counters.txt")
# the sources the batch-40 decode kernels are compiled from (the counter file
# records their digest, so stale counters are never reported)
KERNEL_SOURCES = [os.path.join(ROOT, "fp8_paged_mla_amd", "csrc", f)
                  for f in ("mla_decode.hip", "decode_common.h", "device_common.h")]


def parse_args():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    # untimed warm-up: about 35 ms of back-to-back calls, so that the timed
    # calls run at the GPU's steady-state clocks (after 10 calls they were
    # still ~7% slower)
    ap.add_argument("--warmup", type=int, default=1000)
    ap.add_argument("--config", type=int, default=2, choices=[1, 2, 3, 4, 5])
    ap.add_argument("--layers", type=int, default=78, help="config 3: layers per decode step")
    ap.add_argument("--replicas", type=int, default=0, help="0 = enough for >= 1 GB")
    ap.add_argument("--splits", type=int, default=None,
                    help="bound the decode's split-K segments (mla_decode_fp8_segments); "
                         "default: the library's own partition")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-secondary", action="store_true")
    ap.add_argument("--serving-step", choices=["bf16", "fp8_cast", "fp8_fused"], default=None,
                    help="time one decode step (KV write + attention per layer) of a KV-cache variant")
    ap.add_argument("--trace", default=None,
                    help="with --serving-step: torch-profiler trace (chrome JSON) of the timed steps")
    ap.add_argument("--extend", default=None,
                    choices=["spec4", "chunk1k", "prefill4k_h64"],
                    help="time the extend (prefill) attention mla_extend_fp8 on a named workload")
    ap.add_argument("--write", action="store_true",
                    help="time the BF16 -> FP8 write path (scatter_cast_bf16_fp8) instead")
    ap.add_argument("--probe", action="store_true",
                    help="run the HBM ceiling probes (read, 1:2 read:write, random 576-B rows) only")
    return ap.parse_args()


def _code_only(text):
    """C/C++ source with comments removed and whitespace runs collapsed, so
    that the digest below changes with the code and not with its comments
    (string literals in these sources hold no comment markers)."""
    text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
    text = re.sub(r"//[^\n]*", " ", text)
    return " ".join(text.split())


def source_digest(paths):
    h = hashlib.sha256()
    for path in paths:
        with open(path, encoding="utf-8") as f:
            h.update(_code_only(f.read()).encode())
    return h.hexdigest()[:16]


def read_traffic(launch_units):
    """HBM bytes per call from committed rocprofv3 counter runs, if they were
    taken on the current kernel source; else None."""
    if not os.path.exists(COUNTERS_FILE):
        return None
    vals = {}
    with open(COUNTERS_FILE) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#") and "=" in line:
                k, v = line.split("=", 1)
                vals[k.strip()] = v.strip()
    if vals.get("source_sha256_16") != source_digest(KERNEL_SOURCES):
        return None
    try:
        return float(vals["hbm_bytes_per_call"])
    except (KeyError, ValueError):
        return None


def decode_kernel_name(w, dev):
    """The split kernel the library plans for this workload: 64 heads per
    workgroup at H >= 64 when there are at least 4 x CUs / ceil(H / 64)
    64-token tiles, else 16 heads per workgroup."""
    import torch
    cus = torch.cuda.get_device_properties(dev).multi_processor_count
    tiles = (w.total_tokens + 63) // 64
    if w.H >= 64 and tiles >= 4 * cus // ((w.H + 63) // 64):
        return "mla_split_h64_kernel<false>"
    return "mla_split_kernel<%s>" % ("true" if w.H <= 16 else "false")


def algorithmic_decode_bytes(w):
    """Bytes a decode call must move: every attended token's 576-byte row and
    4-byte slot id, the indptr entries, q (576 BF16 per head) and out (512
    BF16 per head); split-K partials are the implementation's, not the
    method's."""
    return (w.total_tokens * (576 + 4) + 4 * (w.B + 1) + 2 * w.B * w.H * (576 + 512))


def cpu_baseline(w, label, budget_s=15.0):
    """The float64 oracle on the host over the same workload: its requests one
    by one, in repeated passes over the batch, until about budget_s seconds
    have run (at least one full pass)."""
    import numpy as np
    import oracle
    try:
        from threadpoolctl import threadpool_limits
    except ImportError:  # pragma: no cover
        threadpool_limits = None
    cores = len(os.sched_getaffinity(0))
    args = (w.q.view(__import__("torch").int16).cpu().numpy().view(np.uint16),
            w.pool.cpu().numpy(), w.indptr.cpu().numpy(), w.indices.cpu().numpy(),
            w.scale, w.sm_scale)
    ctx = threadpool_limits(limits=cores) if threadpool_limits else None
    tokens = 0
    passes = 0
    t0 = time.perf_counter()
    try:
        if ctx:
            ctx.__enter__()
        while passes == 0 or time.perf_counter() - t0 < budget_s:
            for b in range(w.B):
                oracle.mla_decode_ref(*args, requests=[b])
                tokens += int(w.lengths[b])
            passes += 1
    finally:
        if ctx:
            ctx.__exit__(None, None, None)
    dt = time.perf_counter() - t0
    return {
        "value": round(576.0 * tokens / dt / 1e9, 4),
        "unit": "GB/s",
        "cores": cores,
        "kind": "oracle",
        "sample": "float64 numpy oracle (BLAS on up to %d threads), %d passes over the %d "
                  "requests (%d tokens each pass) of replica 0 of the %s workload: %d tokens "
                  "in %.1f s" % (cores, passes, w.B, tokens // max(passes, 1), label, tokens, dt),
    }


def main():
    args = parse_args()
    if args.gpus != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path "
              "(--gpus %d requested)" % args.gpus, file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import fp8_paged_mla_amd as fm
    import workloads

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    fm.library()
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)

    if args.config == 3:
        print(json.dumps(cast_path_step(fm, workloads, torch, dev, args)), flush=True)
        return
    if args.write:
        print(json.dumps(write_path(fm, workloads, torch, dev)), flush=True)
        return
    if args.extend:
        print(json.dumps(extend_bench(fm, workloads, torch, dev, args)), flush=True)
        return
    if args.serving_step:
        print(json.dumps(serving_step(fm, workloads, torch, dev, args)), flush=True)
        return
    if args.probe:
        print(json.dumps(hbm_probes(torch, dev, full=True)), flush=True)
        return

    base = workloads.config(args.config, 0, device=dev)
    pool_bytes = base.pool.numel()
    R = args.replicas or max(4, math.ceil(1.0e9 / pool_bytes))
    reps = [base] + [workloads.config(args.config, r, device=dev) for r in range(1, R)]
    outs = [torch.empty((w.B, w.H, 512), dtype=torch.bfloat16, device=dev) for w in reps]
    wss = [torch.empty(max(256, fm.mla_decode_fp8_workspace_bytes(w.B, w.H, w.total_tokens)),
                       dtype=torch.uint8, device=dev) for w in reps]
    useful = [w.useful_kv_bytes for w in reps]
    algo = [algorithmic_decode_bytes(w) for w in reps]
    stream = torch.cuda.current_stream(dev)

    # each replica's call checked and marshalled once (the binding's prepared
    # path); every call still goes through the C ABI's own checks and
    # launches all of the decode's kernels
    calls = [fm.prepare_mla_decode_fp8(w.q, w.pool, w.indptr, w.indices, w.scale, w.sm_scale,
                                       out=outs[r], workspace=wss[r], stream=stream,
                                       segments=args.splits)
             for r, w in enumerate(reps)]

    def call(i):
        calls[i % R]()

    for i in range(args.warmup):
        call(i)
    torch.cuda.synchronize(dev)

    # timed region: K calls cycling over replicas, one event pair around all
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize(dev)
    t0 = time.perf_counter()
    start.record(stream)
    for i in range(args.steps):
        call(i)
    host_us = (time.perf_counter() - t0) * 1e6 / args.steps
    stop.record(stream)
    torch.cuda.synchronize(dev)
    wall_ms = (time.perf_counter() - t0) * 1e3
    total_ms = start.elapsed_time(stop)
    ms_per_step = total_ms / args.steps
    bytes_total = sum(useful[i % R] for i in range(args.steps))
    value = bytes_total / (total_ms * 1e-3) / 1e9

    # per-call distribution (same rotation), each call bracketed by events
    per_call = []
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(args.steps)]
    for i in range(args.steps):
        evs[i][0].record(stream)
        call(i)
        evs[i][1].record(stream)
    torch.cuda.synchronize(dev)
    per_call = [a.elapsed_time(b) * 1e3 for a, b in evs]
    q = np.percentile(per_call, [10, 50, 90])

    mean_useful = bytes_total / args.steps
    mean_algo = sum(algo[i % R] for i in range(args.steps)) / args.steps
    achieved = mean_algo / (ms_per_step * 1e-3) / 1e9
    # the call's bound: its algorithmic bytes at the HBM peak against its
    # MFMA flops (scores over 576 dims, P.V over 512, per head and token) at
    # the dense BF16/FP16 peak; at 16 heads the bytes dominate, at 128 the flops
    mean_flops = sum(2.0 * base.H * 1088 * reps[i % R].total_tokens
                     for i in range(args.steps)) / args.steps
    t_hbm_us = mean_algo / (HBM_PEAK_GBPS * 1e9) * 1e6
    t_mfma_us = mean_flops / (MFMA_BF16_PEAK_TFLOPS * 1e12) * 1e6
    if t_mfma_us > t_hbm_us:
        tflops = mean_flops / (ms_per_step * 1e-3) / 1e12
        roof_head = {"bound": "mfma", "achieved": round(tflops, 2), "peak": MFMA_BF16_PEAK_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(tflops / MFMA_BF16_PEAK_TFLOPS, 4)}
    else:
        roof_head = {"bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_PEAK_GBPS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBPS, 4)}
    result = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16 scores / fp16 P.V, fp32 accumulate (fp8 e4m3 KV)",
        "data": "synthetic",
        "config": {
            "workload": workloads.CONFIG_NAMES[args.config],
            "batch": base.B,
            "heads": base.H,
            "kv_width": 576,
            "kv_dtype": "fp8_e4m3fn",
            "mean_tokens_per_call": round(sum(w.total_tokens for w in reps) / R, 1),
            "replicas_rotated": R,
            "rotated_footprint_GB": round(R * pool_bytes / 1e9, 3),
            "split_segments": "library default" if args.splits is None else
                              "at most %d" % args.splits,
        },
        "pct_hbm_peak": round(100.0 * value / HBM_PEAK_GBPS, 2),
        "us_per_call": {"p10": round(float(q[0]), 2), "median": round(float(q[1]), 2),
                        "p90": round(float(q[2]), 2)},
        "wall_ms_timed_region": round(wall_ms, 3),
        "host_us_per_call": round(host_us, 2),
        "roofline": {
            **roof_head,
            # counters are committed for the batch-40 workload (library
            # partition) only
            "traffic": read_traffic(1) if args.config == 2 and args.splits is None else None,
            "kernel": "one mla_decode_fp8 call: %s + mla_combine_kernel" % decode_kernel_name(base, dev),
            "algorithmic_bytes_per_call": int(mean_algo),
            "algorithmic_bytes": "576 B KV + 4 B index per token, 4 B per indptr entry, "
                                 "2 B per q (576) and out (512) element",
            "useful_kv_bytes_per_call": int(mean_useful),
            "algorithmic_GBps": round(achieved, 2),
            "flops_per_call": mean_flops,
            "t_hbm_us_at_peak": round(t_hbm_us, 2),
            "t_mfma_us_at_peak": round(t_mfma_us, 2),
        },
    }

    if not args.no_secondary:
        result["secondary"] = secondary(fm, reps, outs, wss, stream, dev, args)
        probes = hbm_probes(torch, dev)
        result["secondary"]["hbm_probes"] = probes
        # the same decode against the measured ceiling of its access mix
        # (random 576-byte rows: useful bytes against the gather probe's)
        result["roofline"]["probe_ceiling"] = {
            "probe": "gather576_2chunk (random 576-B rows into LDS, no math)",
            "GBps": probes["gather576_2chunk_GBps"],
            "frac_useful": round(value / probes["gather576_2chunk_GBps"], 4)}
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(base, workloads.CONFIG_NAMES[args.config].split(":")[0])
    print(json.dumps(result), flush=True)


def cast_path_step(fm, workloads, torch, dev, args):
    """The pages' per-step comparison over `layers` distinct 495,552-slot FP8
    pools (one request, 4,096 tokens, 64 heads), each summed over the layers:
    the cast kernels alone (full-pool cast, gather-cast of the active slots),
    the two complete fallback paths (cast + BF16-row attention with the
    original indices; gather-cast + BF16-row attention over indices 0..n-1),
    and the fused FP8 decode."""
    L = args.layers
    w0 = workloads.config(3, 0, device=dev)
    pools = [w0.pool] + [workloads.random_pool(495552, seed=3000 + 7 * l + 1, device=dev)
                         for l in range(1, L)]
    stream = torch.cuda.current_stream(dev)
    cast_out = torch.empty((495552, 576), dtype=torch.bfloat16, device=dev)
    g_out = torch.empty((w0.total_tokens, 576), dtype=torch.bfloat16, device=dev)
    out = torch.empty((w0.B, w0.H, 512), dtype=torch.bfloat16, device=dev)
    ws = torch.empty(max(256, fm.mla_decode_fp8_workspace_bytes(w0.B, w0.H, w0.total_tokens)),
                     dtype=torch.uint8, device=dev)
    ws16 = torch.empty(max(256, fm.mla_decode_bf16_workspace_bytes(w0.B, w0.H, w0.total_tokens)),
                       dtype=torch.uint8, device=dev)
    seq = torch.arange(w0.total_tokens, dtype=torch.int32, device=dev)

    # Every call of every path is checked and marshalled once, so that a
    # layer's host time (~6 us through the prepared path, ~15 us through the
    # plain binding) stays below its GPU time and the step is timed on the
    # GPU, not on the host.  Each call still goes through the C ABI's checks.
    lib = fm.library()
    c = ctypes
    h = c.c_void_p(stream.cuda_stream)
    N, T = 495552, w0.total_tokens

    def prep(fn, where, *args):
        return fm.PreparedCall(fn, args, None, None, where)

    cast_calls = [prep(lib.cast_pool_fp8_bf16, "cast_pool_fp8_bf16", c.c_void_p(p.data_ptr()),
                       c.c_int64(N), c.c_void_p(cast_out.data_ptr()), h) for p in pools]
    gather_calls = [prep(lib.gather_cast_fp8_bf16, "gather_cast_fp8_bf16",
                         c.c_void_p(p.data_ptr()), c.c_int64(N), c.c_void_p(w0.indices.data_ptr()),
                         c.c_int64(T), c.c_void_p(g_out.data_ptr()), h) for p in pools]

    def bf16_call(kv, rows, indices):
        return prep(lib.mla_decode_bf16, "mla_decode_bf16", c.c_void_p(w0.q.data_ptr()),
                    c.c_void_p(kv.data_ptr()), c.c_int64(rows), c.c_void_p(w0.indptr.data_ptr()),
                    c.c_void_p(indices.data_ptr()), c.c_int64(T), c.c_int32(w0.B),
                    c.c_int32(w0.H), c.c_float(w0.scale), c.c_float(w0.sm_scale),
                    c.c_void_p(out.data_ptr()), c.c_void_p(ws16.data_ptr()),
                    c.c_size_t(ws16.numel()), h)

    attend_cast = bf16_call(cast_out, N, w0.indices)
    attend_gather = bf16_call(g_out, T, seq)
    fused_calls = [fm.prepare_mla_decode_fp8(w0.q, p, w0.indptr, w0.indices, w0.scale,
                                             w0.sm_scale, out=out, workspace=ws, stream=stream)
                   for p in pools]
    layer_of = {id(p): l for l, p in enumerate(pools)}

    def cast_path(p):
        cast_calls[layer_of[id(p)]]()
        attend_cast()

    def gather_path(p):
        gather_calls[layer_of[id(p)]]()
        attend_gather()

    def timed(fn, reps=3):
        best = None
        for _ in range(reps):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            torch.cuda.synchronize(dev)
            e0.record(stream)
            for l in range(L):
                fn(pools[l])
            e1.record(stream)
            torch.cuda.synchronize(dev)
            ms = e0.elapsed_time(e1)
            best = ms if best is None else min(best, ms)
        return best

    for l in range(L):  # warm-up pass
        cast_calls[l]()
    cast_ms = timed(lambda p: cast_calls[layer_of[id(p)]]())
    gather_ms = timed(lambda p: gather_calls[layer_of[id(p)]]())
    fused_ms = timed(lambda p: fused_calls[layer_of[id(p)]]())
    cast_path_ms = timed(cast_path)
    gather_path_ms = timed(gather_path)
    cast_bytes = 495552 * 576 * 3
    gather_bytes = w0.total_tokens * (4 + 576 + 1152)
    result = {
        "metric": "per-decode-step time over %d layers: full-pool cast vs gather-cast vs fused" % L,
        "unit": "ms/step",
        "higher_is_better": False,
        "data": "synthetic",
        "config": {"workload": workloads.CONFIG_NAMES[3], "layers": L,
                   "pool_bytes_total_GB": round(L * 495552 * 576 / 1e9, 2)},
        "cast_pool_ms_per_step": round(cast_ms, 3),
        "cast_pool_GBps": round(L * cast_bytes / (cast_ms * 1e-3) / 1e9, 1),
        "cast_pool_pct_hbm_peak": round(100 * L * cast_bytes / (cast_ms * 1e-3) / 1e9 / HBM_PEAK_GBPS, 1),
        "gather_cast_ms_per_step": round(gather_ms, 4),
        "gather_cast_GBps": round(L * gather_bytes / (gather_ms * 1e-3) / 1e9, 1),
        "gather_cast_us_per_layer": round(gather_ms * 1e3 / L, 2),
        "fused_decode_ms_per_step": round(fused_ms, 4),
        "fused_decode_us_per_layer": round(fused_ms * 1e3 / L, 2),
        "cast_then_attend_ms_per_step": round(cast_path_ms, 3),
        "gather_then_attend_ms_per_step": round(gather_path_ms, 4),
        "gather_then_attend_us_per_layer": round(gather_path_ms * 1e3 / L, 2),
        "fused_speedup_vs_cast_then_attend": round(cast_path_ms / fused_ms, 1),
        "fused_speedup_vs_gather_then_attend": round(gather_path_ms / fused_ms, 2),
    }
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_cast_baseline(pools[0], L)
    return result


def cpu_cast_baseline(pool, layers, budget_s=10.0):
    """The oracle's full-pool cast (a 256-entry table lookup in numpy, one
    thread) of one 495,552-slot pool on the host, repeated for about budget_s
    seconds; the per-step figure multiplies the per-pool time by the layer
    count (layers x pool and BF16 copy would not fit in host memory)."""
    import oracle
    host = pool.cpu().numpy()
    reps = 0
    t0 = time.perf_counter()
    while reps == 0 or time.perf_counter() - t0 < budget_s:
        oracle.cast_ref(host)
        reps += 1
    per_pool_s = (time.perf_counter() - t0) / reps
    return {
        "value": round(per_pool_s * layers * 1e3, 1),
        "unit": "ms/step",
        "cores": 1,
        "kind": "oracle",
        "sample": "oracle cast (numpy table lookup) of one %d-slot pool (%.0f MB) on one "
                  "host thread, %d repetitions at %.3f s each, times %d layers "
                  "(extrapolated)" % (host.shape[0], host.nbytes / 1e6, reps, per_pool_s, layers),
    }


MFMA_BF16_PEAK_TFLOPS = 2500.0


def extend_bench(fm, workloads, torch, dev, args):
    """mla_extend_fp8 on a named extend workload: device time per call, MFMA
    throughput against the BF16 dense peak (the work is 2 * H * 1088 flops per
    (query token, visible cache token) pair) and cache bytes per second.
    Beside it, the same attention as one decode request per query token
    (mla_decode_fp8 over each token's visible prefix, index lists expanded on
    the host): what sharing each KV tile among a block's tokens saves."""
    import numpy as np
    w = workloads.extend_config(args.extend, device=dev)
    stream = torch.cuda.current_stream(dev)
    out = torch.empty((w.total_q, w.H, 512), dtype=torch.bfloat16, device=dev)
    ws = torch.empty(max(256, fm.mla_extend_fp8_workspace_bytes(w.B, w.H, w.total_q)),
                     dtype=torch.uint8, device=dev)

    def ext():
        fm.mla_extend_fp8(w.q, w.pool, w.qo_indptr, w.kv_indptr, w.kv_indices, w.scale,
                          w.sm_scale, causal=w.causal, out=out, workspace=ws)

    # per-token decode form: request r = query token, its visible prefix as the index list
    qo = w.qo_indptr.cpu().numpy()
    kv = w.kv_indptr.cpu().numpy()
    idx = w.kv_indices.cpu().numpy()
    lists, lens = [], []
    for b in range(w.B):
        ql, kl = int(qo[b + 1] - qo[b]), int(kv[b + 1] - kv[b])
        for i in range(ql):
            n = max(0, min(kl, kl - ql + i + 1)) if w.causal else kl
            lists.append(idx[kv[b]:kv[b] + n])
            lens.append(n)
    tok_indptr = torch.from_numpy(np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)).to(dev)
    tok_indices = torch.from_numpy(np.concatenate(lists).astype(np.int32)).to(dev)
    out_d = torch.empty_like(out)
    ws_d = torch.empty(max(256, fm.mla_decode_fp8_workspace_bytes(w.total_q, w.H, int(sum(lens)))),
                       dtype=torch.uint8, device=dev)

    def per_token():
        fm.mla_decode_fp8(w.q, w.pool, tok_indptr, tok_indices, w.scale, w.sm_scale, out=out_d,
                          workspace=ws_d)

    def timed(fn, k):
        for _ in range(3):
            fn()
        torch.cuda.synchronize(dev)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(k):
            fn()
        e1.record(stream)
        torch.cuda.synchronize(dev)
        return e0.elapsed_time(e1) * 1e3 / k

    K = max(5, min(args.steps, 100))
    us = timed(ext, K)
    us_tok = timed(per_token, K)
    pairs = w.visible_tokens()
    flops = 2.0 * w.H * 1088 * pairs
    tflops = flops / (us * 1e-6) / 1e12
    # algorithmic bytes: every cache row of a request once (576 B + its 4-byte
    # slot id), both indptr arrays, q (576 BF16) and out (512 BF16) per query row
    kv_tokens = int(w.kv_lens.sum())
    algo_bytes = 580 * kv_tokens + 8 * (w.B + 1) + 2 * w.total_q * w.H * (576 + 512)
    t_hbm_us = algo_bytes / (HBM_PEAK_GBPS * 1e9) * 1e6
    t_mfma_us = flops / (MFMA_BF16_PEAK_TFLOPS * 1e12) * 1e6
    if t_mfma_us >= t_hbm_us:
        roof = {"bound": "mfma", "achieved": round(tflops, 2), "peak": MFMA_BF16_PEAK_TFLOPS,
                "unit": "TFLOP/s", "frac": round(tflops / MFMA_BF16_PEAK_TFLOPS, 4)}
    else:
        gbs = algo_bytes / (us * 1e-6) / 1e9
        roof = {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                "frac": round(gbs / HBM_PEAK_GBPS, 4)}
    roof.update({"traffic": None, "t_hbm_us_at_peak": round(t_hbm_us, 2),
                 "t_mfma_us_at_peak": round(t_mfma_us, 2), "algorithmic_bytes_per_call": algo_bytes,
                 "flops_per_call": flops,
                 "kernel": "one mla_extend_fp8 call: pre-pass + mla_split_h64_kernel<true> + combine"})
    return {
        "metric": "extend attention over the FP8 cache: TFLOP/s + us/call",
        "value": round(tflops, 2), "unit": "TFLOP/s", "higher_is_better": True,
        "data": "synthetic", "dtype": "bf16 scores / fp16 P.V, fp32 accumulate (fp8 e4m3 KV)",
        "steps": K,
        "config": {"workload": w.name, "total_q": w.total_q, "heads": w.H,
                   "cache_tokens": kv_tokens, "visible_pairs": pairs,
                   "causal": w.causal},
        "us_per_call": round(us, 2),
        "query_tokens_per_s": round(w.total_q / (us * 1e-6), 1),
        "cache_GBps": round(w.kv_bytes() / (us * 1e-6) / 1e9, 1),
        "roofline": roof,
        "per_token_decode_us": round(us_tok, 2),
        "speedup_vs_per_token_decode": round(us_tok / us, 2),
    }


def serving_step(fm, workloads, torch, dev, args):
    """One decode step of the batch-40 workload over `layers` layers, each with its
    own 495,552-slot pool: per layer, the step's 40 new KV rows are written to
    their requests' newest slots, then attention runs over every request's
    history.  Three KV-cache variants of the same step, as in the pages' paired
    traces ("When a Faster Kernel Doesn't Speed Up Serving", Step 1; "The KV
    Cache Cast Bottleneck", The Context):
      bf16      -- BF16 pools: index write, attention over BF16 rows;
      fp8_cast  -- FP8 pools, the pages' path: BF16 -> FP8 copy + index write,
                   full-pool FP8 -> BF16 copy, attention over the BF16 copy;
      fp8_fused -- FP8 pools: scatter_cast_bf16_fp8, mla_decode_fp8.
    With --trace, the timed steps are recorded with the torch profiler (kernel
    names and durations for fp8_paged_mla_amd.ledger)."""
    L = args.layers
    K = max(1, min(args.steps, 20))
    w = workloads.config(2, 0, device=dev)
    pools8 = [w.pool] + [workloads.random_pool(495552, seed=2000 + 7 * l + 1, device=dev)
                         for l in range(1, L)]
    newest = (w.indptr[1:] - 1).long()
    slots = w.indices[newest].contiguous()
    slots_l = slots.long()
    rows = [workloads.new_kv_rows(w.B, seed=7000 + l, device=dev) for l in range(L)]
    out = torch.empty((w.B, w.H, 512), dtype=torch.bfloat16, device=dev)
    variant = args.serving_step
    if variant == "bf16":
        pools16 = [fm.cast_pool_fp8_bf16(p) for p in pools8]
        del pools8
        ws = torch.empty(max(256, fm.mla_decode_bf16_workspace_bytes(w.B, w.H, w.total_tokens)),
                         dtype=torch.uint8, device=dev)

        def layer(l):
            pools16[l][slots_l] = rows[l]
            fm.mla_decode_bf16(w.q, pools16[l], w.indptr, w.indices, w.scale, w.sm_scale,
                               out=out, workspace=ws)
    elif variant == "fp8_cast":
        cast_out = torch.empty((495552, 576), dtype=torch.bfloat16, device=dev)
        ws = torch.empty(max(256, fm.mla_decode_bf16_workspace_bytes(w.B, w.H, w.total_tokens)),
                         dtype=torch.uint8, device=dev)

        def layer(l):
            pools8[l][slots_l] = rows[l].to(torch.float8_e4m3fn).view(torch.uint8)
            cast_out.copy_(pools8[l].view(torch.float8_e4m3fn))
            fm.mla_decode_bf16(w.q, cast_out, w.indptr, w.indices, w.scale, w.sm_scale,
                               out=out, workspace=ws)
    else:
        ws = torch.empty(max(256, fm.mla_decode_fp8_workspace_bytes(w.B, w.H, w.total_tokens)),
                         dtype=torch.uint8, device=dev)

        def layer(l):
            fm.scatter_cast_bf16_fp8(rows[l], slots, pools8[l])
            fm.mla_decode_fp8(w.q, pools8[l], w.indptr, w.indices, w.scale, w.sm_scale,
                              out=out, workspace=ws)

    stream = torch.cuda.current_stream(dev)

    def steps(k):
        for _ in range(k):
            for l in range(L):
                layer(l)

    steps(2)
    torch.cuda.synchronize(dev)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    steps(K)
    e1.record(stream)
    torch.cuda.synchronize(dev)
    ms = e0.elapsed_time(e1) / K
    res = {"metric": "decode step over %d layers: KV write + attention, %s KV cache" % (L, variant),
           "value": round(ms, 4), "unit": "ms/step", "higher_is_better": False,
           "steps": K, "data": "synthetic",
           "config": {"workload": workloads.CONFIG_NAMES[2], "layers": L, "variant": variant}}
    if args.trace:
        from torch.profiler import ProfilerActivity, profile
        with profile(activities=[ProfilerActivity.CPU, ProfilerActivity.CUDA],
                     record_shapes=True) as prof:
            steps(K)
            torch.cuda.synchronize(dev)
        prof.export_chrome_trace(args.trace)
        from fp8_paged_mla_amd import ledger
        t = ledger.totals_from_kernels(ledger.read_kernel_events(args.trace))
        res["trace"] = args.trace
        res["categories_ms_per_step"] = {c: round(v[1] / K, 4) for c, v in t.rows.items()}
        res["kernels_per_step"] = {c: v[0] / K for c, v in t.rows.items()}
    return res


def write_path(fm, workloads, torch, dev, sizes=(40, 1024, 16384, 65536)):
    """The write path into one layer's 495,552-slot FP8 pool: n new BF16 rows
    quantised and scattered to distinct random slots, for a decode step's 40
    rows and extend chunks.  Sources rotate over >= 256 MB so reads come from
    HBM.  Bytes moved per row: 1152 read + 576 written + 4 slot id.

    `us` is device time per call: the calls are captured once in a HIP graph
    and the graph is replayed, so host launch cost is excluded (the kernel
    allocates and clears nothing, so it captures as is).  `us_eager` is the
    same loop launched from Python, for small n bound by the host.  The pages'
    own path (a BF16 -> FP8 copy, then an index write, two kernels plus a
    temporary) is timed eagerly beside it."""
    stream = torch.cuda.current_stream(dev)
    pool = workloads.random_pool(495552, seed=4242, device=dev)
    res = {"metric": "BF16 -> FP8 write path: quantise + scatter into a 495,552-slot pool",
           "unit": "us/call, GB/s", "higher_is_better": False, "data": "synthetic",
           "dtype": "bf16 -> fp8_e4m3fn", "bytes_per_row": 1152 + 576 + 4, "sizes": {}}
    for n in sizes:
        R = min(64, max(2, -(-256 * 2 ** 20 // (n * 1152))))
        srcs = [workloads.new_kv_rows(n, seed=50 + r, device=dev) for r in range(R)]
        slots = [torch.from_numpy(workloads.free_slots(n, 495552, seed=90 + r)).to(dev)
                 for r in range(R)]
        longs = [s.long() for s in slots]
        iters = max(20, min(2000, int(2e6 // n)))

        def ours(i):
            fm.scatter_cast_bf16_fp8(srcs[i], slots[i], pool)

        def pages_path(i):
            pool[longs[i]] = srcs[i].to(torch.float8_e4m3fn).view(torch.uint8)

        def eager_us(fn):
            for i in range(min(R, 10)):
                fn(i)
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            torch.cuda.synchronize(dev)
            e0.record(stream)
            for i in range(iters):
                fn(i % R)
            e1.record(stream)
            torch.cuda.synchronize(dev)
            return e0.elapsed_time(e1) * 1e3 / iters

        def graph_us(fn, calls):
            side = torch.cuda.Stream(device=dev)
            side.wait_stream(stream)
            with torch.cuda.stream(side):
                for i in range(3):
                    fn(i % R)
            stream.wait_stream(side)
            torch.cuda.synchronize(dev)
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                for i in range(calls):
                    fn(i % R)
            g.replay()
            torch.cuda.synchronize(dev)
            best = None
            for _ in range(5):
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record(stream)
                g.replay()
                e1.record(stream)
                torch.cuda.synchronize(dev)
                t = e0.elapsed_time(e1) * 1e3 / calls
                best = t if best is None else min(best, t)
            del g
            return best

        us = graph_us(ours, max(R, min(400, iters)))
        us_e = eager_us(ours)
        us_t = eager_us(pages_path)
        moved = n * (1152 + 576 + 4)
        res["sizes"][str(n)] = {
            "us": round(us, 2), "GBps": round(moved / (us * 1e-6) / 1e9, 1),
            "pct_hbm_peak": round(100 * moved / (us * 1e-6) / 1e9 / HBM_PEAK_GBPS, 1),
            "us_eager": round(us_e, 2),
            "torch_copy_then_index_us_eager": round(us_t, 2),
            "speedup_eager_vs_torch_path": round(us_t / us_e, 2)}
        del srcs, slots, longs
    return res


def hbm_probes(torch, dev, full=False):
    """Measured HBM ceilings for the library's access mixes (the probes of
    include/fp8mla_probe.h), each the best over a small sweep of launch
    shapes, buffers past the 256 MB Infinity Cache:
      read        sequential 16-byte loads over 2 GiB;
      copy_1to2   512 MiB read, each 16-byte chunk written twice (1 GiB): the cast's mix;
      write       1 GiB of sequential stores;
      gather576   2^20 random 576-byte rows of a 2^21-slot pool into LDS, 1 or 2
                  chunks of 16 rows in flight per wave (2: the decode's LDS budget).
    GB/s counts bytes read + written; the gather counts 576 B per row."""
    import numpy as np
    from fp8_paged_mla_amd import probe
    cus = torch.cuda.get_device_properties(dev).multi_processor_count
    stream = torch.cuda.current_stream(dev)
    sink = torch.zeros(65536 * 8, dtype=torch.int32, device=dev)

    def best_us(fn, reps=5):
        for _ in range(2):
            fn()
        times = []
        for _ in range(reps):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            fn()
            e1.record(stream)
            torch.cuda.synchronize(dev)
            times.append(e0.elapsed_time(e1) * 1e3)
        return min(times)

    res = {}
    src = torch.empty(2 << 30, dtype=torch.uint8, device=dev)
    src.fill_(0x3C)
    sweep = [(g, u) for g in (4 * cus, 8 * cus, 16 * cus) for u in (4, 8, 16)] if full else \
            [(8 * cus, 8), (16 * cus, 8)]
    best = None
    for g, u in sweep:
        us = best_us(lambda: probe.probe_read(src, g, u, sink))
        gbs = src.numel() / (us * 1e-6) / 1e9
        if best is None or gbs > best[0]:
            best = (gbs, g, u)
    res["read_GBps"] = round(best[0], 1)
    res["read_launch"] = "grid %d x 256 lanes, %d loads in flight per lane" % (best[1], best[2])
    del src
    src = torch.empty(512 << 20, dtype=torch.uint8, device=dev).fill_(0x3C)
    dst = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
    best = None
    for g, u in sweep:
        us = best_us(lambda: probe.probe_copy_1to2(src, dst, g, u))
        gbs = 3 * src.numel() / (us * 1e-6) / 1e9
        if best is None or gbs > best[0]:
            best = (gbs, g, u)
    res["copy_1to2_GBps"] = round(best[0], 1)
    res["copy_1to2_launch"] = "grid %d x 256 lanes, %d loads in flight per lane" % (best[1], best[2])
    best = None
    for g, u in sweep:
        us = best_us(lambda: probe.probe_write(dst, g, u))
        gbs = dst.numel() / (us * 1e-6) / 1e9
        if best is None or gbs > best[0]:
            best = (gbs, g, u)
    res["write_GBps"] = round(best[0], 1)
    res["write_launch"] = "grid %d x 256 lanes, %d stores per lane per step" % (best[1], best[2])
    del src, dst
    slots = 1 << 21
    pool = torch.randint(0, 256, (slots, 576), dtype=torch.uint8, device=dev)
    rng = np.random.default_rng(7)
    idx = torch.from_numpy(rng.permutation(slots)[: 1 << 20].astype(np.int32)).to(dev)
    for s_inflight, grids in ((2, (cus,)), (1, (cus, 2 * cus))):
        best = None
        for g in grids:
            us = best_us(lambda: probe.probe_gather_rows(pool, idx, g, s_inflight, sink))
            gbs = 576 * idx.numel() / (us * 1e-6) / 1e9
            if best is None or gbs > best[0]:
                best = (gbs, g)
        res["gather576_%dchunk_GBps" % s_inflight] = round(best[0], 1)
        res["gather576_%dchunk_launch" % s_inflight] = (
            "grid %d x 8 waves, %d x 16 rows (%d B of LDS) in flight per wave"
            % (best[1], s_inflight, s_inflight * 9472))
    del pool, idx
    return res


def secondary(fm, reps, outs, wss, stream, dev, args):
    """Warm (no rotation) decode, and the two cast kernels on one 495,552-slot pool."""
    import torch
    w = reps[0]
    n = 50
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    for _ in range(5):
        fm.mla_decode_fp8(w.q, w.pool, w.indptr, w.indices, w.scale, w.sm_scale, out=outs[0],
                          workspace=wss[0])
    e0.record(stream)
    for _ in range(n):
        fm.mla_decode_fp8(w.q, w.pool, w.indptr, w.indices, w.scale, w.sm_scale, out=outs[0],
                          workspace=wss[0])
    e1.record(stream)
    torch.cuda.synchronize(dev)
    warm_us = e0.elapsed_time(e1) * 1e3 / n
    res = {"decode_warm_us": round(warm_us, 2),
           "decode_warm_GBps": round(w.useful_kv_bytes / (warm_us * 1e-6) / 1e9, 1)}
    # cast paths on pools of 495,552 slots (rotating the replicas' pools)
    pools = [r.pool for r in reps if r.pool.shape[0] == 495552]
    if pools:
        cast_out = torch.empty((495552, 576), dtype=torch.bfloat16, device=dev)
        for p in pools:
            fm.cast_pool_fp8_bf16(p, out=cast_out)
        e0.record(stream)
        for i in range(20):
            fm.cast_pool_fp8_bf16(pools[i % len(pools)], out=cast_out)
        e1.record(stream)
        torch.cuda.synchronize(dev)
        us = e0.elapsed_time(e1) * 1e3 / 20
        moved = 495552 * 576 * 3
        res["cast_pool_us"] = round(us, 2)
        res["cast_pool_GBps"] = round(moved / (us * 1e-6) / 1e9, 1)
        idx = reps[0].indices[:4096].contiguous()
        g_out = torch.empty((4096, 576), dtype=torch.bfloat16, device=dev)
        for p in pools:
            fm.gather_cast_fp8_bf16(p, idx, out=g_out)
        e0.record(stream)
        for i in range(50):
            fm.gather_cast_fp8_bf16(pools[i % len(pools)], idx, out=g_out)
        e1.record(stream)
        torch.cuda.synchronize(dev)
        us = e0.elapsed_time(e1) * 1e3 / 50
        res["gather_cast_4096_us"] = round(us, 2)
        res["gather_cast_4096_GBps"] = round(4096 * (4 + 576 + 1152) / (us * 1e-6) / 1e9, 1)
        allidx = reps[0].indices
        n_all = allidx.shape[0]
        g2 = torch.empty((n_all, 576), dtype=torch.bfloat16, device=dev)
        e0.record(stream)
        for i in range(20):
            fm.gather_cast_fp8_bf16(pools[i % len(pools)], allidx, out=g2)
        e1.record(stream)
        torch.cuda.synchronize(dev)
        us = e0.elapsed_time(e1) * 1e3 / 20
        res["gather_cast_batch40_rows"] = int(n_all)
        res["gather_cast_batch40_us"] = round(us, 2)
        res["gather_cast_batch40_GBps"] = round(n_all * (4 + 576 + 1152) / (us * 1e-6) / 1e9, 1)
        # plain device copy of the same pool (torch's copy kernel): measured HBM ceiling
        src = pools[0]
        dst = torch.empty_like(src)
        big = torch.empty(src.numel() * 3 // 2, dtype=torch.uint8, device=dev)
        dst2 = torch.empty_like(big)
        for _ in range(3):
            dst2.copy_(big)
        e0.record(stream)
        for _ in range(20):
            dst2.copy_(big)
        e1.record(stream)
        torch.cuda.synchronize(dev)
        us = e0.elapsed_time(e1) * 1e3 / 20
        res["torch_copy_428MB_GBps"] = round(2 * big.numel() / (us * 1e-6) / 1e9, 1)
        del dst
    return res


if __name__ == "__main__":
    main()
