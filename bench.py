"""Benchmark of the Gram Newton-Schulz hot path on one MI355X.

    python bench.py [--steps K] [--warmup W] [--workload NAME] [--compute f16|bf16]
                    [--no-cpu-baseline] [--gpus 1]

Default workload: one 1024 x 4096 bf16 momentum matrix (aspect ratio 4), Gram NS with
T = 5 quintic steps of (3.4445, -4.7750, 2.0315), restart after step 2, fp16 iterates
with fp32 accumulation.  A step is one gns_orthogonalize_batched call over the batch,
launched eagerly (a HIP-graph replay of the same call is timed too); inputs are
resident in HBM before the timed region.  One JSON line is printed.

Also measured in the same run:
  * roofline of the dominant kernel (the lower-tile symmetric MFMA product), timed
    live with HIP events by replaying its per-step launch mix through the C ABI;
  * the standard-NS baseline on the same kernels;
  * cpu_baseline: the float64 numpy oracle on the host cores, on a bounded sample.
Other workloads (--workload) print the same line for that workload.
"""
from __future__ import annotations

import argparse
import math
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "orthogonalized matrices/s + TFLOP/s (% bf16 MFMA peak), batched Gram NS, α=4"
DEFAULT_WORKLOAD = "gns_1024x4096_bf16"
PEAK_16BIT_TFLOPS = 2516.6        # MI355X dense bf16/fp16 MFMA
PEAK_HBM_GBS = 8000.0


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=200)
    p.add_argument("--warmup", type=int, default=20)
    p.add_argument("--workload", default=DEFAULT_WORKLOAD)
    p.add_argument("--compute", default="f16")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--cpu-seconds", type=float, default=12.0)
    p.add_argument("--no-extra", action="store_true",
                   help="default workload only: skip the other workloads and the bf16-iterate timing "
                        "that the default line carries as extra keys")
    p.add_argument("--restart-sweep", action="store_true",
                   help="only measure Gram NS error against the float64 oracle for each restart "
                        "position (fp16 and bf16 iterates) on the 1024x4096 and square 2048^2 inputs, "
                        "one JSON line per case, and exit")
    p.add_argument("--calibrate-copy", action="store_true",
                   help="only run a plain 512 MiB device copy 5 times (reference for rocprofv3 "
                        "FETCH_SIZE / WRITE_SIZE scale factors) and exit")
    return p.parse_args()


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only: the library has no multi-GPU path (--gpus {args.gpus} "
              "requested). The batch of same-shape matrices would shard across GPUs, with one all-to-all "
              "per shape group in each direction.",
              file=sys.stderr)
        sys.exit(2)
    import numpy as np
    import torch
    import muon_gram_ns_amd as gns
    import synth
    from muon_gram_ns_amd import flops as F

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.calibrate_copy:
        src = torch.ones(256 << 20, device=dev, dtype=torch.float16)     # 512 MiB
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"calibration": "device copy", "bytes_read": src.numel() * 2,
                          "bytes_written": dst.numel() * 2, "launches": 5}), flush=True)
        return
    if args.restart_sweep:
        return restart_sweep(gns, synth, torch, np)
    w = synth.workload(args.workload)
    if w.name.startswith("dion3"):
        return bench_dion3(args, w)

    st = synth.gns_batch(w)
    if w.dtype == "bf16":
        X = torch.from_numpy(st.view(np.int16)).view(torch.bfloat16).to(dev)
    else:
        X = torch.from_numpy(st).to(dev)
    B, n, m = X.shape
    compute = args.compute if w.dtype != "f32" else "f32"
    out = torch.empty_like(X)
    sched = gns.default_schedule()
    stream = torch.cuda.current_stream(dev)

    def timed_ms(fn, steps, warmup):
        for _ in range(warmup):
            fn()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(steps):
            fn()
        torch.cuda.synchronize()
        return 1e3 * (time.perf_counter() - t0) / steps

    _, issued = gns.orthogonalize(X, out=out, compute=compute, schedule=sched, return_flops=True)
    # the step: one whole Gram NS call over the batch, launched eagerly on the current
    # stream; the same call captured once in a HIP graph (own output and workspace) and
    # replayed is timed too (on ROCm the replay does not beat eager launches here)
    ms = timed_ms(lambda: gns.orthogonalize(X, out=out, compute=compute, schedule=sched),
                  args.steps, args.warmup)
    per_call = per_call_ms(torch, stream, lambda: gns.orthogonalize(X, out=out, compute=compute, schedule=sched),
                           max(20, min(args.steps, 200)))
    graphed = gns.graphed_orthogonalize(X, out=torch.empty_like(X), compute=compute, schedule=sched)
    ms_graph = timed_ms(graphed.replay, args.steps, args.warmup)
    mats_per_s = B / (ms * 1e-3)
    square = (n == m) and sched.square_fallback
    alg = B * (F.standard_schedule(n, m) if square else F.gram_schedule(n, m))
    nominal = B * F.standard_ns_nominal(n, m)

    # standard-NS baseline on the same kernels, timed the same two ways
    out_std = torch.empty_like(X)
    nstd = max(10, args.steps // 4)
    ms_std = timed_ms(lambda: gns.newton_schulz(X, out=out_std, compute=compute, schedule=sched),
                      nstd, max(2, args.warmup // 4))
    graphed_std = gns.graphed_newton_schulz(X, out=torch.empty_like(X), compute=compute, schedule=sched)
    ms_std_graph = timed_ms(graphed_std.replay, nstd, max(2, args.warmup // 4))

    muon = muon_timing(gns, torch, X, compute, sched, timed_ms, nstd, max(2, args.warmup // 4), ms) \
        if w.dtype == "bf16" else None
    roof = dominant_kernel_roofline(gns, F, torch, B, n, m, compute, square, args.steps, w.name)
    line = {
        "metric": METRIC,
        "value": round(mats_per_s, 3),
        "unit": "matrices/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": {"f16": "fp16", "bf16": "bf16", "f32": "fp32"}[compute],
        "data": "synthetic",
        "config": {"workload": w.name, "batch": B, "n": n, "m": m, "alpha": m / n, "T": sched.steps,
                   "restart_after": [s for s in range(1, 16) if (sched.restart_after_mask >> s) & 1],
                   "input_dtype": w.dtype, "iterate_dtype": compute, "accumulate": "fp32",
                   "method": "standard NS (aspect ratio 1 fallback)" if square else "Gram NS"},
        "tflops_standard_ns_equivalent": round(nominal / (ms * 1e-3) / 1e12, 3),
        "tflops_algorithmic": round(alg / (ms * 1e-3) / 1e12, 3),
        "tflops_issued": round(issued / (ms * 1e-3) / 1e12, 3),
        "pct_peak_issued": round(100 * issued / (ms * 1e-3) / 1e12 / PEAK_16BIT_TFLOPS, 3),
        "timing": "eager launches of the whole call on one stream (inputs resident in HBM)",
        "per_call_ms": per_call,
        "graph_replay": {"ms_per_step": round(ms_graph, 5), "matrices_per_s": round(B / (ms_graph * 1e-3), 3)},
        "standard_ns_same_kernels": {"ms_per_step": round(ms_std, 5),
                                     "matrices_per_s": round(B / (ms_std * 1e-3), 3),
                                     "gram_speedup": round(ms_std / ms, 3),
                                     "graph_replay_ms_per_step": round(ms_std_graph, 5)},
        "muon_step_same_batch": muon,
        "roofline": roof,
        "cpu_baseline": None if args.no_cpu_baseline else cpu_baseline(st, w, args.cpu_seconds),
    }
    if w.name == DEFAULT_WORKLOAD and not args.no_extra and compute == "f16":
        del graphed, graphed_std
        # the same call with bf16 iterates (bf16 MFMA; the Gram chain in hi/lo bf16 planes)
        ms_bf = timed_ms(lambda: gns.orthogonalize(X, out=out, compute="bf16", schedule=sched), nstd,
                         max(2, args.warmup // 4))
        ms_bf_std = timed_ms(lambda: gns.newton_schulz(X, out=out_std, compute="bf16", schedule=sched), nstd,
                             max(2, args.warmup // 4))
        _, issued_bf = gns.orthogonalize(X, out=out, compute="bf16", schedule=sched, return_flops=True)
        line["bf16_iterates"] = {"ms_per_step": round(ms_bf, 5), "matrices_per_s": round(B / (ms_bf * 1e-3), 3),
                                 "tflops_issued": round(issued_bf / (ms_bf * 1e-3) / 1e12, 3),
                                 "standard_ns_ms_per_step": round(ms_bf_std, 5),
                                 "gram_speedup": round(ms_bf_std / ms_bf, 3)}
        del X, out, out_std
        torch.cuda.empty_cache()
        line["other_workloads"] = other_workloads(args, gns, F, torch, np, synth)
    print(json.dumps(line), flush=True)


GEMM_SOURCES = ("muon_gram_ns_amd/csrc/gemm_kernel.h", "muon_gram_ns_amd/csrc/gemm_symm.hip",
                "muon_gram_ns_amd/csrc/common.h", "muon_gram_ns_amd/csrc/internal.h")
TRAFFIC_FILE = "profiles/traffic_gemm16_lower_f16_gns_1024x4096.json"


def gemm_source_digest():
    """sha256 over the GEMM kernel sources: HBM traffic counted with rocprofv3 is
    only reported while the kernel is the one it was counted on."""
    import hashlib
    h = hashlib.sha256()
    for f in GEMM_SOURCES:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def measured_traffic(workload_name, launch_mix):
    path = os.path.join(ROOT, TRAFFIC_FILE)
    if not os.path.exists(path):
        return None
    with open(path) as fh:
        t = json.load(fh)
    if (t.get("workload") != workload_name or t.get("launch_mix") != launch_mix
            or t.get("gemm_source_sha256") != gemm_source_digest()):
        return None
    return t["bytes_per_launch"]


DION3_SOURCES = ("muon_gram_ns_amd/csrc/dion3.hip", "muon_gram_ns_amd/csrc/common.h")
DION3_TRAFFIC_FILE = "profiles/traffic_accumulate_score_dion3_8192x28672.json"


def measured_dion3_traffic(workload_name):
    """HBM bytes per accumulate_score launch from rocprofv3 counters, reported only
    while the Dion3 kernel sources are the ones they were counted on."""
    import hashlib
    path = os.path.join(ROOT, DION3_TRAFFIC_FILE)
    if not os.path.exists(path):
        return None
    with open(path) as fh:
        t = json.load(fh)
    h = hashlib.sha256()
    for f in DION3_SOURCES:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    if t.get("workload") != workload_name or t.get("dion3_source_sha256") != h.hexdigest():
        return None
    return t["bytes_per_launch"]


def dominant_kernel_roofline(gns, F, torch, B, n, m, compute, square, steps, workload_name, per_graph=10):
    """The lower-tile symmetric MFMA product in the iterate dtype dominates a Gram NS
    call.  Its per-call launch mix (the n x n products with K = n, plus the restart
    Gram product with K = m) is replayed through the C ABI on the current stream,
    captured once in a HIP graph so the events time back-to-back kernels rather than
    host launch overhead.

    The roof is the lower of the MFMA peak and arithmetic intensity x HBM bandwidth,
    with the algorithmic flops (n(n+1)K per product) and algorithmic bytes of the mix:
    a product of one n x n operand (Za = c R R + b R + a I, read as A, B and the beta C
    term) reads it once and writes one; a product of two distinct n x n operands reads
    both and writes one; the Gram product reads X once and writes n x n.  At n = 1024
    the intensity is below the ridge (~315 flop/B), so the roof is HBM and `achieved`
    is algorithmic GB/s; the MFMA fraction is given beside it."""
    dt = {"f16": torch.float16, "bf16": torch.bfloat16, "f32": torch.float32}[compute]
    e = torch.tensor([], dtype=dt).element_size()
    # Gram NS (T=5, restart after 2), n x n products per call: one Za per step (5) and
    # 9 products of two operands without a C term (t1: Y = R Za, R = Za Y; t2: Q Za;
    # t3: Y, R; t4: Q Za and R Za in one paired launch, R; t5: Q Za); plus the Gram
    # product of the restarted X (K = m).  Standard NS: per step one X X^T (K = m) and
    # one Ba = c A A + b A + a I (K = n).
    sym = lambda t: (t + t.transpose(1, 2)) * 0.5
    R = sym(torch.randn(B, n, n, device="cuda")).to(dt)
    Z = sym(torch.randn(B, n, n, device="cuda")).to(dt)
    Xh = (torch.randn(B, n, m, device="cuda") / m ** 0.5).to(dt)
    D = torch.empty(B, n, n, device="cuda", dtype=dt)
    groups = [(5, "self"), (5, "gram")] if square else [(5, "self"), (9, "pair"), (1, "gram")]
    desc = {"self": f"K={n}, c R R + b R + a I", "pair": f"K={n}, R Z", "gram": f"K={m}, X X^T"}
    launch_mix = " + ".join(f"{k} x (n={n}, {desc[kind]})" for k, kind in groups) + f", batch {B}"
    launches = sum(k for k, _ in groups)

    def mix():
        for k, kind in groups:
            for _ in range(k):
                if kind == "self":
                    gns.symm_gemm(R, R, C=R, alpha=2.0, beta=-4.0, gamma=3.0, out=D)
                elif kind == "pair":
                    gns.symm_gemm(R, Z, out=D)
                else:
                    gns.symm_gemm(Xh, Xh, out=D)

    for _ in range(3):
        mix()
    torch.cuda.synchronize()
    timing = "HIP graph replay"
    try:
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            for _ in range(per_graph):
                mix()
        run = graph.replay
        launches_per_run = per_graph * launches
    except Exception as exc:  # capture unavailable: eager launches, host overhead included
        timing = f"eager launches (graph capture failed: {type(exc).__name__})"
        run = mix
        launches_per_run = launches
    reps = max(5, steps // (4 * per_graph))
    run()
    stream = torch.cuda.current_stream()
    s, ev = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    s.record(stream)
    for _ in range(reps):
        run()
    ev.record(stream)
    torch.cuda.synchronize()
    avg_s = s.elapsed_time(ev) * 1e-3 / (reps * launches_per_run)
    flops_of = {"self": F.sym(n, n), "pair": F.sym(n, n), "gram": F.sym(n, m)}
    bytes_of = {"self": 2 * n * n * e, "pair": 3 * n * n * e, "gram": (n * m + n * n) * e}
    alg_flops = B * sum(k * flops_of[kind] for k, kind in groups) / launches
    alg_bytes = B * sum(k * bytes_of[kind] for k, kind in groups) / launches
    intensity = alg_flops / alg_bytes
    tflops = alg_flops / avg_s / 1e12
    gbs = alg_bytes / avg_s / 1e9
    hbm_bound = intensity * PEAK_HBM_GBS * 1e9 < PEAK_16BIT_TFLOPS * 1e12
    traffic = measured_traffic(workload_name, launch_mix)
    roof = {"bound": "hbm" if hbm_bound else "mfma",
            "kernel": f"gemm16_kernel ({compute}, lower-triangle symmetric)",
            "shape_mix": launch_mix, "timing": timing, "avg_launch_us": round(avg_s * 1e6, 3),
            "algorithmic_flops_per_launch": alg_flops, "algorithmic_bytes_per_launch": alg_bytes,
            "intensity_flop_per_byte": round(intensity, 1),
            "ridge_flop_per_byte": round(PEAK_16BIT_TFLOPS * 1e12 / (PEAK_HBM_GBS * 1e9), 1)}
    if hbm_bound:
        roof.update({"achieved": round(gbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": round(gbs / PEAK_HBM_GBS, 5)})
    else:
        roof.update({"achieved": round(tflops, 3), "peak": PEAK_16BIT_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(tflops / PEAK_16BIT_TFLOPS, 5)})
    roof.update({"traffic": traffic, "mfma_tflops": round(tflops, 3),
                 "mfma_frac": round(tflops / PEAK_16BIT_TFLOPS, 5)})
    return roof


def muon_timing(gns, torch, X, compute, sched, timed_ms, steps, warmup, ms_gram):
    """The whole Muon step (muon_step_batched: momentum with the lookahead, Gram NS,
    decoupled decay and the scaled update) on the same batch, against the Gram NS call
    alone.  The step's element-wise passes move 7 n m bf16 values per matrix (read M,
    G; write M, U; read W, O; write W), and its momentum pass also forms the Frobenius
    norm, so the Gram NS inside the step skips the norm pass of the standalone call:
    the extra time is the element-wise passes less that pass."""
    B, n, m = X.shape
    W, M, G = X.clone(), X.clone(), X
    ms_muon = timed_ms(lambda: gns.muon_step(W, M, G, 1e-4, weight_decay=0.1, compute=compute, schedule=sched),
                       steps, warmup)
    return {"ms_per_step": round(ms_muon, 5), "matrices_per_s": round(B / (ms_muon * 1e-3), 3),
            "gram_ns_alone_ms": round(ms_gram, 5), "extra_ms_over_gram_ns": round(ms_muon - ms_gram, 5),
            "elementwise_bytes": 7.0 * B * n * m * 2, "nesterov": True, "scale": "0.2 sqrt(max(n, m))"}


def per_call_ms(torch, stream, fn, n):
    """HIP events around each of n calls on the launch stream (after the timed
    region): median, 10th and 90th percentile in ms."""
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n)]
    torch.cuda.synchronize()
    for a, b in evs:
        a.record(stream)
        fn()
        b.record(stream)
    torch.cuda.synchronize()
    t = sorted(a.elapsed_time(b) for a, b in evs)
    pick = lambda q: round(t[min(len(t) - 1, int(q * (len(t) - 1) + 0.5))], 5)
    return {"calls": n, "median": pick(0.5), "p10": pick(0.1), "p90": pick(0.9)}


def host_description():
    """CPU model and the BLAS library numpy runs on (for the oracle baseline)."""
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    blas = "unknown"
    try:
        from threadpoolctl import threadpool_info
        libs = [d for d in threadpool_info() if d.get("user_api") == "blas"]
        if libs:
            blas = f"{libs[0].get('internal_api')} {libs[0].get('version')}"
    except Exception:
        pass
    return model, blas


def cpu_baseline(st, w, seconds):
    """The float64 oracle (standard NS) on the host, on a bounded sample."""
    import numpy as np
    import oracle
    try:
        from threadpoolctl import threadpool_info
        threads = max([d.get("num_threads", 1) for d in threadpool_info()] or [os.cpu_count()])
    except Exception:
        threads = os.cpu_count()
    x = oracle.bf16_to_f64(st[0]) if w.dtype == "bf16" else st[0].astype(np.float64)
    done, t0 = 0, time.perf_counter()
    while True:
        oracle.newton_schulz(x)
        done += 1
        el = time.perf_counter() - t0
        if el >= seconds or done >= 1000:
            break
    model, blas = host_description()
    return {"value": round(done / el, 4), "unit": "matrices/s", "cores": threads, "kind": "oracle",
            "cpu_model": model, "blas": blas, "nproc": os.cpu_count(),
            "sample": f"{done} x one {w.n}x{w.m} matrix of the workload, float64 standard NS (numpy/OpenBLAS), "
                      f"{el:.1f} s"}


def sync_timed_ms(torch, fn, steps, warmup):
    """Mean ms per call of `steps` eager calls after `warmup` untimed ones, bracketed by
    device synchronisations."""
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        fn()
    torch.cuda.synchronize()
    return 1e3 * (time.perf_counter() - t0) / steps


def square_gemm_reference(gns, torch, batch, n, steps, warmup):
    """The n x n x n products of the square batch on their own: this library's
    rectangular kernel and torch.bmm (the vendor's GEMM library) on the same contiguous
    fp16 operands, timed alike, so the MFMA fraction has a reference on this machine."""
    g = torch.Generator(device="cuda")
    g.manual_seed(4096)
    A = (torch.randn(batch, n, n, device="cuda", generator=g) * n ** -0.5).half()
    Bm = torch.randn(batch, n, n, device="cuda", generator=g).half()
    D = torch.empty_like(A)
    flops = 2.0 * batch * float(n) ** 3

    def fig(ms):
        tf = flops / (ms * 1e-3) / 1e12
        return {"ms": round(ms, 4), "tflops": round(tf, 2), "pct_peak": round(100 * tf / PEAK_16BIT_TFLOPS, 2)}

    lib = fig(sync_timed_ms(torch, lambda: gns.rect_gemm(A, Bm, out=D), steps, warmup))
    vendor = fig(sync_timed_ms(torch, lambda: torch.bmm(A, Bm, out=D), steps, warmup))
    del A, Bm, D
    torch.cuda.empty_cache()
    return {"shape": f"{batch} x ({n} x {n}) @ ({n} x {n}), fp16 in and out, fp32 accumulation",
            "library_rect_gemm": lib, "torch_bmm": vendor}


def other_workloads(args, gns, F, torch, np, synth):
    """The other configurations, timed in the same run as the default line so that their
    figures are observed by the same driver run: the 32 x 4096^2 square batch (the pages'
    aspect-ratio-1 fallback to standard NS, and the Gram path forced), the 128 x 768x6144
    MoE batch (alpha = 8) and the Dion3 step on the 8192 x 28672 state (f = 1/4, 1/8).
    Each carries a roofline of its dominant kernel, timed live with HIP events on the
    launch stream.  Inputs are synth's seeded bytes (the Dion3 state is drawn on the
    device from a seeded generator with the workload's distribution)."""
    res = {}
    steps = max(3, args.steps // 20)
    warm = 2
    for name in ("gns_32x4096x4096_bf16", "gns_128x768x6144_bf16"):
        t0 = time.perf_counter()
        w = synth.workload(name)
        st = synth.gns_batch(w)
        gen_s = time.perf_counter() - t0
        X = torch.from_numpy(st.view(np.int16)).view(torch.bfloat16).cuda()
        del st
        B, n, m = X.shape
        out = torch.empty_like(X)
        entry = {"batch": B, "n": n, "m": m, "alpha": m / n, "iterate_dtype": "f16", "input_generation_s": round(gen_s, 1)}
        nominal = B * F.standard_ns_nominal(n, m)

        def figures(ms, issued, alg):
            return {"ms_per_step": round(ms, 4), "matrices_per_s": round(B / (ms * 1e-3), 3),
                    "tflops_standard_ns_equivalent": round(nominal / (ms * 1e-3) / 1e12, 3),
                    "tflops_algorithmic": round(alg / (ms * 1e-3) / 1e12, 3),
                    "tflops_issued": round(issued / (ms * 1e-3) / 1e12, 3),
                    "pct_peak_issued": round(100 * issued / (ms * 1e-3) / 1e12 / PEAK_16BIT_TFLOPS, 3)}

        gram_sched = gns.default_schedule(square_fallback=False)
        _, iss_g = gns.orthogonalize(X, out=out, schedule=gram_sched, return_flops=True)
        ms_g = sync_timed_ms(torch, lambda: gns.orthogonalize(X, out=out, schedule=gram_sched), steps, warm)
        _, iss_s = gns.newton_schulz(X, out=out, return_flops=True)
        ms_s = sync_timed_ms(torch, lambda: gns.newton_schulz(X, out=out), steps, warm)
        entry["gram_ns"] = figures(ms_g, iss_g, B * F.gram_schedule(n, m))
        entry["standard_ns_same_kernels"] = figures(ms_s, iss_s, B * F.standard_schedule(n, m))
        entry["gram_speedup"] = round(ms_s / ms_g, 3)
        if n >= 4096:
            best = max(entry["gram_ns"]["pct_peak_issued"], entry["standard_ns_same_kernels"]["pct_peak_issued"])
            entry["mfma_goal"] = {"pct_of_peak": 60.0, "pct_peak_issued": best, "met": best >= 60.0,
                                  "note": "goal for n >= 4096: 60% of the dense fp16/bf16 MFMA peak; under load "
                                          "these products run at about 1.6 GHz with the MFMA pipe 61-67% busy"}
            entry["gemm_reference"] = square_gemm_reference(gns, torch, B, n, steps, warm)
        if n == m:
            entry["default_call"] = ("standard NS: at aspect ratio 1 the Gram form saves nothing and the pages fall "
                                     "back to kernelized standard NS (square_fallback = 1); gram_ns is the Gram "
                                     "path forced (square_fallback = 0)")
        del out
        entry["roofline"] = dominant_kernel_roofline(gns, F, torch, B, n, m, "f16", False, 40, name, per_graph=1)
        del X
        torch.cuda.empty_cache()
        res[name] = entry
    res["dion3_8192x28672_bf16"] = dion3_figures(args, synth.workload("dion3_8192x28672_bf16"), gns, F, torch)
    torch.cuda.empty_cache()
    return res


def dion3_figures(args, w, gns, F, torch, fractions=(0.25, 0.125)):
    """Whole Dion3 steps (l2 row scores, mu = 0.95, wd = 0, lr = 0.01 / sqrt(f)) on the
    workload's state, and the roofline of the accumulate-and-score pass (HBM-bound; the
    largest kernel of the step)."""
    N, m = w.n, w.m
    gen = torch.Generator(device="cuda").manual_seed(1000 + w.index)
    dev_bf16 = lambda: (torch.randn(N, m, device="cuda", generator=gen) * 0.02).to(torch.bfloat16)
    W, G, M = dev_bf16(), dev_bf16(), dev_bf16()
    stream = torch.cuda.current_stream()

    def timed(fn, reps):
        fn()
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        for _ in range(reps):
            fn()
        b.record(stream)
        torch.cuda.synchronize()
        return a.elapsed_time(b) * 1e-3 / reps

    reps = max(5, args.steps // 10)
    res = {"N": N, "m": m, "score": "l2", "mu": 0.95, "wd": 0.0, "iterate_dtype": args.compute}
    for f in fractions:
        k = math.ceil(f * N)
        lr = 0.01 / f ** 0.5
        t = timed(lambda: gns.dion3_step(W, M, G, k, lr, 0.0, 0.95, score_norm=2, compute=args.compute), reps)
        # the same step with the selected rows read in place (no gathered copy of M[S, :])
        inplace = gns.default_schedule(rows_in_place=True)
        t_in = timed(lambda: gns.dion3_step(W, M, G, k, lr, 0.0, 0.95, score_norm=2, compute=args.compute,
                                            schedule=inplace), reps)
        res[f"f={f}"] = {"k": k, "ms_per_step": round(t * 1e3, 4), "steps_per_s": round(1.0 / t, 3),
                         "gram_ns_tflops_algorithmic": round(F.gram_schedule(k, m) / t / 1e12, 2),
                         "rows_in_place_ms_per_step": round(t_in * 1e3, 4)}
    if 0.25 in fractions:
        # the f = 1/4 step on an fp32 state (W, M, G in fp32; the submatrix reaches the
        # 16-bit iterates through a scaled copy), and its accumulate-and-score pass
        k = math.ceil(0.25 * N)
        W32, G32, M32 = W.float(), G.float(), M.float()
        t32 = timed(lambda: gns.dion3_step(W32, M32, G32, k, 0.02, 0.0, 0.95, score_norm=2, compute=args.compute),
                    reps)
        t32_acc = timed(lambda: gns.dion3_accumulate_score(M32, G32, 2), reps)
        res["f=0.25"]["fp32_state_ms_per_step"] = round(t32 * 1e3, 4)
        res["f=0.25"]["fp32_state_accumulate_GB_s"] = round(3.0 * N * m * 4 / t32_acc / 1e9, 1)
        del W32, G32, M32
    t_acc = timed(lambda: gns.dion3_accumulate_score(M, G, 2), reps)
    b_acc = 3.0 * N * m * 2
    res["roofline"] = {"bound": "hbm", "kernel": "accumulate_score_kernel", "achieved": round(b_acc / t_acc / 1e9, 1),
                       "peak": PEAK_HBM_GBS, "unit": "GB/s", "frac": round(b_acc / t_acc / 1e9 / PEAK_HBM_GBS, 4),
                       "traffic": measured_dion3_traffic(w.name), "algorithmic_bytes_per_launch": b_acc,
                       "avg_launch_us": round(t_acc * 1e6, 2)}
    del W, G, M
    return res


def restart_sweep(gns, synth, torch, np):
    """Relative Frobenius error of Gram NS (T = 5, the blog's coefficients) against the
    float64 oracle for each restart position, with fp16 and bf16 iterates.  The pages
    restart once to flush the spurious negative eigenvalues that half-precision Gram
    iterates acquire; where to restart is left to a sweep the pages do not print.
    Standard NS on the same kernels, at the same iterate precision, is measured beside
    it: the pages compare the two only through loss curves."""
    import oracle
    cases = [("gns_1024x4096_bf16", 1, 1024, 4096), ("gns_128x768x6144_bf16", 1, 768, 6144),
             ("gns_32x4096x4096_bf16", 1, 2048, 2048)]
    masks = {"none": (), "after 1": (1,), "after 2": (2,), "after 3": (3,), "after 4": (4,),
             "after 1 and 3": (1, 3), "after 2 and 4": (2, 4)}
    for name, B, n, m in cases:
        st = synth.gns_batch(name, batch=B, n=n, m=m)
        X = torch.from_numpy(st.view(np.int16)).view(torch.bfloat16).cuda()
        t0 = time.perf_counter()
        ref = oracle.newton_schulz(oracle.bf16_to_f64(st[0]))
        t_ref = time.perf_counter() - t0
        for compute in ("f16", "bf16"):
            for label, ra in masks.items():
                sched = gns.default_schedule(restart_after=ra, square_fallback=False)
                got = gns.orthogonalize(X, compute=compute, schedule=sched)[0].float().cpu().double().numpy()
                finite = bool(np.isfinite(got).all())
                err = float(np.linalg.norm(np.nan_to_num(got) - ref) / np.linalg.norm(ref)) if finite else None
                print(json.dumps({"restart_sweep": name, "n": n, "m": m, "iterates": compute, "method": "gram",
                                  "restart": label, "rel_err_vs_oracle": err, "finite": finite,
                                  "oracle_seconds": round(t_ref, 2)}), flush=True)
            got = gns.newton_schulz(X, compute=compute)[0].float().cpu().double().numpy()
            finite = bool(np.isfinite(got).all())
            err = float(np.linalg.norm(np.nan_to_num(got) - ref) / np.linalg.norm(ref)) if finite else None
            print(json.dumps({"restart_sweep": name, "n": n, "m": m, "iterates": compute, "method": "standard",
                              "rel_err_vs_oracle": err, "finite": finite}), flush=True)


def megabatch_dion3(gns, torch, args, B=16, N=2048, m=8192, f=0.25):
    """One batched Dion3 step over B same-shape states against B single steps on the
    same states (the single-GPU analogue of the pages' megabatching)."""
    gen = torch.Generator(device="cuda").manual_seed(77)
    mk = lambda: (torch.randn(B, N, m, device="cuda", generator=gen) * 0.02).to(torch.bfloat16)
    W, G, M = mk(), mk(), mk()
    k = math.ceil(f * N)
    lr = 0.01 / f ** 0.5
    batched = lambda: gns.dion3_step_batched(W, M, G, k, lr, 0.0, 0.95, score_norm=2, compute=args.compute)

    def loop():
        for b in range(B):
            gns.dion3_step(W[b], M[b], G[b], k, lr, 0.0, 0.95, score_norm=2, compute=args.compute)

    res = {}
    for name, fn in (("batched", batched), ("loop", loop)):
        for _ in range(3):
            fn()
        torch.cuda.synchronize()
        reps = max(5, args.steps // 5)
        t0 = time.perf_counter()
        for _ in range(reps):
            fn()
        torch.cuda.synchronize()
        res[name] = (time.perf_counter() - t0) / reps
    del W, G, M
    return {"states": f"{B} x {N}x{m} bf16", "k": k, "batched_ms": round(res["batched"] * 1e3, 4),
            "loop_of_single_steps_ms": round(res["loop"] * 1e3, 4),
            "speedup": round(res["loop"] / res["batched"], 3)}


def tall_columns_vs_rows(gns, torch, args, N=28672, m=8192, f=0.25):
    """The tall transpose of the Dion3 state (28672 x 8192): one step selecting
    k = f m columns (dion3_step_cols, a 28672 x 2048 submatrix) against one step
    selecting k = f N rows (dion3_step, a 7168 x 8192 submatrix)."""
    gen = torch.Generator(device="cuda").manual_seed(88)
    mk = lambda: (torch.randn(N, m, device="cuda", generator=gen) * 0.02).to(torch.bfloat16)
    W, G, M = mk(), mk(), mk()
    kc, kr = math.ceil(f * m), math.ceil(f * N)
    lr = 0.01 / f ** 0.5
    cols = lambda: gns.dion3_step_cols(W, M, G, kc, lr, 0.0, 0.95, score_norm=2, compute=args.compute)
    rows = lambda: gns.dion3_step(W, M, G, kr, lr, 0.0, 0.95, score_norm=2, compute=args.compute)
    res = {}
    for name, fn in (("columns", cols), ("rows", rows)):
        for _ in range(2):
            fn()
        torch.cuda.synchronize()
        reps = max(3, args.steps // 10)
        t0 = time.perf_counter()
        for _ in range(reps):
            fn()
        torch.cuda.synchronize()
        res[name] = (time.perf_counter() - t0) / reps
    del W, G, M
    torch.cuda.empty_cache()
    return {"state": f"{N}x{m} bf16", "f": f, "k_columns": kc, "k_rows": kr,
            "columns_ms": round(res["columns"] * 1e3, 4), "rows_ms": round(res["rows"] * 1e3, 4),
            "columns_speedup": round(res["rows"] / res["columns"], 3)}


def dion3_cpu_baseline(w):
    """The float64 oracle's Dion3 step (accumulate, l2 row scores, top-k, standard NS
    on the selected rows, update, error feedback) on the workload's full seeded state
    at f = 1/4: one step is the bounded sample (about half a minute of CPU work)."""
    import oracle
    import synth
    try:
        from threadpoolctl import threadpool_info
        threads = max([d.get("num_threads", 1) for d in threadpool_info()] or [os.cpu_count()])
    except Exception:
        threads = os.cpu_count()
    W, G, M = synth.dion3_state(n=w.n, m=w.m)
    k = oracle.k_from_fraction(0.25, w.n)
    t0 = time.perf_counter()
    oracle.dion3_step(W, M, G, k, 0.01 / 0.25 ** 0.5, wd=0.0, mu=0.95, norm="l2")
    el = time.perf_counter() - t0
    model, blas = host_description()
    return {"value": round(1.0 / el, 5), "unit": "steps/s", "cores": threads, "kind": "oracle", "cpu_model": model,
            "blas": blas, "nproc": os.cpu_count(),
            "sample": f"one full f = 1/4 step on the {w.n}x{w.m} seeded state (k = {k}), {el:.1f} s"}


def bench_dion3(args, w):
    """Dion3 step on the 8192 x 28672 workload at f = 1/4 and 1/8 (l2 row scores).
    Inputs are drawn on the device from a seeded generator with the workload's
    distribution (W, G, M ~ N(0, 0.02), bf16); the parity tests use synth's bytes.
    Besides whole steps/s, each HBM-bound step is timed alone through its own ABI
    entry point (HIP events on the current stream) and reported in GB/s of
    algorithmic traffic; the roofline names the dominant one."""
    import torch
    import muon_gram_ns_amd as gns
    from muon_gram_ns_amd import flops as F
    N, m = w.n, w.m
    gen = torch.Generator(device="cuda").manual_seed(1000 + w.index)
    dev_bf16 = lambda: (torch.randn(N, m, device="cuda", generator=gen) * 0.02).to(torch.bfloat16)
    W, G, M = dev_bf16(), dev_bf16(), dev_bf16()
    stream = torch.cuda.current_stream()

    def timed(fn, reps):
        fn()
        torch.cuda.synchronize()
        s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        s.record(stream)
        for _ in range(reps):
            fn()
        e.record(stream)
        torch.cuda.synchronize()
        return s.elapsed_time(e) * 1e-3 / reps

    res = {}
    for f in (0.25, 0.125):
        k = math.ceil(f * N)                  # f = 1/4, 1/8: exact
        lr = 0.01 / f ** 0.5
        step = lambda: gns.dion3_step(W, M, G, k, lr, 0.0, 0.95, score_norm=2, compute=args.compute)
        for _ in range(args.warmup):
            step()
        t = timed(step, args.steps)
        graphed = gns.graphed_dion3_step(W, M, G, k, lr, 0.0, 0.95, score_norm=2, compute=args.compute)
        for _ in range(args.warmup):
            graphed.replay()
        t_graph = timed(graphed.replay, args.steps)
        del graphed
        # the same step on k rows drawn at random (the pages' alternative to top-k; the
        # draw, a seeded device permutation, is input generation outside the step)
        S_rand = torch.randperm(N, device="cuda", generator=gen)[:k].sort().values.to(torch.int32)
        step_rows = lambda: gns.dion3_step_rows(W, M, G, S_rand, lr, 0.0, 0.95, compute=args.compute)
        for _ in range(args.warmup):
            step_rows()
        t_rows = timed(step_rows, args.steps)
        inplace = gns.default_schedule(rows_in_place=True)
        step_in = lambda: gns.dion3_step(W, M, G, k, lr, 0.0, 0.95, score_norm=2, compute=args.compute,
                                         schedule=inplace)
        for _ in range(args.warmup):
            step_in()
        t_in = timed(step_in, args.steps)
        res[f] = {"k": k, "ms_per_step": round(t * 1e3, 4), "graph_replay_ms_per_step": round(t_graph * 1e3, 4),
                  "gram_ns_tflops_algorithmic": round(F.gram_schedule(k, m) / t / 1e12, 2),
                  "random_rows_ms_per_step": round(t_rows * 1e3, 4),
                  "rows_in_place_ms_per_step": round(t_in * 1e3, 4)}
    # the HBM-bound pieces, alone (k = 2048)
    k = N // 4
    reps = max(5, args.steps)
    S = gns.dion3_select_topk(gns.dion3_accumulate_score(M, G, 2)[0], k)
    X = gns.dion3_gather_feedback(M, S, 0.95)
    t_acc = timed(lambda: gns.dion3_accumulate_score(M, G, 2), reps)
    t_sel = timed(lambda: gns.dion3_select_topk(gns.dion3_accumulate_score(M, G, 2)[0], k), reps) - t_acc
    t_gat = timed(lambda: gns.dion3_gather_feedback(M, S, 0.95), reps)
    t_upd = timed(lambda: gns.dion3_apply_update(W, S, X, 0.02, 0.0), reps)
    b_acc, b_gat, b_upd = 3.0 * N * m * 2, 3.0 * k * m * 2, 3.0 * k * m * 2
    # what the memory system sustains for the same traffic patterns, with torch's own
    # kernels on the same tensors: an in-place add (read 2, write 1) and a copy
    t_add = timed(lambda: M.add_(G), reps)
    scratch = torch.empty_like(M)
    t_cpy = timed(lambda: scratch.copy_(M), reps)
    reference = {"torch_add_inplace_GB_s": round(b_acc / t_add / 1e9, 1),
                 "torch_copy_GB_s": round(2.0 * N * m * 2 / t_cpy / 1e9, 1)}
    del scratch
    pieces = {"accumulate_score": {"us": round(t_acc * 1e6, 2), "bytes": b_acc, "GB_s": round(b_acc / t_acc / 1e9, 1)},
              "select_topk": {"us": round(t_sel * 1e6, 2)},
              "gather_feedback": {"us": round(t_gat * 1e6, 2), "bytes": b_gat, "GB_s": round(b_gat / t_gat / 1e9, 1)},
              "apply_update": {"us": round(t_upd * 1e6, 2), "bytes": b_upd, "GB_s": round(b_upd / t_upd / 1e9, 1)}}
    # the f = 1/4 step and its accumulate pass on an fp32 state (W, M, G in fp32)
    W32, G32, M32 = W.float(), G.float(), M.float()
    k = N // 4
    step32 = lambda: gns.dion3_step(W32, M32, G32, k, 0.02, 0.0, 0.95, score_norm=2, compute=args.compute)
    for _ in range(args.warmup):
        step32()
    t32 = timed(step32, args.steps)
    t32_acc = timed(lambda: gns.dion3_accumulate_score(M32, G32, 2), reps)
    fp32_state = {"k": k, "ms_per_step": round(t32 * 1e3, 4),
                  "accumulate_score": {"us": round(t32_acc * 1e6, 2), "bytes": 2 * b_acc,
                                       "GB_s": round(2 * b_acc / t32_acc / 1e9, 1)}}
    del W32, G32, M32
    ms = res[0.25]["ms_per_step"]
    roof = {"bound": "hbm", "kernel": "accumulate_score_kernel", "achieved": pieces["accumulate_score"]["GB_s"],
            "peak": PEAK_HBM_GBS, "unit": "GB/s", "frac": round(pieces["accumulate_score"]["GB_s"] / PEAK_HBM_GBS, 4),
            "traffic": measured_dion3_traffic(w.name), "algorithmic_bytes_per_launch": b_acc}
    del W, G, M
    torch.cuda.empty_cache()
    mega = megabatch_dion3(gns, torch, args)
    tall = tall_columns_vs_rows(gns, torch, args)
    cpu = None if args.no_cpu_baseline else dion3_cpu_baseline(w)
    print(json.dumps({"metric": "Dion3 steps/s", "value": round(1e3 / ms, 3), "unit": "steps/s", "n_gpus": 1,
                      "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms, "higher_is_better": True,
                      "scaling": "weak", "vs_baseline": None, "dtype": args.compute, "data": "synthetic",
                      "timing": "eager launches of the whole step (inputs resident in HBM); graph replay also given",
                      "config": {"workload": w.name, "N": N, "m": m, "score": "l2", "mu": 0.95, "wd": 0.0,
                                 "fractions": res},
                      "hbm_pieces_k2048": pieces, "hbm_reference_same_tensors": reference,
                      "fp32_state_f_quarter": fp32_state,
                      "megabatch_f_quarter": mega, "tall_state_columns_vs_rows": tall,
                      "roofline": roof, "cpu_baseline": cpu}), flush=True)


if __name__ == "__main__":
    main()
