#!/usr/bin/env python3
"""Throughput of the MiniMax-M3 pre-attention prologue on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--config all|c1..c5]

A step is one whole prologue call (pre_attn_decode or pre_attn_prefill through
the C ABI) over one batch of synthetic input. The default run measures all five
workloads and prints one JSON line headlined by the largest one (c5, the
prefill of 8192 tokens: FP8 TFLOP/s and its fraction of the MFMA peak), with a
record per workload under "configs" (decode: tokens/s and HBM GB/s; prefill:
TFLOP/s), each with its roofline and its CPU baseline.

Per workload: inputs rotate over a pool of distinct weight / activation sets of
at least 512 MB (twice the 256 MB Infinity Cache) and at least one set per timed
step, and a 512 MB copy runs between the graph's upload replay and the timed
replay, so every timed step reads its weight from HBM. The K timed steps are
captured into one HIP graph (as a serving engine replays decode steps); HIP
events around the replay time them, queued right behind the untimed copy so
that the host's submission is not counted. A second, eager pass over the same
pool records HIP events around every launch of the dominant kernel to get its
average duration for the roofline. Prefill records also carry, as context,
the time of the vendor library's plain FP8 GEMM (hipBLASLt) of the same shape,
and the full run the rates plain streaming kernels reach (hbm_context).

Workloads: c1 tiny decode, c2 decode batch, c3 speculative decode, c4 / c5
prefill, and d1, the DSpark drafter's attention (16 requests of 7 draft rows).
"""

from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
HBM_PEAK_GBS = 8000.0
FP8_PEAK_TFLOPS = 5000.0
KEYS = ["c1", "c2", "c3", "c4", "c5"]
DRAFTER = "d1"  # the DSpark drafter's attention: 16 requests x 7 draft rows
BF16_PEAK_TFLOPS = 2500.0
HEADLINE = "c5"  # the largest configuration
METRIC = "decode tokens/s + HBM GB/s (% of peak); prefill FP8 TFLOP/s (% MFMA peak)"


def parse():
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--config", default="all", choices=["all"] + KEYS + [DRAFTER],
                    help="one workload, or all (headlined by c5); d1 is the drafter's attention")
    ap.add_argument("--pool-mb", type=int, default=512)
    ap.add_argument("--cpu-seconds", type=float, default=4.0,
                    help="approximate CPU time of each oracle baseline measurement (0 = skip)")
    ap.add_argument("--head-options", default="none", choices=["none", "static", "fp8q", "nvfp4"],
                    help="time the pre_attn_*_ex head-step options: unit K/V scales, the FP8 q "
                         "output (scale 0.008) besides bf16 q, or NVFP4 caches (global scales "
                         "0.37 / 1.9)")
    ap.add_argument("--no-graph", action="store_true", help="time eager launches instead")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="only run a plain 256 MiB device-to-device copy 10 times (the known-size "
                         "reference for the HBM byte counters) and exit")
    return ap.parse_args()


def calibrate_copy():
    import torch

    n = 256 << 20
    src = torch.empty(n, dtype=torch.uint8, device="cuda:0").fill_(1)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(10):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"calibration": "copy", "bytes_read_per_launch": n,
                      "bytes_written_per_launch": n, "launches": 10}))


def hbm_context(reps=20):
    """What plain streaming kernels reach on this machine, after the same 512 MB
    cache flush (HIP events, median of `reps`): a 354 MB device-to-device copy
    (708 MB moved) and torch's bf16 add of two [8192, 6144] tensors (2 reads +
    1 write, 302 MB, the prefill norm pass's shape). Context for the HBM
    roofline fractions, which use the published 8 TB/s."""
    import torch

    dev = "cuda:0"
    flush_src = torch.empty(512 << 20, dtype=torch.uint8, device=dev)
    flush_dst = torch.empty_like(flush_src)

    def median_us(fn):
        for _ in range(3):
            fn()
        ts = []
        for _ in range(reps):
            flush_dst.copy_(flush_src)
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record()
            fn()
            e1.record()
            torch.cuda.synchronize()
            ts.append(e0.elapsed_time(e1) * 1e3)
        ts.sort()
        return ts[len(ts) // 2]

    g = torch.Generator(device=dev).manual_seed(0)  # random bits, like the workloads' data
    x = torch.randn(354_000_000 // 4, dtype=torch.float32, device=dev, generator=g)
    y = torch.empty_like(x)
    copy_us = median_us(lambda: y.copy_(x))
    copy_bytes = 2 * x.numel() * 4
    del x, y
    a = torch.randn(8192, 6144, device=dev, generator=g).to(torch.bfloat16)
    b = torch.randn(8192, 6144, device=dev, generator=g).to(torch.bfloat16)
    c = torch.empty_like(a)
    add_us = median_us(lambda: torch.add(a, b, out=c))
    add_bytes = 3 * a.numel() * 2
    del a, b, c, flush_src, flush_dst
    torch.cuda.empty_cache()
    return {"what": "plain streaming kernels on random data after a 512 MB flush, HIP events, median of %d" % reps,
            "copy_bytes": copy_bytes, "copy_us": round(copy_us, 2),
            "copy_tbs": round(copy_bytes / copy_us / 1e6, 3),
            "bf16_add_bytes": add_bytes, "bf16_add_us": round(add_us, 2),
            "bf16_add_tbs": round(add_bytes / add_us / 1e6, 3)}


def algorithmic(wl, structure=0, head_options="none"):
    """(bytes per call, bytes of the dominant kernel per launch, flops per call,
    the dominant kernel's name).

    The decode projection always has a launch of its own; the input norm, the
    head epilogue or both may share it (pa_decode_structure flags). Its launch
    is the dominant kernel: the FP8 weight and activation codes, plus the
    ar / res rows, gamma and the bf16 residual out when the norm is in it, or
    the outputs, cache inserts and per-token inputs of the epilogue when that
    is in it (in place of the activation codes from the norm launch)."""
    S, K, nkv = wl.tokens, wl.hidden, wl.nkv
    N = (19 * nkv + 1) * 128
    norm_bytes = 4 * S * K + 2 * S * K + 2 * K  # ar + res in, h_out out, g_in
    # cache writes: FP8 K and V codes + scales per KV head and the index row, or
    # NVFP4 slots of 64 data + 8 scale bytes for K, V and index_k
    cache_bytes = S * (2 * nkv + 1) * 72 if head_options == "nvfp4" else S * nkv * (256 + 8) + 128 * S
    call_bytes = (N * K + 4 * N + norm_bytes + 4 * 256
                  + S * 16 * nkv * 256 + S * nkv * 256 + cache_bytes
                  + 128 * S + 16 * S)
    if head_options == "fp8q":
        call_bytes += S * 16 * nkv * 128
    flops = 2 * S * N * K
    if wl.mode == "prefill":
        call_bytes += N * K // 32 - 4 * N  # E8M0 block scales instead of row scales
        return call_bytes, N * K + S * K, flops, "prefill_gemm"
    norm_fused = bool(structure & 1)
    epi_fused = bool(structure & 2)
    if norm_fused and epi_fused:
        return call_bytes, call_bytes, flops, "decode_fused (norm + GEMV + head epilogue)"
    if norm_fused:
        return call_bytes, N * K + norm_bytes, flops, "decode_fused (norm + GEMV)"
    if epi_fused:
        return call_bytes, call_bytes - norm_bytes + S * K, flops, "decode_gemv_epi (GEMV + head epilogue)"
    return call_bytes, N * K + S * K, flops, "decode_gemv"


def source_sha(mode: str) -> str:
    name = {"decode": "pa_decode.hip", "prefill": "pa_prefill.hip", "drafter": "pa_drafter.hip"}[mode]
    with open(os.path.join(ROOT, "kv_residual_add_amd", "csrc", name), "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def _profile_record(fname: str, key: str, mode: str):
    """A committed rocprofv3 figure for workload `key`, if it was taken on the
    current kernel source."""
    try:
        with open(os.path.join(ROOT, "profiles", fname)) as f:
            rec = json.load(f).get(key)
    except (OSError, ValueError):
        return None
    if not rec or rec.get("source_sha") != source_sha(mode):
        return None
    return rec


def cpu_baseline(wl, inp, budget_s: float, one_core: bool = False):
    """The oracle, as it stands, on a bounded sample of the same workload: every
    token for decode, 64 tokens for prefill. With one_core, BLAS runs on one
    thread; otherwise on all of them."""
    import contextlib

    import numpy as np

    import oracle
    from tests import parity

    try:
        from threadpoolctl import threadpool_info, threadpool_limits
    except Exception:  # pragma: no cover - threadpoolctl missing
        threadpool_info, threadpool_limits = None, None
    ctx = threadpool_limits(limits=1, user_api="blas") if (one_core and threadpool_limits) \
        else contextlib.nullcontext()
    S = wl.tokens
    rows = np.arange(S) if wl.mode == "decode" else np.arange(min(S, 64))
    sub = inp if len(rows) == S else parity.subset(inp, rows)
    fn = oracle.decode if wl.mode == "decode" else oracle.prefill
    times = []
    with ctx:
        cores = 1
        if threadpool_info is not None:
            blas = [i for i in threadpool_info() if i.get("user_api") == "blas"]
            cores = max((i["num_threads"] for i in blas), default=1)
        t_start = time.perf_counter()
        while True:
            t0 = time.perf_counter()
            fn(sub)
            times.append(time.perf_counter() - t0)
            if (time.perf_counter() - t_start > budget_s and len(times) >= 3) or len(times) >= 1000:
                break
    t = float(np.median(times))
    N = (19 * wl.nkv + 1) * 128
    if wl.mode == "decode":
        value, unit = len(rows) / t, "tokens/s"
    else:
        value, unit = 2 * len(rows) * N * wl.hidden / t / 1e12, "TFLOP/s"
    return {"value": value, "unit": unit, "cores": int(cores), "kind": "oracle",
            "sample": f"{len(rows)} of {S} tokens per oracle call, median of {len(times)} calls "
                      f"({sum(times):.1f} s), float64 NumPy"}


def library_gemm(M, N, K, dev, flush_src, flush_dst, reps):
    """A plain FP8 GEMM of the projection's shape from the vendor library
    (hipBLASLt through torch._scaled_mm: E4M3 operands, row-wise float32 scales,
    bf16 out, no epilogue, no block scales), each launch timed by HIP events
    after the same 512 MB cache flush. Context for the fused GEMM's time (what a
    tuned library reaches on this shape and chip), not a baseline of the path."""
    import numpy as np
    import torch

    g = torch.Generator(device=dev).manual_seed(0)
    a = (torch.randn(M, K, device=dev, generator=g) * 0.5).to(torch.float8_e4m3fn)
    b = (torch.randn(N, K, device=dev, generator=g) * 0.5).to(torch.float8_e4m3fn)
    sa = torch.ones(M, 1, device=dev)
    sb = torch.ones(1, N, device=dev)

    def gemm():
        return torch._scaled_mm(a, b.t(), scale_a=sa, scale_b=sb, out_dtype=torch.bfloat16)

    try:
        for _ in range(3):
            gemm()
        torch.cuda.synchronize()
    except RuntimeError as e:  # a torch build without FP8 GEMMs for this device
        return {"error": str(e)[:200]}
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(reps)]
    for e0, e1 in evs:
        flush_dst.copy_(flush_src)
        e0.record()
        gemm()
        e1.record()
    torch.cuda.synchronize()
    ms = float(np.mean([e0.elapsed_time(e1) for e0, e1 in evs]))
    tflops = 2.0 * M * N * K / (ms / 1e3) / 1e12
    del a, b
    return {"what": "hipBLASLt FP8 GEMM via torch._scaled_mm, E4M3 x E4M3, row-wise scales, bf16 out, "
                    "same M x N x K, no epilogue; mean of per-launch hip events after a 512 MB flush",
            "M": M, "N": N, "K": K, "launches": reps, "kernel_ms": round(ms, 5),
            "tflops": round(tflops, 1), "frac": round(tflops / FP8_PEAK_TFLOPS, 4)}


def run_config(key, args):
    """Measures one workload; returns its record."""
    import numpy as np
    import torch

    import synth
    from kv_residual_add_amd import _binding as B
    from kv_residual_add_amd.runner import Problem

    wl = synth.named_config(key)
    inp = synth.make_workload(wl, seed=0)
    if args.head_options == "static":
        inp["static_kv_scale"] = True
    elif args.head_options == "fp8q":
        inp["q_fp8_scale"] = 0.008
    elif args.head_options == "nvfp4":
        inp = synth.with_nvfp4_caches(inp, 0.37, 1.9)
    prob = Problem(inp)
    dev = prob.device
    S, K = wl.tokens, wl.hidden
    N = prob.N
    structure = B.pa_decode_structure(prob.dims) if prob.mode == B.PA_MODE_DECODE else 0
    call_bytes, kernel_bytes, flops, kernel_name = algorithmic(wl, structure, args.head_options)

    # rotating pool of distinct weight + activation sets: >= pool_mb, and one
    # set per timed step when that is more
    set_bytes = prob.w_packed.numel() + prob.w_scales.numel() * prob.w_scales.element_size() \
        + 4 * S * K
    n_sets = max(2, math.ceil(args.pool_mb * 2**20 / set_bytes))
    if set_bytes < 256 << 20:  # a set smaller than the Infinity Cache: one per timed step
        n_sets = max(n_sets, min(args.steps, 64))
    w_dev = torch.from_numpy(inp["w"]).to(dev)
    sets = []
    for i in range(n_sets):
        sh = (i * 128) % K
        wp = torch.empty_like(prob.w_packed)
        if prob.mode == B.PA_MODE_DECODE:
            B.pa_pack_weight_decode(torch.roll(w_dev, sh, dims=1).contiguous(), wp)
            ws = torch.roll(prob.w_scales, i)
        else:
            we = torch.from_numpy(inp["w_e8m0"]).to(dev)
            ws = torch.empty_like(prob.w_scales)
            B.pa_pack_weight_prefill(torch.roll(w_dev, sh, dims=1).contiguous(),
                                     torch.roll(we, sh // 32, dims=1).contiguous(), wp, ws)
        ar = torch.roll(prob.t["ar"], sh, dims=1).contiguous()
        res = torch.roll(prob.t["res"], sh, dims=1).contiguous()
        sets.append((wp, ws, ar, res))
    del w_dev
    flush_src = torch.empty(512 << 20, dtype=torch.uint8, device=dev)
    flush_dst = torch.empty_like(flush_src)
    torch.cuda.synchronize()

    def step(i):
        wp, ws, ar, res = sets[i % n_sets]
        prob.run(w_packed=wp, w_scales=ws, ar=ar, res=res)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()

    # timed region: K steps
    graph = None
    if not args.no_graph:
        graph = torch.cuda.CUDAGraph()
        cap = torch.cuda.Stream()
        cap.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(cap):
            with torch.cuda.graph(graph, stream=cap):
                for i in range(args.steps):
                    step(args.warmup + i)
        torch.cuda.synchronize()
        graph.replay()  # first replay uploads the graph; not timed
        torch.cuda.synchronize()
    t_ev0 = torch.cuda.Event(enable_timing=True)
    t_ev1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    # The cache flush (the Infinity Cache then holds none of the timed steps'
    # sets) is untimed GPU work queued just ahead of the timed steps: the GPU
    # copies while the host enqueues them, so the events around the K steps time
    # the steps themselves, not the host's submission latency.
    flush_dst.copy_(flush_src)
    t_ev0.record()
    if graph is not None:
        graph.replay()
    else:
        for i in range(args.steps):
            step(args.warmup + i)
    t_ev1.record()
    torch.cuda.synchronize()
    elapsed = t_ev0.elapsed_time(t_ev1) / 1e3
    del graph

    # eager pass with HIP events around every launch of the dominant kernel
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(args.steps)]
    for a, b in evs:  # torch creates an event at its first record
        a.record()
        b.record()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    flush_dst.copy_(flush_src)
    torch.cuda.synchronize()
    e0.record()
    for i in range(args.steps):
        B.pa_set_kernel_events(*evs[i])
        step(args.warmup + i)
    e1.record()
    B.pa_set_kernel_events(None, None)
    torch.cuda.synchronize()
    kern_ms = float(np.mean([a.elapsed_time(b) for a, b in evs]))
    eager_s = e0.elapsed_time(e1) / 1e3
    B.pa_workspace_status(prob.workspace)  # raises if an in-kernel wait gave up

    traffic_rec = _profile_record("traffic.json", key, wl.mode) if args.head_options == "none" else None
    prof_rec = _profile_record("kernel_times.json", key, wl.mode) if args.head_options == "none" else None
    prof_ms = prof_rec["avg_ns"] / 1e6 if prof_rec else None
    if wl.mode == "decode":
        metric, unit = "decode tokens/s", "tokens/s"
        value = S * args.steps / elapsed
        work, peak, bound, runit = kernel_bytes / 1e9, HBM_PEAK_GBS, "hbm", "GB/s"
        extra = {"step_hbm_gbs": round(call_bytes * args.steps / elapsed / 1e9, 1),
                 "step_hbm_frac": round(call_bytes * args.steps / elapsed / 1e9 / HBM_PEAK_GBS, 4),
                 "algorithmic_bytes_per_step": call_bytes}
        per_launch = {"algorithmic_bytes_per_launch": kernel_bytes}
    else:
        metric, unit = "prefill FP8 TFLOP/s", "TFLOP/s"
        value = flops * args.steps / elapsed / 1e12
        work, peak, bound, runit = flops / 1e12, FP8_PEAK_TFLOPS, "mfma", "TFLOP/s"
        extra = {"step_tflops_frac": round(value / FP8_PEAK_TFLOPS, 4),
                 "tokens_per_s": round(S * args.steps / elapsed, 1)}
        per_launch = {"algorithmic_flops_per_launch": flops}
    achieved = work / (kern_ms / 1e3)
    roof = {"bound": bound, "achieved": round(achieved, 1), "peak": peak, "unit": runit,
            "frac": round(achieved / peak, 4),
            "traffic": traffic_rec.get("bytes_per_launch") if traffic_rec else None,
            "kernel": kernel_name, "kernel_ms": round(kern_ms, 5), "kernel_ms_from": "hip events, eager pass",
            **per_launch}
    if prof_ms:
        roof["kernel_ms_rocprof"] = round(prof_ms, 5)
        roof["frac_rocprof"] = round(work / (prof_ms / 1e3) / peak, 4)
    rec = {
        "workload": wl.name, "metric": metric, "value": round(value, 3), "unit": unit,
        "ms_per_step": round(elapsed / args.steps * 1e3, 5),
        "dtype": "fp8_e4m3" if wl.mode == "decode" else "mxfp8_e4m3",
        "config": {"workload": wl.name, "tokens": S, "hidden": K, "nkv": wl.nkv, "n_rows": N,
                   "pool_sets": n_sets, "pool_mb": round(n_sets * set_bytes / 2**20),
                   "distinct_sets_timed": min(args.steps, n_sets), "cache_flush_mb": 512,
                   "timing": ("hip graph replay" if not args.no_graph else "eager")
                             + "; hip events around the K steps, queued behind the untimed cache flush",
                   **({} if args.head_options == "none" else {"head_options": args.head_options})},
        "roofline": roof,
        "eager_ms_per_step": round(eager_s / args.steps * 1e3, 5),
        **extra,
    }
    if wl.mode == "prefill" and args.head_options == "none":
        rec["library_fp8_gemm"] = library_gemm(S, N, K, dev, flush_src, flush_dst, min(args.steps, 20))
    del sets, prob, flush_src, flush_dst
    torch.cuda.empty_cache()
    if args.cpu_seconds > 0:
        rec["cpu_baseline"] = cpu_baseline(wl, inp, args.cpu_seconds)
        if wl.mode == "decode":
            rec["cpu_baseline_1core"] = cpu_baseline(wl, inp, args.cpu_seconds, one_core=True)
    else:
        rec["cpu_baseline"] = None
    return rec


def drafter_inputs(seed=0):
    """d1: 16 requests of 7 draft rows, seq_len ~ U[2048, 12000], 2-block partitions."""
    import synth
    return synth.make_drafter(16, 12000, seed=seed, split=2, min_seq=2048)


def drafter_work(inp):
    """(algorithmic bytes, flops) of one drafter attention call: the K and V codes
    of every key some row of its request sees (256 bytes a key), the rows' q codes
    and MXFP8 outputs, the new rows' bf16 q / k / v; flops 2 x 2 x 16 x 128 per
    (row, visible key) for Q K^T and P V."""
    from oracle import drafter as D

    pos = inp["positions"]
    keys, pairs = 0, 0
    for r in range(inp["requests"]):
        lo, hi, _, _ = D.window(int(pos[7 * r]), int(inp["seq_lens"][r]))
        keys += hi - lo + 1
        for j in range(7):
            qp = int(pos[7 * r + j])
            pairs += hi - max(lo, qp - 4095) + 1
    T = 7 * inp["requests"]
    nbytes = keys * 256 + T * (2048 + 2048 + 64) + T * (16 * 256 + 2 * 256)
    return nbytes, 4 * 16 * 128 * pairs


def run_drafter(args):
    import numpy as np
    import torch

    from kv_residual_add_amd import _binding as B
    from kv_residual_add_amd.runner import DrafterProblem

    inp = drafter_inputs()
    nbytes, flops = drafter_work(inp)
    prob = DrafterProblem(inp)
    # a pool of caches (and block tables shifted over them) past the Infinity Cache
    set_bytes = prob.t["kv_cache"].numel()
    n_sets = max(2, math.ceil(args.pool_mb * 2**20 / set_bytes), min(args.steps, 64))
    caches = [prob.t["kv_cache"]] + [prob.t["kv_cache"].clone() for _ in range(n_sets - 1)]
    flush_src = torch.empty(512 << 20, dtype=torch.uint8, device=prob.device)
    flush_dst = torch.empty_like(flush_src)

    def step(i):
        prob.run(kv_cache=caches[i % n_sets])

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    cap = torch.cuda.Stream()
    cap.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(cap):
        with torch.cuda.graph(graph, stream=cap):
            for i in range(args.steps):
                step(args.warmup + i)
    torch.cuda.synchronize()
    graph.replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    flush_dst.copy_(flush_src)  # untimed, queued ahead of the timed steps (as for the prologue)
    e0.record()
    graph.replay()
    e1.record()
    torch.cuda.synchronize()
    elapsed = e0.elapsed_time(e1) / 1e3
    del graph
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    for a, b in evs:
        a.record()
        b.record()
    flush_dst.copy_(flush_src)
    torch.cuda.synchronize()
    for i in range(args.steps):
        B.pa_set_kernel_events(*evs[i])
        step(args.warmup + i)
    B.pa_set_kernel_events(None, None)
    torch.cuda.synchronize()
    kern_ms = float(np.mean([a.elapsed_time(b) for a, b in evs]))
    rows = 7 * inp["requests"]
    gbs = nbytes / (kern_ms / 1e3) / 1e9
    tfs = flops / (kern_ms / 1e3) / 1e12
    prof = _profile_record("kernel_times.json", DRAFTER, "drafter")
    traffic_rec = _profile_record("traffic.json", DRAFTER, "drafter")
    rec = {
        "workload": "drafter_attention_r16_seq2k_12k_split2", "metric": "drafter rows/s", "unit": "rows/s",
        "value": round(rows * args.steps / elapsed, 1), "ms_per_step": round(elapsed / args.steps * 1e3, 5),
        "dtype": "fp8_e4m3 (bf16 MFMA on exact widening)",
        "config": {"workload": "drafter_attention_r16_seq2k_12k_split2", "requests": inp["requests"],
                   "rows": rows, "split_blocks": inp["split"], "seq_lens": inp["seq_lens"].tolist(),
                   "pool_sets": n_sets, "cache_flush_mb": 512,
                   "timing": "hip graph replay; hip events around the K steps, queued behind the untimed cache flush"},
        "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(gbs / HBM_PEAK_GBS, 4),
                     "traffic": traffic_rec.get("bytes_per_launch") if traffic_rec else None, "kernel": "drafter_split",
                     "kernel_ms": round(kern_ms, 5), "kernel_ms_from": "hip events, eager pass",
                     "algorithmic_bytes_per_launch": nbytes, "algorithmic_flops_per_launch": flops,
                     "mfma_bf16_tflops": round(tfs, 1), "mfma_bf16_frac": round(tfs / BF16_PEAK_TFLOPS, 4)},
    }
    if prof:
        rec["roofline"]["kernel_ms_rocprof"] = round(prof["avg_ns"] / 1e6, 5)
        rec["roofline"]["frac_rocprof"] = round(nbytes / (prof["avg_ns"] / 1e9) / 1e9 / HBM_PEAK_GBS, 4)
    del caches, prob, flush_src, flush_dst
    torch.cuda.empty_cache()
    if args.cpu_seconds > 0:
        from oracle import drafter as D
        import synth

        sub = synth.make_drafter(2, 12000, seed=1, split=2, min_seq=2048)
        cores = 1
        try:
            from threadpoolctl import threadpool_info
            blas = [i for i in threadpool_info() if i.get("user_api") == "blas"]
            cores = max((i["num_threads"] for i in blas), default=1)
        except ImportError:
            pass
        times = []
        t_start = time.perf_counter()
        while True:
            t1 = time.perf_counter()
            D.attention(sub)
            times.append(time.perf_counter() - t1)
            if (time.perf_counter() - t_start > args.cpu_seconds and len(times) >= 2) or len(times) >= 100:
                break
        rec["cpu_baseline"] = {"value": 14 / float(np.median(times)), "unit": "rows/s", "cores": int(cores),
                               "kind": "oracle",
                               "sample": f"2 requests (14 rows) of the same recipe per call, median of "
                                         f"{len(times)} calls ({sum(times):.1f} s), float64 NumPy"}
    return rec


def main():
    args = parse()
    if args.calibrate_copy:
        calibrate_copy()
        return
    if args.gpus != 1:
        print(f"bench.py: this build measures one GPU only (asked for --gpus {args.gpus}); "
              "the prologue shards by heads with no exchange, so per-GPU throughput is the "
              "figure that matters", file=sys.stderr)
        sys.exit(2)
    import torch

    torch.cuda.set_device(0)
    keys = KEYS + [DRAFTER] if args.config == "all" else [args.config]
    head = HEADLINE if args.config == "all" else args.config
    recs = {}
    for key in keys:
        print(f"bench: {key} ...", file=sys.stderr, flush=True)
        recs[key] = run_drafter(args) if key == DRAFTER else run_config(key, args)
        r = recs[key]
        print(f"bench: {key} {r['value']:.1f} {r['unit']}, {r['ms_per_step'] * 1e3:.2f} us a step, "
              f"roofline frac {r['roofline']['frac']}", file=sys.stderr, flush=True)
    h = recs[head]
    line = {
        "metric": METRIC, "value": h["value"], "unit": h["unit"], "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": h["ms_per_step"],
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": h["dtype"], "data": "synthetic",
        "config": dict(h["config"], headline=f"{head} ({h['metric']})"),
        "roofline": h["roofline"],
        "cpu_baseline": h.get("cpu_baseline"),
    }
    if len(keys) > 1:
        line["configs"] = recs
        line["hbm_context"] = hbm_context()
    else:
        line.update({k: v for k, v in h.items() if k not in line and k not in ("workload", "metric", "value",
                                                                                  "unit", "config")})
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
