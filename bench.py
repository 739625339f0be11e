#!/usr/bin/env python3
"""Benchmark of the decode hot path on one MI355X.

Workload: batch-64 paged GQA decode (32 query heads over 8 KV heads, head_dim
128), slot-list lengths uniform in [2048, 8192], 16 groups of 4 requests
sharing a 1024-slot prefix, scattered slots in a 600k-slot bf16 pool, and 36
layers per step with one pa_plan reused by all of them; every layer has its
own pools, so caches cannot serve one layer's K/V to the next.  Inputs are
seeded synthetic data (workloads.py), resident in HBM before timing starts.

A step = pa_plan (host partition + async upload of the tables) + the 36
pa_decode_run calls, replayed from a HIP graph captured once (`--eager`:
launched one by one).
The JSON line reports:
  value            algorithmic HBM bytes of the step / step time (GB/s)
  us_per_step_layer  step time / 36
  roofline         the decode kernel alone: algorithmic bytes per launch /
                   its average duration from HIP events recorded around each
                   launch on the launch stream (in a second pass of the same
                   steps, since those events keep consecutive launches from
                   overlapping), against 8 TB/s; `traffic` comes from
                   committed rocprofv3 counters when they were taken on the
                   current kernel source, else null
  cpu_baseline     the fp64 oracle on the host cores, on layer 0 of the same
                   workload (all rows), repeated for about --cpu-seconds
Algorithmic bytes per layer = unique slots x Hkv x D x 2 (K) x 2 (V) + list
entries x 4 (slot ids) + B x Hq x D x 2 (q) + B x Hq x D x 4 (out) + (B+1) x 4.

Other decode workloads (`--workload single_request | batch8 | hd256`): one
request of 256 slots; 8 requests of 512..4096 slots (Qwen3-4B head shapes);
32 requests of 1024..16384 slots at head_dim 256 -- each 36 layers per step
with per-layer pools.  Each step's 36 layer runs are replayed from one
captured HIP graph (pa_plan stays outside the graph; the CUDA Graph decode
of the Agent-Infer page, section "CUDA Graph 解码"); `--eager` launches them
one by one instead.
`--workload prefill_chunk512 | prefill_chunk64` measures the chunked-prefill
kernel (MFMA roofline); `--workload append` the KV append + RoPE of a
batch-64 step; `--workload system_prompt --cascade` the cascade decode of 64
requests sharing a 4096-slot prompt; `--workload copy --copy-gib N` runs a
plain device copy of N GiB (for calibrating the HBM counters).  `--kv fp8`
runs a decode, prefill or append workload over pools of OCP FP8 E4M3 codes
(per-pool scales 0.25 for K and 0.5 for V) instead of bf16.
"""
from __future__ import annotations

import argparse
import gc
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "decode-attn µs/step/layer + achieved HBM GB/s (% of MI355X peak), batch 64"
HBM_PEAK_GBS = 8000.0
PREFILL_METRIC = "chunked-prefill attention TFLOP/s (% of MI355X dense bf16 MFMA peak)"
BF16_MFMA_PEAK_TFLOPS = 2500.0
PREFILL_LAYERS = 8
CSRC = os.path.join(ROOT, "paged_gqa_decode_pa_amd", "csrc")
COUNTERS = os.path.join(ROOT, "profiles", "decode_b64_counters.json")
DECODE_COUNTERS = {
    "b64_l2048_8192_prefix16x4x1024_36layers": COUNTERS,
    "b64_l4096_8192_prefix16x4x1024_36layers": os.path.join(ROOT, "profiles", "decode_b64_4k8k_counters.json"),
    "b64_l2048_8192_prefix16x4x1024_36layers_fp8kv": os.path.join(ROOT, "profiles", "decode_b64_fp8_counters.json"),
}
DECODE_SOURCES = ("decode.hip", "pa_internal.h")
PREFILL_COUNTERS = {
    "prefill_8x4096_chunk512": os.path.join(ROOT, "profiles", "prefill_chunk512_counters.json"),
    "prefill_8x4096_chunk64": os.path.join(ROOT, "profiles", "prefill_chunk64_counters.json"),
    "prefill_8x4096_chunk512_fp8kv": os.path.join(ROOT, "profiles", "prefill_chunk512_fp8_counters.json"),
    "prefill_8x4096_chunk64_fp8kv": os.path.join(ROOT, "profiles", "prefill_chunk64_fp8_counters.json"),
}
# the partition decides how many partial rows a prefill launch writes
PREFILL_SOURCES = ("prefill.hip", "pa_internal.h", "plan.cpp")


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def cpu_model() -> str:
    """The host CPU's model name (from /proc/cpuinfo), or the platform's."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    import platform
    return platform.processor() or "unknown"


def algorithmic_bytes(spec, kv_indptr, kv_indices, kv_elem_bytes: int = 2) -> int:
    import numpy as np
    B, Hq, Hkv, D = spec.batch, spec.num_qo_heads, spec.num_kv_heads, spec.head_dim
    unique = int(np.unique(kv_indices).size)
    return (unique * Hkv * D * kv_elem_bytes * 2 + int(kv_indptr[-1]) * 4 + B * Hq * D * 2
            + B * Hq * D * 4 + (B + 1) * 4)


def kernel_source_hash(names=DECODE_SOURCES) -> str:
    h = hashlib.sha256()
    for name in names:
        with open(os.path.join(CSRC, name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def traffic_per_launch(path=COUNTERS, sources=DECODE_SOURCES):
    """HBM bytes per launch from committed counters, if they match the kernel source."""
    if path is None or not os.path.exists(path):
        return None
    with open(path) as f:
        c = json.load(f)
    if c.get("kernel_source_sha256") != kernel_source_hash(sources):
        return None
    return int((c["fetch_kib_per_dispatch"] * c["fetch_scale"] +
                c["write_kib_per_dispatch"] * c["write_scale"]) * 1024)


def run_copy(gib: float, steps: int):
    import torch
    n = int(gib * (1 << 30)) // 4
    src = torch.ones(n, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(2):
        dst.copy_(src)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        dst.copy_(src)
    torch.cuda.synchronize()
    dt = (time.perf_counter() - t0) / steps
    log(f"copy {gib} GiB: {dt * 1e3:.3f} ms, {2 * n * 4 / dt / 1e9:.1f} GB/s (read+write)")


def cpu_baseline(case, spec, bytes_per_layer, seconds, gpu_out_layer0, fp8=False):
    import numpy as np

    import oracle
    import workloads as W
    ref = oracle.load()
    qb = W.bits(case.q)
    if fp8:   # E4M3 code pools, widened by the oracle inside the timed loop
        kc = W.codes(case.k_pools[0])
        vc = W.codes(case.v_pools[0])
    else:
        kb = W.bits(case.k_pools[0])
        vb = W.bits(case.v_pools[0])
    reps = 0
    t0 = time.perf_counter()
    out = None
    while True:
        if fp8:
            out, _ = ref.decode_fp8(qb, kc, vc, case.kv_indptr, case.kv_indices, case.sm_scale,
                                    W.FP8_K_SCALE, W.FP8_V_SCALE, spec.num_kv_heads)
        else:
            out, _ = ref.decode(qb, kb, vb, case.kv_indptr, case.kv_indices, case.sm_scale,
                                spec.num_kv_heads)
        reps += 1
        if time.perf_counter() - t0 >= seconds:
            break
    dt = time.perf_counter() - t0
    err = float(np.abs(gpu_out_layer0 - out).max())
    return {
        "value": round(bytes_per_layer * reps / dt / 1e9, 3),
        "unit": "GB/s",
        "cores": ref.num_threads(),
        "cpu_model": cpu_model(),
        "host_cpus": os.cpu_count(),
        "kind": "oracle",
        "us_per_layer": round(dt / reps * 1e6, 1),
        "sample": f"layer 0 of the same workload, all {spec.batch}x{spec.num_qo_heads} rows, "
                  f"{reps} repetition(s), {dt:.1f} s"
                  + (" (the oracle reads the E4M3 codes directly)" if fp8 else ""),
    }, err


def prefill_flops(spec, qo_indptr, kv_indptr) -> int:
    """4*D flops (QK^T and PV) per (query row, visible list entry)."""
    total = 0
    for b in range(spec.batch):
        C = int(qo_indptr[b + 1] - qo_indptr[b])
        L = int(kv_indptr[b + 1] - kv_indptr[b])
        P = L - C
        total += C * (P + 1) + C * (C - 1) // 2   # row i sees P + i + 1 entries
    return total * spec.num_qo_heads * 4 * spec.head_dim


def prefill_bytes(spec, qo_indptr, kv_indices, kv_elem_bytes: int = 2) -> int:
    import numpy as np
    T = int(qo_indptr[-1])
    unique = int(np.unique(kv_indices).size)
    Hq, Hkv, D = spec.num_qo_heads, spec.num_kv_heads, spec.head_dim
    return unique * Hkv * D * kv_elem_bytes * 2 + int(kv_indices.size) * 4 + T * Hq * D * (2 + 4)


def cpu_baseline_prefill(case, spec, flops_per_row_entry, seconds, fp8=False):
    """fp64 oracle on a bounded sample of rows: the last chunk token of every
    request, all heads (the rows that see the most entries), repeated (over
    the E4M3 codes with fp8)."""
    import numpy as np

    import oracle
    import workloads as W
    ref = oracle.load()
    qb = W.bits(case.q)
    kb, vb = (W.codes(case.k_pool), W.codes(case.v_pool)) if fp8 else (W.bits(case.k_pool), W.bits(case.v_pool))
    Hq = spec.num_qo_heads
    rows = []
    entries = 0
    for b in range(spec.batch):
        t = int(case.qo_indptr[b + 1]) - 1
        L = int(case.kv_indptr[b + 1] - case.kv_indptr[b])
        rows.extend(t * Hq + h for h in range(Hq))
        entries += L * Hq
    rows = np.asarray(rows, np.int32)
    reps = 0
    t0 = time.perf_counter()
    while True:
        if fp8:
            ref.prefill_fp8(qb, kb, vb, case.qo_indptr, case.kv_indptr, case.kv_indices, case.sm_scale,
                            W.FP8_K_SCALE, W.FP8_V_SCALE, spec.num_kv_heads, sel=rows)
        else:
            ref.prefill(qb, kb, vb, case.qo_indptr, case.kv_indptr, case.kv_indices, case.sm_scale,
                        spec.num_kv_heads, sel=rows)
        reps += 1
        if time.perf_counter() - t0 >= seconds:
            break
    dt = time.perf_counter() - t0
    return {
        "value": round(entries * flops_per_row_entry * reps / dt / 1e12, 5),
        "unit": "TFLOP/s",
        "cores": ref.num_threads(),
        "cpu_model": cpu_model(),
        "host_cpus": os.cpu_count(),
        "kind": "oracle",
        "sample": f"{rows.size} rows (last chunk token of each request, all heads), "
                  f"{reps} repetition(s), {dt:.1f} s",
    }


def run_prefill_bench(args):
    import numpy as np
    import torch

    import paged_gqa_decode_pa_amd as pa
    import workloads as W

    spec = W.PREFILL_CHUNK512 if args.workload == "prefill_chunk512" else W.PREFILL_CHUNK64
    layers = args.layers or PREFILL_LAYERS
    dev = torch.device("cuda", 0)
    log(f"generating {spec.name}")
    case = W.make_prefill_case(spec, dev)
    T = int(case.qo_indptr[-1])
    B, Hq, Hkv, D = spec.batch, spec.num_qo_heads, spec.num_kv_heads, spec.head_dim
    fp8 = args.kv == "fp8"
    if fp8:
        # the same workload over pools of E4M3 codes (N(0,1) / scale, nearest even)
        case.k_pool = case.v_pool = None
        case.k_pool, case.v_pool = W.make_pools_e4m3(spec.num_slots, Hkv, D, W.layer_seed(spec.seed, 0), dev)
    idx = torch.as_tensor(case.kv_indices, device=dev)
    flops = prefill_flops(spec, case.qo_indptr, case.kv_indptr)
    nbytes = prefill_bytes(spec, case.qo_indptr, case.kv_indices, 1 if fp8 else 2)
    outs = [torch.empty((T, Hq, D), dtype=torch.float32, device=dev) for _ in range(layers)]
    plan = pa.Plan(B, int(case.kv_indptr[-1]), Hq, Hkv, D, max_q_total=T)
    stream = torch.cuda.current_stream(dev)

    def step():
        plan.plan(case.kv_indptr, case.qo_indptr, flags=args.flags, stream=stream)
        for layer in range(layers):
            if fp8:
                plan.prefill_fp8(case.q, case.k_pool, case.v_pool, idx, case.sm_scale, W.FP8_K_SCALE,
                                 W.FP8_V_SCALE, outs[layer], stream=stream)
            else:
                plan.prefill(case.q, case.k_pool, case.v_pool, idx, case.sm_scale, outs[layer],
                             stream=stream)

    gc.collect()
    gc.disable()   # no collector pauses while steps are issued (see the decode bench)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    marks = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    marks[0].record(stream)
    for i in range(args.steps):
        step()
        marks[i + 1].record(stream)
    torch.cuda.synchronize()
    gc.enable()
    ms_per_step = marks[0].elapsed_time(marks[-1]) / args.steps
    step_ms = np.array([marks[i].elapsed_time(marks[i + 1]) for i in range(args.steps)])
    pa.pa_profile_begin(plan.handle, args.steps * layers)
    torch.cuda.synchronize()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    kernel_ms, launches = pa.pa_profile_end(plan.handle)
    kernel_avg_ms = kernel_ms / max(1, launches)
    log(f"step {ms_per_step:.3f} ms ({ms_per_step * 1e3 / layers:.1f} us per layer); prefill kernel "
        f"avg {kernel_avg_ms * 1e3:.1f} us over {launches} launches")
    value = flops * layers / (ms_per_step * 1e-3) / 1e12
    achieved = flops / (kernel_avg_ms * 1e-3) / 1e12
    result = {
        "metric": PREFILL_METRIC,
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8-e4m3 KV widened to bf16/fp16 MFMA" if fp8 else "bf16",
        "data": "synthetic",
        "config": {
            "workload": spec.name + ("_fp8kv" if fp8 else ""),
            "batch": B, "num_qo_heads": Hq, "num_kv_heads": Hkv, "head_dim": D,
            "cached_len": spec.cached_len, "chunk_len": spec.chunk_len,
            "layers_per_step": layers, "pool_slots": spec.num_slots, "plan_flags": args.flags,
        },
        "us_per_step_layer": round(ms_per_step * 1e3 / layers, 2),
        "step_ms": {"mean": round(ms_per_step, 4), "median": round(float(np.median(step_ms)), 4),
                    "min": round(float(step_ms.min()), 4), "max": round(float(step_ms.max()), 4)},
        "algorithmic_flops_per_layer": flops,
        "algorithmic_bytes_per_layer": nbytes,
        "achieved_hbm_gbs": round(nbytes / (kernel_avg_ms * 1e-3) / 1e9, 1),
        "roofline": {
            "bound": "mfma",
            "achieved": round(achieved, 2),
            "peak": BF16_MFMA_PEAK_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(achieved / BF16_MFMA_PEAK_TFLOPS, 4),
            "traffic": traffic_per_launch(PREFILL_COUNTERS.get(spec.name + ("_fp8kv" if fp8 else "")),
                                          PREFILL_SOURCES),
            "kernel": (f"prefill_kernel<{D},{Hq // Hkv},KV8> (pa_prefill_chunk_run_fp8)" if fp8
                       else f"prefill_kernel<{D},{Hq // Hkv}> (pa_prefill_chunk_run)"),
            "kernel_avg_us": round(kernel_avg_ms * 1e3, 2),
        },
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        log(f"cpu baseline: fp64 oracle on sampled rows for ~{args.cpu_seconds:.0f} s")
        result["cpu_baseline"] = cpu_baseline_prefill(case, spec, 4 * D, args.cpu_seconds, fp8)
    plan.close()
    print(json.dumps(result), flush=True)


def run_append_bench(args):
    """The append step of a batch-64 decode step: 64 new tokens' K/V rows
    (Hkv=8, D=128) written to scattered slots of a 600k-slot pool, K and the
    32 query heads rotated by RoPE; 36 calls (one per layer) per step, the
    query rows rotated again by every call (the arithmetic is the same)."""
    import numpy as np
    import torch

    import paged_gqa_decode_pa_amd as pa
    import workloads as W
    dev = torch.device("cuda", 0)
    T, Hq, Hkv, D, N, layers = 64, 32, 8, 128, 600_000, args.layers or 36
    fp8 = args.kv == "fp8"
    rng = np.random.Generator(np.random.PCG64(1006))
    if fp8:
        k_pools = [W.make_pools_e4m3(N, Hkv, D, 1006 + l, dev) for l in range(min(layers, 4))]
    else:
        k_pools = [W.make_pools(N, Hkv, D, 1006 + l, dev) for l in range(min(layers, 4))]
    k_new = W.normal_bf16((T, Hkv, D), 7, dev)
    v_new = W.normal_bf16((T, Hkv, D), 8, dev)
    q = W.normal_bf16((T, Hq, D), 9, dev)
    loc = torch.as_tensor(rng.permutation(N)[:T].astype(np.int32), device=dev)
    pos = torch.as_tensor(rng.integers(2048, 8193, T).astype(np.int32), device=dev)

    def calls(stream):
        for l in range(layers):
            kp, vp = k_pools[l % len(k_pools)]
            if fp8:
                pa.pa_kv_append_fp8(k_new, v_new, loc, kp, vp, W.FP8_K_SCALE, W.FP8_V_SCALE, positions=pos,
                                    rope_theta=1e6, q=q, stream=stream)
            else:
                pa.pa_kv_append(k_new, v_new, loc, kp, vp, positions=pos, rope_theta=1e6, q=q,
                                stream=stream)

    # the 36 calls of a step replayed from a HIP graph, so the time is the
    # GPU's and not the Python binding's
    side = torch.cuda.Stream(dev)
    side.wait_stream(torch.cuda.current_stream(dev))
    with torch.cuda.stream(side):
        calls(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=side):
        calls(side)
    for _ in range(args.warmup):
        graph.replay()
    torch.cuda.synchronize()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record()
    for _ in range(args.steps):
        graph.replay()
    end.record()
    torch.cuda.synchronize()
    us = start.elapsed_time(end) * 1e3 / (args.steps * layers)
    # K and V read (bf16) and written (bf16, or 1-byte codes), Q read and written; ids
    moved = 2 * T * Hkv * D * (2 + (1 if fp8 else 2)) + 2 * T * Hq * D * 2 + 2 * T * 4
    log(f"append: {us:.2f} us per call ({moved / (us * 1e-6) / 1e9:.1f} GB/s)")
    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline_append(k_new, v_new, q, loc, pos, N, args.cpu_seconds, fp8)
        log(f"cpu baseline {cpu['value']} us per call on {cpu['cores']} threads")
    print(json.dumps({
        "metric": f"append + RoPE µs per layer call, batch-64 decode step, {args.kv} KV", "value": round(us, 3),
        "unit": "us", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "higher_is_better": False, "dtype": "f64", "data": "synthetic",
        "config": {"workload": "append_rope_b64_hkv8_hq32_d128" + ("_fp8kv" if fp8 else ""), "tokens": T,
                   "layers_per_step": layers},
        "bytes_per_call": moved, "vs_baseline": None,
        "roofline": {"bound": "hbm", "achieved": round(moved / (us * 1e-6) / 1e9, 1),
                     "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(moved / (us * 1e-6) / 1e9 / HBM_PEAK_GBS, 5), "traffic": None,
                     "kernel": "append_kernel<true> (pa_kv_append_fp8)" if fp8 else "append_kernel<false> (pa_kv_append)"},
        "cpu_baseline": cpu,
    }), flush=True)


def cpu_baseline_append(k_new, v_new, q, loc, pos, num_slots, seconds, fp8=False):
    """The oracle's RoPE of the call's K and query rows, and the K and V rows
    stored at their slots of host pools (float64, allocated lazily; with fp8,
    the oracle's E4M3 codes into uint8 pools)."""
    import numpy as np

    import oracle
    import workloads as W
    ref = oracle.load()
    kb, vb, qb = W.bits(k_new), W.bits(v_new), W.bits(q)
    slots = loc.cpu().numpy()
    positions = pos.cpu().numpy()
    T, Hkv, D = kb.shape
    k_pool = np.zeros((num_slots, Hkv, D), np.uint8 if fp8 else np.float64)
    v_pool = np.zeros((num_slots, Hkv, D), np.uint8 if fp8 else np.float64)
    reps = 0
    t0 = time.perf_counter()
    while True:
        if fp8:
            k_pool[slots], v_pool[slots], _ = ref.append_e4m3(kb, vb, positions, 1e6, W.FP8_K_SCALE,
                                                              W.FP8_V_SCALE)
        else:
            k_pool[slots] = ref.rope(kb, positions, 1e6)
            v_pool[slots] = (vb.astype(np.uint32) << 16).view(np.float32)   # V rows as they are
        ref.rope(qb, positions, 1e6)
        reps += 1
        if time.perf_counter() - t0 >= seconds:
            break
    dt = time.perf_counter() - t0
    return {"value": round(dt / reps * 1e6, 2), "unit": "us", "cores": ref.num_threads(),
            "cpu_model": cpu_model(), "host_cpus": os.cpu_count(), "kind": "oracle",
            "sample": f"one call of the same shape ({T} tokens, {q.shape[1]} query and {Hkv} KV heads, "
                      f"D={D}), {reps} repetitions, {dt:.1f} s"}


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--layers", type=int, default=None, help="layers per step (default: 36)")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--flags", type=int, default=0x2,
                    help="pa_plan flags (default PA_PLAN_SPEED_FEEDBACK: per-compute-unit budgets from measured speed)")
    ap.add_argument("--workload", default="batch64",
                    choices=["batch64", "batch64_4k8k", "single_request", "batch8", "hd256", "system_prompt",
                             "prefill_chunk512", "prefill_chunk64", "append", "copy"])
    ap.add_argument("--kv", default="bf16", choices=["bf16", "fp8"],
                    help="decode, prefill and append: pool element type (fp8 = OCP E4M3 codes with per-pool scales)")
    ap.add_argument("--graph", action="store_true", default=True,
                    help="decode: replay each step's layer runs from a captured HIP graph (the default)")
    ap.add_argument("--eager", dest="graph", action="store_false",
                    help="decode: launch each step's layer runs one by one")
    ap.add_argument("--cascade", action="store_true",
                    help="decode: plan with pa_plan_cascade over the workload's shared-prefix groups")
    ap.add_argument("--copy-gib", type=float, default=4.0)
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU only: the decode path is built and measured on a single "
              "MI355X (its multi-GPU sharding is a design note, not a measured configuration). "
              "Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    if args.workload == "copy":
        run_copy(args.copy_gib, args.steps)
        return

    if args.workload.startswith("prefill"):
        run_prefill_bench(args)
        return
    if args.workload == "append":
        run_append_bench(args)
        return

    import paged_gqa_decode_pa_amd as pa
    import workloads as W

    spec = {"batch64": W.BATCH64_SHARED_PREFIX, "batch64_4k8k": W.BATCH64_4K_8K,
            "single_request": W.SINGLE_REQUEST_256,
            "batch8": W.QWEN3_4B_BATCH8, "hd256": W.HEADDIM256_BATCH32,
            "system_prompt": W.SYSTEM_PROMPT_B64}[args.workload]
    # every decode workload runs 36 layers per step, each with its own pools
    layers = args.layers or 36
    dev = torch.device("cuda", 0)
    log(f"generating {spec.name}: {layers} layers of {spec.num_slots}-slot pools")
    t0 = time.perf_counter()
    fp8 = args.kv == "fp8"
    if fp8:   # the same lists and queries over 8-bit pools
        case = W.make_decode_case(spec, dev, layers=0)
        for layer in range(layers):
            k, v = W.make_pools_e4m3(spec.num_slots, spec.num_kv_heads, spec.head_dim,
                                     W.layer_seed(spec.seed, layer), dev)
            case.k_pools.append(k)
            case.v_pools.append(v)
    else:
        case = W.make_decode_case(spec, dev, layers=layers)
    torch.cuda.synchronize()
    log(f"inputs ready in {time.perf_counter() - t0:.1f} s "
        f"({torch.cuda.memory_allocated() / 2**30:.1f} GiB on device)")
    idx = torch.as_tensor(case.kv_indices, device=dev)
    B, Hq, Hkv, D = spec.batch, spec.num_qo_heads, spec.num_kv_heads, spec.head_dim
    bytes_per_layer = algorithmic_bytes(spec, case.kv_indptr, case.kv_indices, 1 if fp8 else 2)
    outs = [torch.empty((B, Hq, D), dtype=torch.float32, device=dev) for _ in range(layers)]
    plan = pa.Plan(B, int(case.kv_indptr[-1]), Hq, Hkv, D)
    stream = torch.cuda.current_stream(dev)
    plan_host_s = []
    if args.cascade and not spec.prefix_group_size:
        raise SystemExit(f"--cascade needs a workload with shared prefixes ({spec.name} has none)")
    if args.cascade:
        # the workload's prefix groups: consecutive requests sharing their
        # leading slot ids (what a radix prefix cache reports)
        group_indptr = np.arange(0, B + 1, spec.prefix_group_size, dtype=np.int32)
        prefix_len = np.full(group_indptr.size - 1, spec.prefix_len, np.int32)

    # the partition sized for the kernel of the pools' element type
    plan_flags = args.flags | (pa.PA_PLAN_KV_FP8 if fp8 else 0)

    def do_plan():
        if args.cascade:
            plan.plan_cascade(case.kv_indptr, group_indptr, prefix_len, flags=plan_flags,
                              stream=stream)
        else:
            plan.plan(case.kv_indptr, flags=plan_flags, stream=stream)

    def layer_runs(s):
        for layer in range(layers):
            if fp8:
                plan.decode_fp8(case.q, case.k_pools[layer], case.v_pools[layer], idx, case.sm_scale,
                                W.FP8_K_SCALE, W.FP8_V_SCALE, outs[layer], stream=s)
            else:
                plan.decode(case.q, case.k_pools[layer], case.v_pools[layer], idx, case.sm_scale,
                            outs[layer], stream=s)

    graph = None
    if args.graph:
        # the step's layer runs captured once; every step's pa_plan rewrites
        # the same device tables (same lists, hence the same grid), which the
        # replayed kernels read
        do_plan()
        side = torch.cuda.Stream(dev)
        side.wait_stream(stream)
        with torch.cuda.stream(side):
            layer_runs(side)
        stream.wait_stream(side)
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph, stream=side):
            layer_runs(side)
        torch.cuda.synchronize()

    def step(eager=False):
        do_plan()
        plan_host_s.append(pa.pa_plan_host_timing(plan.handle))
        if graph is not None and not eager:
            graph.replay()
        else:
            layer_runs(stream)

    # Python's cyclic garbage collector pauses the host for several
    # milliseconds every few hundred steps (measured: one step in 40 took
    # 13 ms instead of 7), long enough to starve the GPU, which the host
    # otherwise keeps two steps ahead of; it stays off while steps are issued
    gc.collect()
    gc.disable()
    wmarks = [torch.cuda.Event(enable_timing=True) for _ in range(args.warmup + 1)]
    wmarks[0].record(stream)
    for i in range(args.warmup):
        step()
        wmarks[i + 1].record(stream)
    torch.cuda.synchronize()
    log("warmup done; per-step ms: " + " ".join(f"{wmarks[i].elapsed_time(wmarks[i + 1]):.3f}"
                                                for i in range(args.warmup)))

    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)

    # timed region: K steps bracketed by HIP events on the launch stream, with
    # one more event between consecutive steps for the per-step spread (events
    # around every launch would slow the step down: they are taken in a
    # second pass below)
    plan_host_s.clear()
    step_marks = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    torch.cuda.synchronize()
    step_marks[0].record(stream)
    for i in range(args.steps):
        step()
        step_marks[i + 1].record(stream)
    torch.cuda.synchronize()
    ms_per_step = step_marks[0].elapsed_time(step_marks[-1]) / args.steps
    step_ms = np.array([step_marks[i].elapsed_time(step_marks[i + 1]) for i in range(args.steps)])
    log(f"step {ms_per_step:.3f} ms ({ms_per_step * 1e3 / layers:.1f} us per layer); per step "
        f"median {np.median(step_ms):.3f} min {step_ms.min():.3f} max {step_ms.max():.3f} ms")
    log("per-step ms: " + " ".join(f"{t:.3f}" for t in step_ms))
    wgw = plan.workgroup_weights()
    wg_weight_range = [round(float(wgw.min()), 3), round(float(wgw.max()), 3)]
    if args.flags & pa.PA_PLAN_SPEED_FEEDBACK:
        log(f"workgroup weights after the timed steps: min {wgw.min():.3f} max {wgw.max():.3f} "
            f"std {wgw.std():.3f}")

    # the same K steps again with HIP events recorded by the library in pairs
    # around every decode kernel on the launch stream: the kernel's own
    # duration (the pairs add a few microseconds between launches, so this
    # pass's step time is not the headline)
    pa.pa_profile_begin(plan.handle, args.steps * layers)
    torch.cuda.synchronize()
    start.record(stream)
    for _ in range(args.steps):
        step(eager=True)
    end.record(stream)
    torch.cuda.synchronize()
    ms_per_step_events = start.elapsed_time(end) / args.steps
    kernel_ms, launches = pa.pa_profile_end(plan.handle)
    kernel_avg_ms = kernel_ms / max(1, launches)
    log(f"decode kernel avg {kernel_avg_ms * 1e3:.1f} us over {launches} launches "
        f"(step with kernel event pairs {ms_per_step_events:.3f} ms)")

    gc.enable()

    # pa_plan's own host time (inside the library): within the timed steps the
    # call also waits for the upload of two steps back, so the host cost is
    # taken from calls made with nothing queued, and the in-step wait reported
    # beside it
    in_step = np.asarray(plan_host_s[: args.steps])
    idle = []
    for _ in range(50):
        torch.cuda.synchronize()
        do_plan()
        idle.append(pa.pa_plan_host_timing(plan.handle)[0])
    torch.cuda.synchronize()
    plan_host_us = float(np.median(idle))
    log(f"pa_plan host {plan_host_us:.1f} us (idle GPU); inside the timed steps "
        f"{np.median(in_step[:, 0] - in_step[:, 1]):.1f} us of work, plus "
        f"{np.median(in_step[:, 1]):.1f} us waiting for the GPU (the host runs two steps ahead)")

    step_bytes = bytes_per_layer * layers
    value = step_bytes / (ms_per_step * 1e-3) / 1e9
    achieved = bytes_per_layer / (kernel_avg_ms * 1e-3) / 1e9
    # HBM bytes per launch from the committed counters of this workload's
    # plain decode, bf16 or E4M3 (none for cascade plans)
    traffic = (traffic_per_launch(DECODE_COUNTERS.get(spec.name + ("_fp8kv" if fp8 else "")))
               if not args.cascade else None)

    G = Hq // Hkv
    result = {
        "metric": METRIC if spec is W.BATCH64_SHARED_PREFIX and not fp8 else
        f"decode-attn µs/step/layer + achieved HBM GB/s (% of MI355X peak), {spec.name}, {args.kv} KV",
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8-e4m3 KV, bf16 q, fp32 math" if fp8 else "bf16",
        "data": "synthetic",
        "config": {
            "workload": spec.name + ("_fp8kv" if fp8 else ""),
            "batch": B, "num_qo_heads": Hq, "num_kv_heads": Hkv, "head_dim": D,
            "layers_per_step": layers,
            "kv_len": f"uniform [{spec.len_lo}, {spec.len_hi}]",
            "shared_prefix": (f"{spec.batch // spec.prefix_group_size} groups x "
                              f"{spec.prefix_group_size} requests x {spec.prefix_len} slots"
                              if spec.prefix_group_size else "none"),
            "layer_runs": "hip graph replay" if graph is not None else "eager",
            "plan": "pa_plan_cascade (shared prefixes read once per group)" if args.cascade else "pa_plan",
            "list_entries": int(case.kv_indptr[-1]),
            "unique_slots": int(np.unique(case.kv_indices).size),
            "pool_slots": spec.num_slots,
            "plan_flags": plan_flags,
            "workgroup_weight_range": wg_weight_range,
        },
        "us_per_step_layer": round(ms_per_step * 1e3 / layers, 2),
        "step_ms": {"mean": round(ms_per_step, 4), "median": round(float(np.median(step_ms)), 4),
                    "min": round(float(step_ms.min()), 4), "max": round(float(step_ms.max()), 4)},
        "us_per_step_layer_median": round(float(np.median(step_ms)) * 1e3 / layers, 2),
        "frac_of_peak": round(value / HBM_PEAK_GBS, 4),
        "ms_per_step_with_kernel_event_pairs": round(ms_per_step_events, 4),
        "plan_host_us": round(plan_host_us, 1),
        # the plan's own work inside the timed steps, and separately the time
        # it blocked because the host was two steps ahead of the GPU
        "plan_host_us_in_step": round(float(np.median(in_step[:, 0] - in_step[:, 1])), 1),
        "plan_backpressure_wait_us_in_step": round(float(np.median(in_step[:, 1])), 1),
        "algorithmic_bytes_per_layer": bytes_per_layer,
        "roofline": {
            "bound": "hbm",
            "achieved": round(achieved, 1),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4),
            "traffic": traffic,
            "kernel": f"decode_kernel<{D},{G},{'e4m3' if fp8 else 'bf16'}> "
                      f"({'pa_decode_run_fp8' if fp8 else 'pa_decode_run'})"
                      + (" after the cascade prefix units (prefill_kernel); time of both" if args.cascade else ""),
            "kernel_avg_us": round(kernel_avg_ms * 1e3, 2),
            "kernel_timing": f"HIP event pairs around each of {launches} launches, second pass of the "
                             "timed steps",
        },
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        log(f"cpu baseline: fp64 oracle on layer 0 for ~{args.cpu_seconds:.0f} s")
        torch.cuda.synchronize()
        cpu, err = cpu_baseline(case, spec, bytes_per_layer, args.cpu_seconds, outs[0].cpu().numpy(),
                                fp8=fp8)
        result["cpu_baseline"] = cpu
        result["parity_layer0_max_abs_err"] = err
        log(f"cpu baseline {cpu['value']} GB/s on {cpu['cores']} threads; layer-0 max|d| {err:.3g}")
    plan.close()
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
