#!/usr/bin/env python3
"""Benchmark of the fused MoE-LoRA layer (align + forward) on one MI355X.

Prints ONE JSON line: tokens/s of the whole layer, the roofline position of
the dominant kernel (HIP-event durations measured inside the timed region),
the other synthetic workloads' layer rates, and the CPU reference timed on
the host cores as a baseline.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload 5]

Each timed step is one align + forward call with L2 and the 256 MB MALL
flushed before it (a 512 MB fill outside the events); ``value`` is T over
the median call time.  Default workload: the DeepSeek-like prefill layer
(8192 tokens, hidden 7168, intermediate 2048, 256 experts top-8, 8 adapters
of rank 64), the largest shape and the one whose MFMA rate is the target.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "MoE-LoRA layer tokens/s at 1 GPU; % HBM roofline (decode) / % MFMA peak (prefill)"
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, GB/s
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 MFMA
FLUSH_MB = 512                 # > L2 (8 x 4 MB) + MALL (256 MB)


class Flush:
    """Evicts L2 and the MALL before a timed call: a FLUSH_MB write, then a
    read of a second FLUSH_MB buffer, so the caches hold clean lines of
    neither the layer's data nor anything dirty (a write alone leaves up to
    ~288 MB of dirty lines whose write-back would land in the timed call).
    ``dirty=True`` does the write only."""

    def __init__(self, dirty=False):
        import torch
        self.w = torch.empty(FLUSH_MB << 20, dtype=torch.uint8, device="cuda")
        self.r = None if dirty else torch.ones(FLUSH_MB << 18, dtype=torch.int32, device="cuda")

    def __call__(self):
        self.w.fill_(1)
        if self.r is not None:
            self.r.sum()


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", type=int, default=5, help="synthetic workload number 1..6")
    ap.add_argument("--block-m", type=int, default=0)
    ap.add_argument("--no-tuning", action="store_true",
                    help="the library's built-in configuration instead of the shipped tuning table")
    ap.add_argument("--others", default="1,2,3,4,6",
                    help="further workloads summarised under 'workloads' ('' for none)")
    ap.add_argument("--other-steps", type=int, default=10)
    ap.add_argument("--no-extras", action="store_true",
                    help="skip the warm, graph and from-logits timings of the main workload")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=10.0,
                    help="target CPU time of the reference baseline sample")
    ap.add_argument("--read-probe-mb", type=int, default=0,
                    help="time a bf16 reduction and a device copy over this many MiB (attainable HBM rates)")
    ap.add_argument("--copy-probe-mb", type=int, default=0,
                    help="only run a plain device copy of this many MB (counter calibration)")
    ap.add_argument("--gemm-probe", action="store_true",
                    help="time the vendor bf16 GEMM on dense problems with the projections' flops, and this "
                         "library's GEMM stages with equal experts (context for the MFMA roofline)")
    return ap.parse_args()


def stage_bytes_flops(wl, work):
    """Algorithmic bytes and flops of each kernel stage for this instance."""
    T, H, I, k, r = wl.T, wl.H, wl.I, wl.topk, wl.r
    b = work["bytes_parts"]
    P, P_l = work["P"], work["P_l"]
    return {
        "gemm_gate_up": dict(bytes=b["W_gu"] + b["B_gu"] + T * H * 2 + P_l * r * 4 + P * I * 2,
                             flops=2 * P * 2 * I * H + 2 * P_l * 2 * I * r),
        "gemm_down": dict(bytes=b["W_down"] + b["B_down"] + P * I * 2 + P_l * r * 4 + P * H * 4,
                          flops=2 * P * H * I + 2 * P_l * H * r),
        "shrink_gate_up": dict(bytes=b["A_gu"] + P_l * H * 2 + P_l * r * 4, flops=2 * P_l * r * H),
        "shrink_down": dict(bytes=b["A_down"] + P_l * I * 2 + P_l * r * 4, flops=2 * P_l * r * I),
        "combine": dict(bytes=P * H * 4 + T * H * 2, flops=P * H),
    }


def kernel_sources(stage: str, block_m: int) -> list:
    """Source files the kernel of `stage` is built from at this block_m."""
    if stage.startswith("gemm"):
        fam = ["gemm.hip"] if block_m <= 32 else ["gemm_dma.hip", "gemm_expand.h"]
    elif stage.startswith("shrink"):
        fam = ["shrink.hip"]
    elif stage.startswith("align"):
        fam = ["align.hip", "router_device.h"]
    elif stage.startswith("route"):
        fam = ["router.hip", "router_device.h"]
    else:
        fam = ["combine.hip"]
    return fam + ["device_util.h", "internal.h"]


def kernel_source_sha(stage: str, block_m: int) -> str:
    """Hash of the sources of the stage's kernel; HBM traffic taken from
    counters is reported only while it still matches."""
    h = hashlib.sha256()
    for name in kernel_sources(stage, block_m):
        with open(os.path.join(ROOT, "lora_moe_amd", "csrc", name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def measured_traffic(kernel: str, workload: str, block_m: int):
    """HBM bytes per launch of `kernel` from the committed counter summary
    (FETCH_SIZE and WRITE_SIZE runs, each scaled by what the counter reads for
    a plain copy of known size), or None when absent or stale."""
    path = os.path.join(ROOT, "profiles", f"traffic_{kernel}_{workload}.txt")
    if not os.path.exists(path):
        return None
    vals = {}
    for line in open(path):
        if ":" in line and not line.startswith(("#", " ", "`")):
            k, v = line.split(":", 1)
            vals[k.strip()] = v.strip()
    if vals.get("kernel_source_sha") != kernel_source_sha(kernel, block_m):
        return None
    if vals.get("block_m") != str(block_m):  # counted at another tile size
        return None
    try:
        return float(vals["traffic_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def copy_probe(mb):
    import torch
    n = mb * (1 << 20) // 4
    a = torch.ones(n, dtype=torch.float32, device="cuda")
    b = torch.empty_like(a)
    for _ in range(5):
        b.copy_(a)
    torch.cuda.synchronize()
    print(json.dumps({"copy_probe_bytes_read": n * 4, "copy_probe_bytes_written": n * 4,
                      "launches": 5}), flush=True)


def read_probe(mb, iters=10):
    """Attainable HBM rates on this device as context for the nominal 8 TB/s:
    a reduction over an mb-MiB bf16 buffer (torch.sum, fp32 accumulation;
    reads the buffer once) and a device copy of it (reads and writes it),
    each timed over `iters` launches after two warm-ups."""
    import torch
    n = mb * (1 << 20) // 2
    a = torch.ones(n, dtype=torch.bfloat16, device="cuda")
    b = torch.empty_like(a)
    out = {"read_probe_bytes": n * 2}
    for name, fn, moved in (("sum", lambda: a.sum(dtype=torch.float32), n * 2),
                            ("copy", lambda: b.copy_(a), n * 4)):
        for _ in range(2):
            fn()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(iters):
            fn()
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / iters
        out[f"{name}_ms"] = ms
        out[f"{name}_GBps"] = moved / (ms * 1e-3) / 1e9
    print(json.dumps(out), flush=True)


def gemm_probe(iters=20):
    """Context for the MFMA roofline, printed as one JSON line.

    vendor: torch.matmul (hipBLASLt) on dense bf16 problems x[M,K] . W[N,K]^T
    with the flops of the DeepSeek-like projections (M = T*k = 65536 pairs;
    gate_up N = 2I = 4096, K = H = 7168; down N = 7168, K = 2048) and of the
    Qwen3-MoE-like ones (M = 16384), median of `iters` launches.
    library: this library's gemm_gate_up and gemm_down stages (caller-owned
    profiler) at the DeepSeek-like sizes with every expert equally loaded
    (T = 8192 tokens spread evenly over 8 experts, top-8, so every row tile
    is full) and with one expert (T = 65536, top-1): the grouped kernels
    without the routed shape's ragged tiles.  Random inputs (N(0, 0.02))."""
    import statistics
    import torch
    import lora_moe_amd as lm
    torch.manual_seed(0)
    out = {"vendor": [], "library": []}
    for (what, M, N, K) in (("deepseek-like gate_up", 65536, 4096, 7168), ("deepseek-like down", 65536, 7168, 2048),
                            ("qwen3moe-like gate_up", 16384, 1536, 2048), ("qwen3moe-like down", 16384, 2048, 768)):
        a = torch.randn(M, K, device="cuda").to(torch.bfloat16)
        b = torch.randn(N, K, device="cuda").to(torch.bfloat16)
        for _ in range(3):
            c = a @ b.t()
        torch.cuda.synchronize()
        ev = []
        for _ in range(iters):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            c = a @ b.t()
            e1.record()
            ev.append((e0, e1))
        torch.cuda.synchronize()
        ms = statistics.median(x.elapsed_time(y) for x, y in ev)
        tf = 2 * M * N * K / ms / 1e9
        out["vendor"].append({"problem": what, "M": M, "N": N, "K": K, "ms": round(ms, 4),
                              "TFLOPs": round(tf, 1), "frac_of_2500": round(tf / 2500, 4)})
        del a, b, c
    H, I, L, r = 7168, 2048, 8, 64
    lm.load_library()
    scratch = torch.empty(512 << 20, dtype=torch.uint8, device="cuda")
    for T, k, E in ((8192, 8, 8), (65536, 1, 1)):
        g = lambda *sh: (torch.randn(*sh, device="cuda") * 0.02).to(torch.bfloat16)
        dev = dict(x=g(T, H), W_gu=g(E, 2 * I, H), W_down=g(E, H, I), A_gu=g(L, E, r, H), B_gu=g(L, E, 2 * I, r),
                   A_down=g(L, E, r, I), B_down=g(L, E, H, r))
        ids = torch.argsort(torch.rand(T, E, device="cuda"), dim=1)[:, :k].to(torch.int32).contiguous()
        wts = torch.full((T, k), 1.0 / k, device="cuda")
        lids = torch.randint(0, L, (T,), device="cuda", dtype=torch.int32)
        y = torch.empty((T, H), dtype=torch.bfloat16, device="cuda")
        shape = lm.make_shape(T, H, I, E, k, L, r, 256, 1.0)
        ws = lm.alloc_workspace(shape)
        prof = lm.Profiler(iters)

        def step(pr=None):
            lm.moe_lora_align(shape, ids, lids, ws, profiler=pr)
            lm.moe_lora_forward(shape, dev["x"], ids, wts, lids, dev["W_gu"], dev["W_down"], dev["A_gu"],
                                dev["B_gu"], dev["A_down"], dev["B_down"], ws, y, profiler=pr)
        for _ in range(2):
            step()
        for _ in range(iters):
            scratch.fill_(1)
            step(prof)
        torch.cuda.synchronize()
        st, calls = prof.read()
        prof.close()
        P = T * k
        for stage, flops in (("gemm_gate_up", 2 * P * 2 * I * H), ("gemm_down", 2 * P * H * I)):
            ms = st[stage] / calls
            out["library"].append({"stage": stage, "T": T, "topk": k, "E": E, "block_m": 256, "ms": round(ms, 4),
                                   "TFLOPs": round(flops / ms / 1e9, 1),
                                   "frac_of_2500": round(flops / ms / 1e9 / 2500, 4)})
        del dev, ws, y
        torch.cuda.empty_cache()
    print(json.dumps(out), flush=True)


def flushed_calls(step, iters, flush, profiler=None):
    """Per-call milliseconds of `iters` align + forward calls, each after
    `flush()` (outside the events) evicts L2 and the MALL."""
    import torch
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(iters)]
    for a, b in ev:
        flush()
        a.record()
        step(profiler)
        b.record()
    torch.cuda.synchronize()
    return [a.elapsed_time(b) for a, b in ev]


def warm_calls(step, iters):
    """Mean milliseconds of back-to-back calls (no flush)."""
    import torch
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(iters):
        step()
    torch.cuda.synchronize()
    return (time.perf_counter() - t0) * 1e3 / iters


def layer_fracs(work, ms):
    s = ms * 1e-3
    return {"hbm_frac": work["bytes"] / s / (HBM_PEAK_GBS * 1e9),
            "mfma_frac": work["flops"] / s / (MFMA_BF16_PEAK_TFLOPS * 1e12)}


def binding(work):
    """The roofline that bounds the layer: MFMA when its arithmetic intensity
    is above the ridge (312.5 flop/B), HBM otherwise."""
    ridge = MFMA_BF16_PEAK_TFLOPS * 1e12 / (HBM_PEAK_GBS * 1e9)
    return "mfma" if work["flops"] / max(work["bytes"], 1) >= ridge else "hbm"


def cpu_baseline(inp, target_s):
    """The fp64 reference on the host cores over a bounded sample of the same
    workload's tokens (the first n, with the weight slabs they read generated
    on the host); returns tokens/s and what was run."""
    import numpy as np

    import oracle
    import synth
    wl = inp.wl
    nthreads = oracle.default_threads()
    o = oracle.Oracle()
    # calibrate with one token per thread, then size the sample for ~target_s
    n0 = min(wl.T, nthreads)
    toks = np.arange(n0, dtype=np.int32)
    synth.host_slabs_for_tokens(inp, toks)
    t0 = time.perf_counter()
    oracle.layer_from_inputs(inp, tokens=toks, oracle=o, nthreads=nthreads)
    dt = time.perf_counter() - t0
    n = n0 * max(1, int(round(target_s / max(dt, 1e-3))))
    toks = (np.arange(n) % wl.T).astype(np.int32)
    synth.host_slabs_for_tokens(inp, np.unique(toks))
    t0 = time.perf_counter()
    oracle.layer_from_inputs(inp, tokens=toks, oracle=o, nthreads=nthreads)
    dt = time.perf_counter() - t0
    return {"value": n / dt, "unit": "tokens/s", "cores": nthreads, "kind": "oracle",
            "sample": f"{n} token evaluations of workload {wl.name} (tokens 0..{min(n, wl.T) - 1}"
                      f"{', cycled' if n > wl.T else ''}), fp64, {dt:.1f} s wall"}


def run_other(lm, synth, n, steps, flush, tuning):
    """Flushed median of one more workload (generated, timed, freed)."""
    import torch
    wl = synth.WORKLOADS[n]
    print(f"bench: workload {n} ({wl.name})", file=sys.stderr, flush=True)
    dev, inp = synth.device_inputs(wl, touched_only=True)
    work = synth.algorithmic_work(wl, inp.topk_ids, inp.lora_ids)
    shape = lm.make_shape(wl.T, wl.H, wl.I, wl.E, wl.topk, wl.L, wl.r, 0, wl.scale, tuning=tuning)
    ws = lm.alloc_workspace(shape)
    y = torch.empty((wl.T, wl.H), dtype=torch.bfloat16, device="cuda")

    def step(prof=None):
        lm.moe_lora_align(shape, dev["topk_ids"], dev["lora_ids"], ws, profiler=prof)
        lm.moe_lora_forward(shape, dev["x"], dev["topk_ids"], dev["topk_weights"], dev["lora_ids"],
                            dev["W_gu"], dev["W_down"], dev["A_gu"], dev["B_gu"], dev["A_down"],
                            dev["B_down"], ws, y, profiler=prof)

    for _ in range(3):
        step()
    ts = flushed_calls(step, steps, flush)
    med = statistics.median(ts)
    out = {"workload": wl.name, "block_m": lm.moe_lora_resolve_block_m(shape),
           "knobs": {k: getattr(shape, k) for k in lm.KNOBS},
           "flushed_median_ms": med, "flushed_min_ms": min(ts), "tokens_per_s": wl.T / (med * 1e-3),
           "bound": binding(work), **layer_fracs(work, med)}
    del dev, ws, y
    torch.cuda.empty_cache()
    return out


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py runs on one GPU only: this library has no multi-GPU path "
              "(collectives and sharding are out of scope); rerun with --gpus 1.",
              file=sys.stderr, flush=True)
        sys.exit(2)
    import torch

    if args.copy_probe_mb:
        copy_probe(args.copy_probe_mb)
        return
    if args.read_probe_mb:
        read_probe(args.read_probe_mb)
        return
    if args.gemm_probe:
        gemm_probe()
        return
    import lora_moe_amd as lm
    import synth

    lm.load_library()
    wl = synth.WORKLOADS[args.workload]
    print(f"bench: generating workload {args.workload} ({wl.name}) on the device", file=sys.stderr,
          flush=True)
    dev, inp = synth.device_inputs(wl, touched_only=True, keep_host=not args.no_cpu_baseline)
    work = synth.algorithmic_work(wl, inp.topk_ids, inp.lora_ids)
    tuning = None if args.no_tuning else lm.load_tuning()
    shape = lm.make_shape(wl.T, wl.H, wl.I, wl.E, wl.topk, wl.L, wl.r, args.block_m, wl.scale, tuning=tuning)
    bm = lm.moe_lora_resolve_block_m(shape)
    ws = lm.alloc_workspace(shape)
    y = torch.empty((wl.T, wl.H), dtype=torch.bfloat16, device="cuda")
    stream = torch.cuda.current_stream()
    flush = Flush()

    def step(prof=None, st=stream):
        lm.moe_lora_align(shape, dev["topk_ids"], dev["lora_ids"], ws, st, profiler=prof)
        lm.moe_lora_forward(shape, dev["x"], dev["topk_ids"], dev["topk_weights"], dev["lora_ids"],
                            dev["W_gu"], dev["W_down"], dev["A_gu"], dev["B_gu"], dev["A_down"],
                            dev["B_down"], ws, y, st, profiler=prof)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    print(f"bench: warmup done ({args.warmup} steps)", file=sys.stderr, flush=True)

    # untimed pass with events around every stage (flushed calls, like the
    # timed ones): the per-stage breakdown, and which stage dominates
    nbreak = max(1, min(args.steps, 10))
    prof = lm.Profiler(nbreak)
    flushed_calls(step, nbreak, flush, prof)
    stage_ms, calls = prof.read()
    prof.close()
    per_stage = {k: v / max(calls, 1) for k, v in stage_ms.items()}
    sbf = stage_bytes_flops(wl, work)
    dom = max(sbf, key=lambda s: per_stage.get(s, 0.0))

    # timed region: K flushed calls, events around each call and, inside it,
    # around the dominant stage's kernel (on the launch stream)
    prof = lm.Profiler(args.steps, [dom])
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    call_ms = flushed_calls(step, args.steps, flush, prof)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    dom_ms, dom_calls = prof.read()
    prof.close()
    print(f"bench: timed {args.steps} flushed steps in {elapsed:.3f} s", file=sys.stderr, flush=True)

    ms_per_step = statistics.median(call_ms)
    value = wl.T / (ms_per_step * 1e-3)
    dom_avg_ms = dom_ms[dom] / max(dom_calls, 1)
    dur_s = dom_avg_ms * 1e-3
    ai = sbf[dom]["flops"] / max(sbf[dom]["bytes"], 1)
    ridge = MFMA_BF16_PEAK_TFLOPS * 1e12 / (HBM_PEAK_GBS * 1e9)
    if ai < ridge:
        achieved = sbf[dom]["bytes"] / dur_s / 1e9
        roof = {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": achieved / HBM_PEAK_GBS}
    else:
        achieved = sbf[dom]["flops"] / dur_s / 1e12
        roof = {"bound": "mfma", "achieved": achieved, "peak": MFMA_BF16_PEAK_TFLOPS,
                "unit": "TFLOP/s", "frac": achieved / MFMA_BF16_PEAK_TFLOPS}
    roof.update({"traffic": measured_traffic(dom, wl.name, bm), "kernel": dom,
                 "avg_launch_ms": dom_avg_ms,
                 "alg_bytes_per_launch": sbf[dom]["bytes"], "alg_flops_per_launch": sbf[dom]["flops"],
                 "kernel_source_sha": kernel_source_sha(dom, bm)})
    out = {
        "metric": METRIC, "value": value, "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": ms_per_step, "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": wl.name, "T": wl.T, "H": wl.H, "I": wl.I, "E": wl.E,
                   "topk": wl.topk, "L": wl.L, "r": wl.r,
                   "block_m": bm, "seed": wl.seed, **{k: getattr(shape, k) for k in lm.KNOBS}},
        "roofline": roof,
        "timing": {"per_step": "one align + forward call after a 512 MB write and a read of "
                               "another 512 MB (L2 and MALL cold and clean), HIP events around "
                               "the call; value and ms_per_step from the median call",
                   "median_ms": ms_per_step,
                   "min_ms": min(call_ms), "max_ms": max(call_ms),
                   "wall_s_timed_region": elapsed},
        "layer": {"alg_bytes": work["bytes"], "alg_flops": work["flops"], "bound": binding(work),
                  **layer_fracs(work, ms_per_step),
                  "experts_touched": work["experts_touched"],
                  "adapter_expert_pairs_touched": work["pairs_touched"]},
        "stages_ms": per_stage,
        "stages_ms_note": f"average of {calls} untimed flushed calls with events around every stage",
    }
    if not args.no_extras:
        out["warm"] = {"ms_per_step": warm_calls(step, args.steps),
                       "note": "back-to-back calls, caches warm"}
        dirty = Flush(dirty=True)
        out["flushed_dirty"] = {"median_ms": statistics.median(flushed_calls(step, args.steps, dirty)),
                                "note": "each call after the 512 MB write only (its dirty lines are "
                                        "written back during the call)"}
        del dirty
        # the path from router logits: moe_lora_route_align (router fused into
        # the align for small batches) + moe_lora_forward.  The logits are built
        # so the router reproduces the workload's routing: log(w) at each chosen
        # expert, -1e30 elsewhere (softmax of log w over the chosen experts is w).
        logits = torch.full((wl.T, wl.E), -1e30, dtype=torch.float32, device="cuda")
        logits.scatter_(1, dev["topk_ids"].long(), torch.log(dev["topk_weights"].clamp_min(1e-30)))
        r_ids = torch.empty_like(dev["topk_ids"])
        r_w = torch.empty_like(dev["topk_weights"])

        def step_routed():
            lm.moe_lora_route_align(shape, logits, dev["lora_ids"], r_ids, r_w, ws, stream)
            lm.moe_lora_forward(shape, dev["x"], r_ids, r_w, dev["lora_ids"],
                                dev["W_gu"], dev["W_down"], dev["A_gu"], dev["B_gu"], dev["A_down"],
                                dev["B_down"], ws, y, stream)

        for _ in range(args.warmup):
            step_routed()
        out["from_logits"] = {"ms_per_step": warm_calls(step_routed, args.steps),
                              "note": "moe_lora_route_align + moe_lora_forward from logits that "
                                      "reproduce the workload's routing, warm"}
        # the same step captured once in a HIP graph and replayed
        g = torch.cuda.CUDAGraph()
        gs = torch.cuda.Stream()
        gs.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(gs):
            with torch.cuda.graph(g, stream=gs):
                step(None, gs)
        torch.cuda.current_stream().wait_stream(gs)
        for _ in range(args.warmup):
            g.replay()
        out["graph"] = {"ms_per_step": warm_calls(g.replay, args.steps),
                        "note": "align + forward captured once in a HIP graph, replayed, warm"}
        del g
    # the host reference runs while the GPU is idle, then the other workloads
    if not args.no_cpu_baseline:
        print("bench: timing the CPU reference", file=sys.stderr, flush=True)
        out["cpu_baseline"] = cpu_baseline(inp, args.cpu_seconds)
    del dev, ws, y
    torch.cuda.empty_cache()
    others = [int(w) for w in args.others.split(",") if w.strip()] if args.others else []
    if others:
        out["workloads"] = {"note": "flushed median of align + forward per workload, "
                                    f"{args.other_steps} calls, configuration from "
                                    + ("the library's built-in choice" if args.no_tuning
                                       else "the shipped tuning table"),
                            args.workload: {"workload": wl.name, "block_m": bm,
                                            "flushed_median_ms": ms_per_step,
                                            "flushed_min_ms": min(call_ms),
                                            "tokens_per_s": value, "bound": binding(work),
                                            **layer_fracs(work, ms_per_step)}}
        for n in others:
            if n != args.workload:
                out["workloads"][n] = run_other(lm, synth, n, args.other_steps, flush, tuning)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
