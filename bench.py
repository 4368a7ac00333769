#!/usr/bin/env python3
"""Benchmark of the fused MoE-LoRA layer (align + forward) on one MI355X.

Prints ONE JSON line: tokens/s of the whole layer, the roofline position of
the dominant kernel (HIP-event durations measured inside the timed region),
and the CPU reference timed on the host cores as a baseline.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload 2]

Default workload: the pages' illustrative expert (hidden 4096, intermediate
11008, rank 32), 8 experts top-2, 8 adapters, 16 decode tokens.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "MoE-LoRA layer tokens/s at 1 GPU; % HBM roofline (decode) / % MFMA peak (prefill)"
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, GB/s
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 MFMA


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", type=int, default=2, help="synthetic workload number 1..6")
    ap.add_argument("--block-m", type=int, default=0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=10.0,
                    help="target CPU time of the reference baseline sample")
    ap.add_argument("--cold-iters", type=int, default=-1,
                    help="extra per-call timings with L2 and MALL flushed before each call "
                         "(default 20, 10 for workload 5; 0 disables)")
    ap.add_argument("--read-probe-mb", type=int, default=0,
                    help="time a bf16 reduction and a device copy over this many MiB (attainable HBM rates)")
    ap.add_argument("--copy-probe-mb", type=int, default=0,
                    help="only run a plain device copy of this many MB (counter calibration)")
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


def cold_timing(step, iters, flush_mb=512):
    """Per-call times of align+forward with the caches flushed first: a
    flush_mb-MB fill before every call evicts L2 and the 256 MB MALL; the fill
    is outside the events.  Median and minimum in ms."""
    import torch
    scratch = torch.empty(flush_mb << 20, dtype=torch.uint8, device="cuda")
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(iters)]
    for a, b in ev:
        scratch.fill_(1)
        a.record()
        step()
        b.record()
    torch.cuda.synchronize()
    ts = sorted(a.elapsed_time(b) for a, b in ev)
    del scratch
    return {"iters": iters, "median_ms": ts[len(ts) // 2], "min_ms": ts[0],
            "flush_bytes_before_each": flush_mb << 20}


def cpu_baseline(inp, target_s):
    """The fp64 reference on the host cores over a bounded sample of the same
    workload's tokens; returns tokens/s and what was run."""
    import numpy as np

    import oracle
    import synth
    wl = inp.wl
    nthreads = oracle.default_threads()
    o = oracle.Oracle()
    # calibrate with one token per thread, then size the sample for ~target_s
    n0 = min(wl.T, nthreads)
    toks = np.arange(n0, dtype=np.int32)
    synth.host_slabs_for_tokens(inp, np.arange(wl.T))
    t0 = time.perf_counter()
    oracle.layer_from_inputs(inp, tokens=toks, oracle=o, nthreads=nthreads)
    dt = time.perf_counter() - t0
    n = n0 * max(1, int(round(target_s / max(dt, 1e-3))))
    toks = (np.arange(n) % wl.T).astype(np.int32)
    t0 = time.perf_counter()
    oracle.layer_from_inputs(inp, tokens=toks, oracle=o, nthreads=nthreads)
    dt = time.perf_counter() - t0
    return {"value": n / dt, "unit": "tokens/s", "cores": nthreads, "kind": "oracle",
            "sample": f"{n} token evaluations of workload {wl.name} (tokens cycled 0..{wl.T - 1}),"
                      f" fp64, {dt:.1f} s wall"}


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
    import lora_moe_amd as lm
    import synth

    lm.load_library()
    wl = synth.WORKLOADS[args.workload]
    print(f"bench: generating workload {args.workload} ({wl.name}) on the device", file=sys.stderr,
          flush=True)
    dev, inp = synth.device_inputs(wl, touched_only=True)
    work = synth.algorithmic_work(wl, inp.topk_ids, inp.lora_ids)
    shape = lm.make_shape(wl.T, wl.H, wl.I, wl.E, wl.topk, wl.L, wl.r, args.block_m, wl.scale)
    bm = lm.moe_lora_resolve_block_m(shape)
    ws = lm.alloc_workspace(shape)
    y = torch.empty((wl.T, wl.H), dtype=torch.bfloat16, device="cuda")
    stream = torch.cuda.current_stream()

    def step(st=stream):
        lm.moe_lora_align(shape, dev["topk_ids"], dev["lora_ids"], ws, st)
        lm.moe_lora_forward(shape, dev["x"], dev["topk_ids"], dev["topk_weights"], dev["lora_ids"],
                            dev["W_gu"], dev["W_down"], dev["A_gu"], dev["B_gu"], dev["A_down"],
                            dev["B_down"], ws, y, st)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    print(f"bench: warmup done ({args.warmup} steps)", file=sys.stderr, flush=True)

    # untimed pass with events around every stage: the per-stage breakdown,
    # and which stage dominates
    nbreak = max(1, min(args.steps, 10))
    lm.moe_lora_profile_begin(nbreak)
    for _ in range(nbreak):
        step()
    torch.cuda.synchronize()
    stage_ms, calls = lm.moe_lora_profile_end()
    per_stage = {k: v / max(calls, 1) for k, v in stage_ms.items()}
    sbf = stage_bytes_flops(wl, work)
    dom = max(sbf, key=lambda s: per_stage.get(s, 0.0))

    # timed region: events only around the dominant stage's kernel (two event
    # records per step on the launch stream)
    lm.moe_lora_profile_begin(args.steps, [dom])
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    dom_ms, dom_calls = lm.moe_lora_profile_end()
    print(f"bench: timed {args.steps} steps in {elapsed:.3f} s", file=sys.stderr, flush=True)

    ms_per_step = elapsed * 1e3 / args.steps
    value = wl.T * args.steps / elapsed
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
    roof.update({"kernel": dom, "avg_launch_ms": dom_avg_ms,
                 "alg_bytes_per_launch": sbf[dom]["bytes"], "alg_flops_per_launch": sbf[dom]["flops"],
                 "traffic": measured_traffic(dom, wl.name, bm),
                 "kernel_source_sha": kernel_source_sha(dom, bm)})
    layer_s = ms_per_step * 1e-3
    out = {
        "metric": METRIC, "value": value, "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": ms_per_step, "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": wl.name, "T": wl.T, "H": wl.H, "I": wl.I, "E": wl.E,
                   "topk": wl.topk, "L": wl.L, "r": wl.r,
                   "block_m": bm, "seed": wl.seed},
        "roofline": roof,
        "layer": {"alg_bytes": work["bytes"], "alg_flops": work["flops"],
                  "hbm_frac": work["bytes"] / layer_s / (HBM_PEAK_GBS * 1e9),
                  "mfma_frac": work["flops"] / layer_s / (MFMA_BF16_PEAK_TFLOPS * 1e12),
                  "experts_touched": work["experts_touched"],
                  "adapter_expert_pairs_touched": work["pairs_touched"]},
        "stages_ms": per_stage,
        "stages_ms_note": f"average of {calls} untimed calls with events around every stage",
    }
    # the path from router logits: moe_lora_route_align (router fused into the
    # align for small batches) + moe_lora_forward.  The logits are built so the
    # router reproduces the workload's routing: log(w) at each chosen expert,
    # -1e30 elsewhere (softmax of log w over the chosen experts is w itself).
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
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step_routed()
    torch.cuda.synchronize()
    routed_s = (time.perf_counter() - t0) / args.steps
    out["from_logits"] = {"ms_per_step": routed_s * 1e3, "tokens_per_s": wl.T / routed_s,
                          "note": "moe_lora_route_align + moe_lora_forward from logits that "
                                  "reproduce the workload's routing"}
    # the same step captured once in a HIP graph and replayed (no per-launch
    # host work, launches queued back to back)
    g = torch.cuda.CUDAGraph()
    gs = torch.cuda.Stream()
    gs.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(gs):
        with torch.cuda.graph(g, stream=gs):
            step(gs)
    torch.cuda.current_stream().wait_stream(gs)
    for _ in range(args.warmup):
        g.replay()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        g.replay()
    torch.cuda.synchronize()
    graph_s = (time.perf_counter() - t0) / args.steps
    out["graph"] = {"ms_per_step": graph_s * 1e3, "tokens_per_s": wl.T / graph_s,
                    "note": "align + forward captured once in a HIP graph, replayed"}
    del g
    cold_iters = args.cold_iters if args.cold_iters >= 0 else (10 if args.workload == 5 else 20)
    if cold_iters > 0:
        out["cold"] = cold_timing(step, cold_iters)
    if not args.no_cpu_baseline:
        print("bench: timing the CPU reference", file=sys.stderr, flush=True)
        out["cpu_baseline"] = cpu_baseline(inp, args.cpu_seconds)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
