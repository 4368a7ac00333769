"""Offline sweep for the tile-configuration table (GPU).

For each synthetic workload, times ``moe_lora_align + moe_lora_forward``
(median of flushed calls: L2 and the MALL evicted before each) at every
block_m the library has tiles for (16 and 32: the register-streaming GEMM;
64, 128, 192 and 256: the LDS-DMA GEMM with 64 x 128, 128 x 128, 192 x 256
and 256 x 256 tiles; block_m also sets the align padding and the shrink
tile), then, at the fastest block_m, each kernel knob in turn -- the shrinks'
K splits and z column blocks, the streaming down GEMM's K splits, the tiled
GEMMs' workgroup order -- keeping a value only when it beats the library's
own choice by at least MARGIN; and writes the configuration per shape class
as a table that ``load_tuning`` / ``moe_lora_tune_apply`` read.  The pages tune their
kernel configurations per shape in the same spirit ("Multi-LoRA for MoE
models", section "Tuning kernel configurations for Amazon SageMaker AI and
Amazon Bedrock").

    python -m lora_moe_amd.tune --workloads 2,3,4,5,6 --out lora_moe_amd/tuning/gfx950.json
"""
from __future__ import annotations

import argparse
import json
import os
import statistics
import sys

CANDIDATES = (16, 32, 64, 128, 192, 256)
MARGIN = 0.015  # a knob value replaces the library's choice only when this much faster


def time_layer(lm, shape, dev, y, iters: int, warmup: int, scratch) -> float:
    """Median milliseconds of align + forward over `iters` calls, each after
    a write of scratch[0] and a read of scratch[1] (outside the events) that
    leave L2 and the MALL holding clean, unrelated lines."""
    import torch
    ws = lm.alloc_workspace(shape)

    def step():
        lm.moe_lora_align(shape, dev["topk_ids"], dev["lora_ids"], ws)
        lm.moe_lora_forward(shape, dev["x"], dev["topk_ids"], dev["topk_weights"], dev["lora_ids"],
                            dev["W_gu"], dev["W_down"], dev["A_gu"], dev["B_gu"], dev["A_down"],
                            dev["B_down"], ws, y)

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    ev = []
    for _ in range(iters):
        scratch[0].fill_(1)
        scratch[1].sum()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        step()
        b.record()
        ev.append((a, b))
    torch.cuda.synchronize()
    del ws
    return statistics.median(a.elapsed_time(b) for a, b in ev)


def knob_candidates(wl, bm: int) -> dict:
    """Values to try for each knob at this block_m (0 = the library's choice
    is always the reference)."""
    K = {"shrink_splits": [1, 2, 4, 8, 16],
         "shrink_zblocks": [d for d in (1, 2, 4, 8) if wl.r % d == 0 and (wl.r // d) % 8 == 0]}
    if bm <= 32 or wl.I >= 4096:  # the streaming down GEMM runs
        K["down_splits"] = [1, 2, 4, 8, 10, 12, 16]
    if bm >= 64:  # the LDS-tiled GEMMs run
        K["tile_order"] = [1, 2]
        if wl.L <= 64:  # both forms of their expand can run
            K["expand_mode"] = [1, 2]
    return K


def main(argv=None) -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--workloads", default="2,3,4,5,6")
    ap.add_argument("--out", default=None, help="JSON table to write (default: print only)")
    ap.add_argument("--iters", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--no-knobs", action="store_true", help="sweep block_m only")
    args = ap.parse_args(argv)

    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    if root not in sys.path:
        sys.path.insert(0, root)
    import torch
    import lora_moe_amd as lm
    import synth

    lm.load_library()
    scratch = (torch.empty(512 << 20, dtype=torch.uint8, device="cuda"),
               torch.ones(512 << 18, dtype=torch.int32, device="cuda"))
    entries = []
    for n in (int(w) for w in args.workloads.split(",")):
        wl = synth.WORKLOADS[n]
        dev, _ = synth.device_inputs(wl, touched_only=True)
        y = torch.empty((wl.T, wl.H), dtype=torch.bfloat16, device="cuda")

        def run(bm, **knobs):
            shape = lm.make_shape(wl.T, wl.H, wl.I, wl.E, wl.topk, wl.L, wl.r, bm, wl.scale, **knobs)
            if lm.moe_lora_workspace_bytes(shape) == 0:
                return None  # no valid layout
            t = time_layer(lm, shape, dev, y, args.iters, args.warmup, scratch)
            print(f"tune: workload {n} ({wl.name}) block_m {bm} {knobs or ''}: {t:.4f} ms", flush=True)
            return t

        ms = {}
        for bm in CANDIDATES:
            t = run(bm)
            if t is not None:
                ms[bm] = t
        best = min(ms, key=ms.get)
        knobs, knob_ms = {}, {}
        if not args.no_knobs:
            ref = ms[best]
            for k, vals in knob_candidates(wl, best).items():
                tried = {}
                for v in vals:
                    t = run(best, **knobs, **{k: v})
                    if t is not None:
                        tried[v] = t
                knob_ms[k] = {str(v): round(t, 4) for v, t in tried.items()}
                if tried:
                    v = min(tried, key=tried.get)
                    if tried[v] < ref * (1 - MARGIN):
                        knobs[k] = v
                        ref = tried[v]
        P = wl.T * wl.topk
        touched = max(1, min(wl.E, P))
        entries.append({"rows_per_expert": -(-P // touched), "H": wl.H, "I": wl.I, "E": wl.E,
                        "r": wl.r, "L": wl.L, "block_m": best,
                        **{k: knobs.get(k, 0) for k in lm.KNOBS},
                        "workload": wl.name, "ms": {str(k): round(v, 4) for k, v in ms.items()},
                        "knob_ms": knob_ms,
                        "tuned_ms": round(run(best, **knobs), 4) if knobs else round(ms[best], 4)})
        del dev, y
        torch.cuda.empty_cache()
    doc = {"arch": "gfx950", "device": torch.cuda.get_device_name(0),
           "command": "python -m lora_moe_amd.tune --workloads " + args.workloads,
           "metric": "median ms of align + forward, L2 and MALL flushed (512 MB write + 512 MB read) "
                     "before each call",
           "margin": MARGIN, "entries": entries}
    text = json.dumps(doc, indent=1)
    if args.out:
        os.makedirs(os.path.dirname(os.path.abspath(args.out)), exist_ok=True)
        with open(args.out, "w") as f:
            f.write(text + "\n")
    print(text, flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
