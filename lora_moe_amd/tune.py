"""Offline sweep for the tile-configuration table (GPU).

For each synthetic workload, times ``moe_lora_align + moe_lora_forward`` at
every block_m the library has tiles for (16 and 32: the register-streaming
GEMM; 64, 128, 192 and 256: the LDS-DMA GEMM with 64 x 128, 128 x 128,
192 x 256 and 256 x 256 tiles; block_m also sets the align padding and the
shrink tile), and writes the fastest per shape class as a table that
``load_tuning`` / ``moe_lora_tune_block_m`` read.  The pages tune their
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


def time_layer(lm, shape, dev, y, iters: int, warmup: int) -> float:
    """Median milliseconds of align + forward over `iters` calls."""
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
    times = []
    for _ in range(iters):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        step()
        b.record()
        b.synchronize()
        times.append(a.elapsed_time(b))
    del ws
    return statistics.median(times)


def main(argv=None) -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--workloads", default="2,3,4,5,6")
    ap.add_argument("--out", default=None, help="JSON table to write (default: print only)")
    ap.add_argument("--iters", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    args = ap.parse_args(argv)

    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    if root not in sys.path:
        sys.path.insert(0, root)
    import torch
    import lora_moe_amd as lm
    import synth

    lm.load_library()
    entries = []
    for n in (int(w) for w in args.workloads.split(",")):
        wl = synth.WORKLOADS[n]
        dev, _ = synth.device_inputs(wl, touched_only=True)
        y = torch.empty((wl.T, wl.H), dtype=torch.bfloat16, device="cuda")
        ms = {}
        for bm in CANDIDATES:
            shape = lm.make_shape(wl.T, wl.H, wl.I, wl.E, wl.topk, wl.L, wl.r, bm, wl.scale)
            if lm.moe_lora_workspace_bytes(shape) == 0:
                continue  # no valid layout at this block_m
            it = max(5, args.iters // 2) if wl.T * wl.topk > 16384 else args.iters
            ms[bm] = time_layer(lm, shape, dev, y, it, args.warmup)
            print(f"tune: workload {n} ({wl.name}) block_m {bm}: {ms[bm]:.4f} ms", flush=True)
        best = min(ms, key=ms.get)
        P = wl.T * wl.topk
        touched = max(1, min(wl.E, P))
        entries.append({"rows_per_expert": -(-P // touched), "H": wl.H, "I": wl.I, "E": wl.E,
                        "r": wl.r, "L": wl.L, "block_m": best, "workload": wl.name,
                        "ms": {str(k): round(v, 4) for k, v in ms.items()}})
        del dev, y
        torch.cuda.empty_cache()
    doc = {"arch": "gfx950", "device": torch.cuda.get_device_name(0),
           "command": "python -m lora_moe_amd.tune --workloads " + args.workloads,
           "metric": "median ms of align + forward, warm", "entries": entries}
    text = json.dumps(doc, indent=1)
    if args.out:
        os.makedirs(os.path.dirname(os.path.abspath(args.out)), exist_ok=True)
        with open(args.out, "w") as f:
            f.write(text + "\n")
    print(text, flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
