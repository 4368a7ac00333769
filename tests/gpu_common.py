"""Helpers for the GPU parity tests: run the HIP library through its C ABI and
compare with the fp64 CPU reference."""
from __future__ import annotations

import sys

import numpy as np

import lora_moe_amd as lm
import oracle
import synth

ATOL = 1e-2
RTOL = 1e-2


def log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def shape_for(wl, block_m=0, **knobs):
    return lm.make_shape(wl.T, wl.H, wl.I, wl.E, wl.topk, wl.L, wl.r, block_m, wl.scale, **knobs)


def check_shapes(dev, wl):
    """Host-side check that operand dtypes and shapes match what the kernels
    assume (the package's own check, run before every launch anyway)."""
    lm.check_operands(shape_for(wl), **{n: dev[n] for n in (
        "x", "topk_ids", "topk_weights", "lora_ids", "W_gu", "W_down", "A_gu", "B_gu", "A_down",
        "B_down")})


def run_gpu(dev, wl, block_m=0, lora_ids=None, workspace=None, knobs=None):
    """align + forward through the C ABI; returns (y as fp64 numpy, shape, workspace)."""
    import torch
    check_shapes(dev, wl)
    shape = shape_for(wl, block_m, **(knobs or {}))
    ws = workspace if workspace is not None else lm.alloc_workspace(shape)
    lids = dev["lora_ids"] if lora_ids is None else lora_ids
    y = torch.empty((wl.T, wl.H), dtype=torch.bfloat16, device="cuda")
    lm.moe_lora_align(shape, dev["topk_ids"], lids, ws)
    lm.moe_lora_forward(shape, dev["x"], dev["topk_ids"], dev["topk_weights"], lids, dev["W_gu"],
                        dev["W_down"], dev["A_gu"], dev["B_gu"], dev["A_down"], dev["B_down"], ws, y)
    torch.cuda.synchronize()
    return y.float().cpu().numpy().astype(np.float64), shape, ws


def to_device(inp):
    """Upload a host ``synth.Inputs`` bundle."""
    import torch
    out = {}
    for n, a in inp.arrays().items():
        if a.dtype == np.uint16:
            out[n] = torch.from_numpy(a.view(np.int16)).cuda().view(torch.bfloat16)
        else:
            out[n] = torch.from_numpy(np.ascontiguousarray(a)).cuda()
    return out


def compare(y_gpu, y_ref, what=""):
    """Element-wise |gpu - ref| <= 1e-2 + 1e-2*|ref| and relative L2 <= 1e-2."""
    err = np.abs(y_gpu - y_ref)
    bound = ATOL + RTOL * np.abs(y_ref)
    bad = err > bound
    rel_l2 = float(np.linalg.norm(y_gpu - y_ref) / max(np.linalg.norm(y_ref), 1e-30))
    worst = float(np.max(err / bound)) if err.size else 0.0
    log(f"[{what}] max err/tol {worst:.3f}, rel L2 {rel_l2:.2e}, bad {int(bad.sum())}/{bad.size}")
    assert not bad.any(), f"{what}: {int(bad.sum())} elements out of tolerance (worst {worst:.2f}x)"
    assert rel_l2 <= 1e-2, f"{what}: relative L2 {rel_l2:.3e}"
    return worst, rel_l2


def compare_delta(y_gpu, y_gpu_base, y_ref, y_ref_base, what=""):
    """The adapters' contribution must match: ||dgpu - dref|| / ||dref|| <= 0.1."""
    dg = y_gpu - y_gpu_base
    dr = y_ref - y_ref_base
    n = float(np.linalg.norm(dr))
    assert n > 0, f"{what}: reference adapter delta is zero"
    rel = float(np.linalg.norm(dg - dr)) / n
    log(f"[{what}] adapter-delta rel L2 {rel:.3e}")
    assert rel <= 0.1, f"{what}: adapter delta off by {rel:.3f}"
    return rel


def gpu_views(shape, ws):
    """Align outputs from the workspace as host numpy arrays."""
    t = lm.workspace_tensors(shape, ws)
    out = {}
    for n in ("sorted_ids", "expert_off", "seg_start", "seg_cnt", "block_expert", "pos_of_pair"):
        out[n] = t[n].cpu().numpy()
    out["num_padded"] = int(t["num_padded"].cpu().item())
    out["err_count"] = int(t["err_count"].cpu().item())
    out["cap_rows"], out["cap_blocks"], out["block_m"] = t["cap_rows"], t["cap_blocks"], t["block_m"]
    return out


def oracle_tokens(inp, tokens, lora_ids=None, scale=None):
    o = oracle.Oracle()
    wl = inp.wl
    shape = (wl.T, wl.H, wl.I, wl.E, wl.topk, wl.L, wl.r)
    lids = inp.lora_ids if lora_ids is None else lora_ids
    return o.layer(shape, inp.x, inp.topk_ids, inp.topk_weights, lids, inp.W_gu, inp.W_down,
                   inp.A_gu, inp.B_gu, inp.A_down, inp.B_down, tokens=tokens,
                   scale=wl.scale if scale is None else scale)


def sample_tokens(T, n, seed=123):
    if n >= T:
        return np.arange(T, dtype=np.int32)
    rng = np.random.default_rng(seed)
    pick = set(rng.choice(T, n - 2, replace=False).tolist()) | {0, T - 1}
    return np.array(sorted(pick), dtype=np.int32)
