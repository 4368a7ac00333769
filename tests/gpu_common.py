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


def shape_for(wl, block_m=0):
    return lm.make_shape(wl.T, wl.H, wl.I, wl.E, wl.topk, wl.L, wl.r, block_m, wl.scale)


def check_shapes(dev, wl):
    """Host-side check that operand shapes match what the kernels assume."""
    T, H, I, E, k, L, r = wl.T, wl.H, wl.I, wl.E, wl.topk, wl.L, wl.r
    want = dict(x=(T, H), topk_ids=(T, k), topk_weights=(T, k), lora_ids=(T,), W_gu=(E, 2 * I, H),
                W_down=(E, H, I), A_gu=(L, E, r, H), B_gu=(L, E, 2 * I, r), A_down=(L, E, r, I),
                B_down=(L, E, H, r))
    for n, s in want.items():
        assert tuple(dev[n].shape) == s, (n, tuple(dev[n].shape), s)
        assert dev[n].is_contiguous(), n


def run_gpu(dev, wl, block_m=0, lora_ids=None, workspace=None):
    """align + forward through the C ABI; returns (y as fp64 numpy, shape, workspace)."""
    import torch
    check_shapes(dev, wl)
    shape = shape_for(wl, block_m)
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


def dense_tol_scale(I):
    """Tolerance factor for layers beyond the stated workloads' down-projection
    depth.  The dominant error is h rounded to bf16 (relative 2^-9 per element)
    feeding the down GEMM, so its absolute size grows with sqrt(I); the stated
    tolerance holds with margin up to I = 2048 at the DeepSeek-like shape
    (max err/tol ~0.7), so a layer with larger I gets sqrt(I / 2048)."""
    return max(1.0, float(np.sqrt(I / 2048.0)))


def compare(y_gpu, y_ref, what="", tol_scale=1.0):
    """Element-wise |gpu - ref| <= atol + rtol*|ref| (both times tol_scale) and
    relative L2 <= 1e-2."""
    err = np.abs(y_gpu - y_ref)
    bound = tol_scale * (ATOL + RTOL * np.abs(y_ref))
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
