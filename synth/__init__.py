"""Seeded synthetic inputs for the fused MoE-LoRA layer.

Shared by the tests, ``bench.py`` and the CPU reference.  This module holds
none of the layer's arithmetic: it draws x, router logits, adapter ids and the
weight slabs, and turns router logits into (topk_ids, topk_weights) the way a
softmax top-k router does.  The router is the input generator here, not part
of the layer (the layer receives routed ids and weights).

Random numbers come from ``synth.c`` (counter-based SplitMix64 + Box-Muller),
so every slab -- one expert's base weight, one (adapter, expert) A or B -- can
be regenerated on its own and always gives the same bf16 bits.

Stream tags: 0 router logits, 1 per-expert router bias, 2 adapter ids,
3 x, 4 W_gu, 5 W_down, 6 A_gu, 7 B_gu, 8 A_down, 9 B_down.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from dataclasses import dataclass, field, replace

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "synth.c")
_SO = os.path.join(_HERE, "libsynth.so")
_lib = None


def build(force: bool = True) -> str:
    """Compile synth.c into libsynth.so (plain C, OpenMP)."""
    if force or not os.path.exists(_SO):
        tmp = _SO + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c11",
                               _SRC, "-o", tmp, "-lm"])
        os.replace(tmp, _SO)
    return _SO


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_SO):
            build(force=False)
        lib = ctypes.CDLL(_SO)
        u64, i64, dp, vp = ctypes.c_uint64, ctypes.c_int64, ctypes.c_double, ctypes.c_void_p
        lib.synth_stream_key.restype = u64
        lib.synth_stream_key.argtypes = [u64, u64, u64, u64]
        lib.synth_uniform_f64.argtypes = [u64, i64, vp]
        lib.synth_normal_f64.argtypes = [u64, i64, dp, dp, vp]
        lib.synth_normal_bf16.argtypes = [u64, i64, dp, vp]
        lib.synth_f32_to_bf16.argtypes = [vp, i64, vp]
        _lib = lib
    return _lib


def stream_key(seed: int, tag: int, a: int = 0, b: int = 0) -> int:
    return _load().synth_stream_key(seed, tag, a, b)


def uniform(key: int, n: int) -> np.ndarray:
    out = np.empty(n, dtype=np.float64)
    _load().synth_uniform_f64(key, n, out.ctypes.data)
    return out


def normal(key: int, n: int, mean: float = 0.0, std: float = 1.0) -> np.ndarray:
    out = np.empty(n, dtype=np.float64)
    _load().synth_normal_f64(key, n, mean, std, out.ctypes.data)
    return out


def normal_bf16_into(key: int, out: np.ndarray, std: float) -> None:
    assert out.dtype == np.uint16 and out.flags.c_contiguous
    _load().synth_normal_bf16(key, out.size, std, out.ctypes.data)


def to_bf16(a) -> np.ndarray:
    """fp32 values -> bf16 bit patterns (round to nearest even)."""
    f = np.ascontiguousarray(np.asarray(a, dtype=np.float32))
    out = np.empty(f.shape, dtype=np.uint16)
    _load().synth_f32_to_bf16(f.ctypes.data, f.size, out.ctypes.data)
    return out


def bf16_to_f64(u: np.ndarray) -> np.ndarray:
    """bf16 bit patterns -> exact fp64 values."""
    return (np.asarray(u, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


@dataclass(frozen=True)
class Workload:
    """One synthetic layer workload: sizes plus how ids and weights are drawn."""
    name: str
    T: int
    H: int
    I: int
    E: int
    topk: int
    L: int
    r: int
    lora_mode: str = "uniform"        # uniform | uniform_with_none | zipf | none_fraction
    zipf_s: float = 1.1
    none_fraction: float = 0.0
    bias_std: float = 0.0
    w_std: float = 0.02
    x_std: float = 1.0
    scale: float = 1.0
    seed: int = 0

    @property
    def P(self) -> int:
        return self.T * self.topk


# The layer workloads.  Shapes, adapter-id distributions and routing skew
# follow the synthetic layer shapes this library is measured on; the
# "illustrative" one is the 4096/11008/r=32 expert of the pages' Figure 1.
WORKLOADS = {
    1: Workload("tiny", T=64, H=256, I=512, E=8, topk=2, L=4, r=8, lora_mode="uniform_with_none"),
    2: Workload("illustrative-decode", T=16, H=4096, I=11008, E=8, topk=2, L=8, r=32),
    3: Workload("gptoss-like", T=256, H=2880, I=2880, E=32, topk=4, L=16, r=32, lora_mode="zipf"),
    4: Workload("qwen3moe-like", T=2048, H=2048, I=768, E=128, topk=8, L=32, r=16,
                lora_mode="none_fraction", none_fraction=0.2),
    5: Workload("deepseek-like", T=8192, H=7168, I=2048, E=256, topk=8, L=8, r=64, bias_std=2.0),
    # dense multi-LoRA decode (one expert, every token routed to it with
    # weight 1): a Qwen3-32B-sized MLP with 8 adapters of rank 16
    6: Workload("dense-qwen3-32b-like", T=32, H=5120, I=25600, E=1, topk=1, L=8, r=16),
}


def route(logits: np.ndarray, topk: int):
    """Softmax top-k router: highest logits first, ties to the lower expert
    index; weights are the softmax over the k selected logits."""
    order = np.argsort(-logits, axis=1, kind="stable")[:, :topk]
    sel = np.take_along_axis(logits, order, axis=1)
    sel = sel - sel.max(axis=1, keepdims=True)
    w = np.exp(sel)
    w /= w.sum(axis=1, keepdims=True)
    return order.astype(np.int32), w.astype(np.float32)


def adapter_ids(wl: Workload) -> np.ndarray:
    T, L = wl.T, wl.L
    u = uniform(stream_key(wl.seed, 2, 0, 0), T)
    if wl.lora_mode == "uniform":
        ids = np.minimum((u * L).astype(np.int64), L - 1)
    elif wl.lora_mode == "uniform_with_none":
        ids = np.minimum((u * (L + 1)).astype(np.int64), L) - 1
    elif wl.lora_mode == "zipf":
        p = (np.arange(1, L + 1, dtype=np.float64)) ** (-wl.zipf_s)
        cdf = np.cumsum(p / p.sum())
        ids = np.minimum(np.searchsorted(cdf, u, side="right"), L - 1)
    elif wl.lora_mode == "none_fraction":
        ids = np.minimum((u * L).astype(np.int64), L - 1)
        perm = np.argsort(uniform(stream_key(wl.seed, 2, 1, 0), T), kind="stable")
        ids[perm[: int(np.floor(wl.none_fraction * T))]] = -1
    elif wl.lora_mode == "none":
        ids = np.full(T, -1, dtype=np.int64)
    else:
        raise ValueError(wl.lora_mode)
    return ids.astype(np.int32)


@dataclass
class Inputs:
    wl: Workload
    x: np.ndarray
    topk_ids: np.ndarray
    topk_weights: np.ndarray
    lora_ids: np.ndarray
    W_gu: np.ndarray
    W_down: np.ndarray
    A_gu: np.ndarray
    B_gu: np.ndarray
    A_down: np.ndarray
    B_down: np.ndarray
    extra: dict = field(default_factory=dict)

    def arrays(self):
        return dict(x=self.x, topk_ids=self.topk_ids, topk_weights=self.topk_weights,
                    lora_ids=self.lora_ids, W_gu=self.W_gu, W_down=self.W_down,
                    A_gu=self.A_gu, B_gu=self.B_gu, A_down=self.A_down, B_down=self.B_down)


def make_routing(wl: Workload):
    logits = normal(stream_key(wl.seed, 0, 0, 0), wl.T * wl.E).reshape(wl.T, wl.E)
    if wl.bias_std > 0:
        logits = logits + normal(stream_key(wl.seed, 1, 0, 0), wl.E, 0.0, wl.bias_std)[None, :]
    return route(logits, wl.topk)


def make_inputs(wl, seed: int | None = None, T: int | None = None, touched_only: bool = False,
                **overrides) -> Inputs:
    """Generate one workload.  ``wl`` is a workload number or a Workload.

    ``touched_only`` leaves weight slabs that no (token, slot) pair reads as
    zeros, which saves host time on the largest shapes."""
    if isinstance(wl, int):
        wl = WORKLOADS[wl]
    if seed is not None:
        overrides["seed"] = seed
    if T is not None:
        overrides["T"] = T
    if overrides:
        wl = replace(wl, **overrides)
    T, H, I, E, k, L, r = wl.T, wl.H, wl.I, wl.E, wl.topk, wl.L, wl.r
    topk_ids, topk_weights = make_routing(wl)
    lora_ids = adapter_ids(wl)
    x = np.empty((T, H), dtype=np.uint16)
    normal_bf16_into(stream_key(wl.seed, 3, 0, 0), x.reshape(-1), wl.x_std)

    arrays = {}
    for name, shp in weight_shapes(wl).items():
        arrays[name] = np.zeros(shp, dtype=np.uint16)
    for spec in slab_specs(wl, topk_ids, lora_ids, touched_only):
        fill_slab(spec, arrays[spec.name][spec.index].reshape(-1))
    W_gu, W_down = arrays["W_gu"], arrays["W_down"]
    A_gu, B_gu, A_down, B_down = arrays["A_gu"], arrays["B_gu"], arrays["A_down"], arrays["B_down"]
    return Inputs(wl, x, topk_ids, topk_weights, lora_ids, W_gu, W_down, A_gu, B_gu, A_down, B_down)


# weight stacks: (stream tag, per-slab shape, outer (slab) dims)
def weight_layout(wl: Workload) -> dict:
    T, H, I, E, L, r = wl.T, wl.H, wl.I, wl.E, wl.L, wl.r
    return {"W_gu": (4, (2 * I, H), (E,)), "W_down": (5, (H, I), (E,)),
            "A_gu": (6, (r, H), (L, E)), "B_gu": (7, (2 * I, r), (L, E)),
            "A_down": (8, (r, I), (L, E)), "B_down": (9, (H, r), (L, E))}


def weight_shapes(wl: Workload) -> dict:
    return {n: outer + per for n, (tag, per, outer) in weight_layout(wl).items()}


@dataclass(frozen=True)
class SlabSpec:
    name: str
    index: tuple
    size: int
    key: int
    std: float


def touched(wl: Workload, topk_ids: np.ndarray, lora_ids: np.ndarray):
    """Experts and (adapter, expert) pairs that some (token, slot) pair reads."""
    used_e = np.zeros(wl.E, dtype=bool)
    used_le = np.zeros((wl.L, wl.E), dtype=bool)
    ok = (topk_ids >= 0) & (topk_ids < wl.E)
    used_e[np.unique(topk_ids[ok])] = True
    for l in range(wl.L):
        sel = topk_ids[(lora_ids == l)[:, None] & ok]
        if sel.size:
            used_le[l, np.unique(sel)] = True
    return used_e, used_le


def slab_specs(wl: Workload, topk_ids, lora_ids, touched_only: bool = False, only=None):
    """Every weight slab to draw: (stack name, slab index, element count, stream key).
    ``only`` optionally restricts to a set of expert ids."""
    used_e, used_le = touched(wl, topk_ids, lora_ids)
    out = []
    for name, (tag, per, outer) in weight_layout(wl).items():
        size = int(np.prod(per))
        for idx in np.ndindex(*outer):
            e = idx[-1]
            if only is not None and e not in only:
                continue
            if touched_only and (not used_e[e] if len(idx) == 1 else not used_le[idx[0], e]):
                continue
            a = idx[0]
            b = idx[1] if len(idx) > 1 else 0
            out.append(SlabSpec(name, idx, size, stream_key(wl.seed, tag, a, b), wl.w_std))
    return out


def fill_slab(spec: SlabSpec, out: np.ndarray) -> None:
    normal_bf16_into(spec.key, out, spec.std)


def device_inputs(wl, seed=None, touched_only=True, device="cuda", keep_host=False, **overrides):
    """Generate a workload straight into device tensors, slab by slab through a
    pinned staging buffer (the largest shape has ~28 GB of weights).  Returns
    (dict of device tensors, host Inputs).  The host Inputs hold the ids, x
    and router outputs; its weight stacks are zero-filled placeholders unless
    ``keep_host`` is set (lazily allocated, so untouched pages cost nothing)."""
    import torch
    if isinstance(wl, int):
        wl = WORKLOADS[wl]
    if seed is not None:
        overrides["seed"] = seed
    if overrides:
        wl = replace(wl, **overrides)
    topk_ids, topk_weights = make_routing(wl)
    lora_ids = adapter_ids(wl)
    x = np.empty((wl.T, wl.H), dtype=np.uint16)
    normal_bf16_into(stream_key(wl.seed, 3, 0, 0), x.reshape(-1), wl.x_std)
    dev = dict(
        x=torch.from_numpy(x.view(np.int16)).to(device).view(torch.bfloat16),
        topk_ids=torch.from_numpy(topk_ids).to(device),
        topk_weights=torch.from_numpy(topk_weights).to(device),
        lora_ids=torch.from_numpy(lora_ids).to(device))
    host_w = {}
    for name, shp in weight_shapes(wl).items():
        dev[name] = torch.zeros(shp, dtype=torch.bfloat16, device=device)
        host_w[name] = np.zeros(shp, dtype=np.uint16)
    specs = slab_specs(wl, topk_ids, lora_ids, touched_only)
    biggest = max((s.size for s in specs), default=1)
    stage = torch.empty(biggest, dtype=torch.int16, pin_memory=True)
    stage_np = stage.numpy().view(np.uint16)
    for spec in specs:
        buf = stage_np[:spec.size]
        fill_slab(spec, buf)
        dst = dev[spec.name][spec.index].view(-1).view(torch.int16)
        dst.copy_(stage[:spec.size], non_blocking=True)
        torch.cuda.current_stream().synchronize()  # the staging buffer is reused
        if keep_host:
            host_w[spec.name][spec.index].reshape(-1)[:] = buf
    inp = Inputs(wl, x, topk_ids, topk_weights, lora_ids, **host_w)
    inp.extra["host_weights"] = bool(keep_host)  # host stacks hold every slab drawn
    return dev, inp


def host_slabs_for_tokens(inp: Inputs, tokens) -> None:
    """Fill the host weight stacks of ``inp`` with the slabs that the given
    tokens read (for a CPU reference on a sample of tokens).  A no-op when
    the bundle already holds every drawn slab (device_inputs(keep_host=True))."""
    if inp.extra.get("host_weights"):
        return
    wl = inp.wl
    ids = inp.topk_ids[tokens]
    lids = inp.lora_ids[tokens]
    arrays = dict(W_gu=inp.W_gu, W_down=inp.W_down, A_gu=inp.A_gu, B_gu=inp.B_gu,
                  A_down=inp.A_down, B_down=inp.B_down)
    for spec in slab_specs(wl, ids, lids, touched_only=True):
        fill_slab(spec, arrays[spec.name][spec.index].reshape(-1))


def algorithmic_work(wl: Workload, topk_ids: np.ndarray, lora_ids: np.ndarray) -> dict:
    """Bytes and flops the layer must move / compute for this routed instance:
    every touched expert's base weights once, every touched (adapter, expert)
    A and B once, x read, y written, ids and weights read.  Padding, materialised
    intermediates and untouched slabs are excluded."""
    T, H, I, E, k, L, r = wl.T, wl.H, wl.I, wl.E, wl.topk, wl.L, wl.r
    valid = (topk_ids >= 0) & (topk_ids < E)
    e_touched = np.unique(topk_ids[valid])
    lid = np.broadcast_to(lora_ids[:, None], topk_ids.shape)
    has = valid & (lid >= 0) & (lid < L)
    le = np.unique(lid[has].astype(np.int64) * E + topk_ids[has])
    P = int(valid.sum())
    P_l = int(has.sum())
    n_e, n_le = len(e_touched), len(le)
    w_gu = n_e * 2 * I * H * 2
    w_down = n_e * H * I * 2
    a_gu = n_le * r * H * 2
    b_gu = n_le * 2 * I * r * 2
    a_down = n_le * r * I * 2
    b_down = n_le * H * r * 2
    io = T * H * 2 + T * H * 2 + T * k * 8 + T * 4
    return dict(
        bytes=w_gu + w_down + a_gu + b_gu + a_down + b_down + io,
        flops=2 * P * 3 * H * I + 2 * P_l * r * (2 * H + 3 * I),
        bytes_parts=dict(W_gu=w_gu, W_down=w_down, A_gu=a_gu, B_gu=b_gu, A_down=a_down,
                         B_down=b_down, io=io),
        experts_touched=n_e, pairs_touched=n_le, P=P, P_l=P_l)
