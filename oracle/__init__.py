"""fp64 CPU reference ("oracle") of the fused MoE-LoRA layer.

TEST INFRASTRUCTURE ONLY: only ``tests/``, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` may import this package.  The HIP library in
``lora_moe_amd`` never uses it.  The arithmetic lives in
``moe_lora_oracle.c``; this module compiles it and marshals numpy arrays.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "moe_lora_oracle.c")
_SO = os.path.join(_HERE, "libmoe_lora_oracle.so")
_lib = None


def compile_to(out_path: str, src: str = _SRC) -> str:
    """Compile the reference (plain C, fp64, OpenMP, no fast-math)."""
    tmp = out_path + ".tmp%d" % os.getpid()
    subprocess.check_call(["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c11", src,
                           "-o", tmp, "-lm"])
    os.replace(tmp, out_path)
    return out_path


def build(force: bool = True) -> str:
    if force or not os.path.exists(_SO):
        compile_to(_SO)
    return _SO


def _bind(lib):
    i, d, vp = ctypes.c_int, ctypes.c_double, ctypes.c_void_p
    lib.orc_layer.restype = i
    lib.orc_layer.argtypes = [i, i, i, i, i, i, i, d] + [vp] * 10 + [vp, i, vp, i]
    lib.orc_pair.restype = i
    lib.orc_pair.argtypes = [i, i, i, i, i, i, i, d] + [vp] * 9 + [i, i] + [vp] * 5
    lib.orc_align.restype = i
    lib.orc_align.argtypes = [i, i, i, i, i, vp, vp, i, i] + [vp] * 8
    lib.orc_route.restype = i
    lib.orc_route.argtypes = [i, i, i, vp, vp, vp]
    return lib


def load(path: str | None = None):
    """Load the compiled reference (the default build, or another .so such as
    a deliberately broken copy used to check that the pins catch mistakes)."""
    global _lib
    if path is not None:
        return _bind(ctypes.CDLL(path))
    if _lib is None:
        if not os.path.exists(_SO):
            build(force=False)
        _lib = _bind(ctypes.CDLL(_SO))
    return _lib


def _c(a, dtype):
    a = np.ascontiguousarray(a, dtype=dtype)
    return a, a.ctypes.data


def default_threads() -> int:
    try:
        return len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        return os.cpu_count() or 1


class Oracle:
    """Calls into one compiled copy of the reference."""

    def __init__(self, path: str | None = None):
        self.lib = load(path)

    def layer(self, shape, x, topk_ids, topk_weights, lora_ids, W_gu, W_down, A_gu, B_gu,
              A_down, B_down, tokens=None, scale=None, nthreads=None) -> np.ndarray:
        """y[t, :] in fp64 for every token (or for ``tokens``)."""
        T, H, I, E, k, L, r = shape
        s = 1.0 if scale is None else float(scale)
        keep = []
        ptrs = []
        for a, dt in ((x, np.uint16), (topk_ids, np.int32), (topk_weights, np.float32),
                      (lora_ids, np.int32), (W_gu, np.uint16), (W_down, np.uint16),
                      (A_gu, np.uint16), (B_gu, np.uint16), (A_down, np.uint16),
                      (B_down, np.uint16)):
            arr, p = _c(a, dt)
            keep.append(arr)
            ptrs.append(p)
        if tokens is None:
            n = T
            tok_p = None
        else:
            tok, tok_p = _c(tokens, np.int32)
            keep.append(tok)
            n = len(tok)
        y = np.zeros((n, H), dtype=np.float64)
        rc = self.lib.orc_layer(T, H, I, E, k, L, r, s, *ptrs, tok_p, n, y.ctypes.data,
                                nthreads or default_threads())
        if rc != 0:
            raise MemoryError("oracle scratch allocation failed")
        return y

    def pair(self, shape, x, topk_ids, lora_ids, W_gu, W_down, A_gu, B_gu, A_down, B_down,
             t, j, scale=None) -> dict | None:
        """Intermediates of pair (t, j): g, zg, h, zd, d (fp64)."""
        T, H, I, E, k, L, r = shape
        s = 1.0 if scale is None else float(scale)
        keep, ptrs = [], []
        for a, dt in ((x, np.uint16), (topk_ids, np.int32), (lora_ids, np.int32),
                      (W_gu, np.uint16), (W_down, np.uint16), (A_gu, np.uint16),
                      (B_gu, np.uint16), (A_down, np.uint16), (B_down, np.uint16)):
            arr, p = _c(a, dt)
            keep.append(arr)
            ptrs.append(p)
        out = dict(g=np.zeros(2 * I), zg=np.zeros(max(r, 1)), h=np.zeros(I), zd=np.zeros(max(r, 1)),
                   d=np.zeros(H))
        rc = self.lib.orc_pair(T, H, I, E, k, L, r, s, *ptrs, int(t), int(j),
                               *(out[n].ctypes.data for n in ("g", "zg", "h", "zd", "d")))
        if rc != 0:
            return None
        out["zg"] = out["zg"][:r]
        out["zd"] = out["zd"][:r]
        return out

    def align(self, T, k, E, L, block_m, topk_ids, lora_ids, cap_rows=None, cap_blocks=None):
        """Reference align outputs as a dict of int32 arrays."""
        P = T * k
        if cap_rows is None:
            cap_rows = P + E * (block_m - 1)
        if cap_blocks is None:
            cap_blocks = (cap_rows + block_m - 1) // block_m
        ids, ids_p = _c(np.asarray(topk_ids).reshape(-1), np.int32)
        lids, lids_p = _c(lora_ids, np.int32)
        out = dict(sorted_ids=np.zeros(max(cap_rows, 1), np.int32),
                   expert_off=np.zeros(E + 1, np.int32),
                   seg_start=np.zeros(E * (L + 1), np.int32),
                   seg_cnt=np.zeros(E * (L + 1), np.int32),
                   block_expert=np.zeros(max(cap_blocks, 1), np.int32),
                   pos_of_pair=np.zeros(max(P, 1), np.int32),
                   num_padded=np.zeros(1, np.int32), err_count=np.zeros(1, np.int32))
        rc = self.lib.orc_align(T, k, E, L, block_m, ids_p, lids_p, cap_rows, cap_blocks,
                                *(out[n].ctypes.data for n in (
                                    "sorted_ids", "expert_off", "seg_start", "seg_cnt",
                                    "block_expert", "pos_of_pair", "num_padded", "err_count")))
        if rc != 0:
            raise ValueError("align capacity too small")
        out["sorted_ids"] = out["sorted_ids"][:cap_rows]
        out["block_expert"] = out["block_expert"][:cap_blocks]
        out["pos_of_pair"] = out["pos_of_pair"][:P]
        out["num_padded"] = int(out["num_padded"][0])
        out["err_count"] = int(out["err_count"][0])
        return out


    def route(self, logits, k):
        """Reference router: (ids [T][k] int32, weights [T][k] float64)."""
        lg, lg_p = _c(logits, np.float32)
        T, E = lg.shape
        ids = np.zeros((T, k), np.int32)
        w = np.zeros((T, k), np.float64)
        if T == 0:
            return ids, w
        rc = self.lib.orc_route(T, E, k, lg_p, ids.ctypes.data, w.ctypes.data)
        if rc != 0:
            raise ValueError("k outside [1, E]")
        return ids, w


def layer_from_inputs(inp, tokens=None, oracle: Oracle | None = None, nthreads=None, scale=None):
    """Convenience: run the reference on a ``synth.Inputs`` bundle."""
    o = oracle or Oracle()
    wl = inp.wl
    shape = (wl.T, wl.H, wl.I, wl.E, wl.topk, wl.L, wl.r)
    return o.layer(shape, inp.x, inp.topk_ids, inp.topk_weights, inp.lora_ids, inp.W_gu,
                   inp.W_down, inp.A_gu, inp.B_gu, inp.A_down, inp.B_down, tokens=tokens,
                   scale=wl.scale if scale is None else scale, nthreads=nthreads)
