"""Python binding of the MoE-LoRA C ABI (``include/moe_lora.h``).

Argument marshalling only: every step of the layer runs in the HIP kernels of
``libmoe_lora.so``.  Functions carry the C names; tensors are torch tensors on
the current HIP device (PyTorch supplies device memory and streams).  Loading
fails loudly when the library has not been built -- there is no fallback.
"""
from __future__ import annotations

import ctypes
import os

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libmoe_lora.so")
TUNING_PATH = os.path.join(PKG, "tuning", "gfx950.json")

MOE_LORA_OK = 0
MOE_LORA_EINVAL = -1
MOE_LORA_EALIGN = -2
MOE_LORA_EWORKSPACE = -3
MOE_LORA_EUNSUPPORTED = -4
MOE_LORA_EHIP = -5
MOE_LORA_NOALLOC_WORKSPACE_BYTES = 64 << 20  # the static workspace of moe_lora_forward_noalloc

_lib = None


class MoeLoraError(RuntimeError):
    def __init__(self, func: str, code: int):
        self.code = code
        super().__init__(f"{func} failed: {moe_lora_status_str(code)} ({code})")


KNOBS = ("shrink_splits", "shrink_zblocks", "down_splits", "tile_order", "expand_mode")


class moe_lora_shape(ctypes.Structure):
    _fields_ = [("T", ctypes.c_int32), ("H", ctypes.c_int32), ("I", ctypes.c_int32),
                ("E", ctypes.c_int32), ("topk", ctypes.c_int32), ("L", ctypes.c_int32),
                ("r", ctypes.c_int32), ("block_m", ctypes.c_int32),
                ("lora_scale", ctypes.c_float)] + [(k, ctypes.c_int32) for k in KNOBS]

    def __repr__(self):
        return ("moe_lora_shape(" + ", ".join(f"{n}={getattr(self, n)}" for n, _ in self._fields_)
                + ")")


class moe_lora_views(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in (
        "sorted_ids", "expert_off", "seg_start", "seg_cnt", "block_expert", "pos_of_pair",
        "num_padded", "err_count", "z_gu", "z_down", "h", "d")] + [
        ("cap_rows", ctypes.c_int64), ("cap_blocks", ctypes.c_int64), ("block_m", ctypes.c_int32),
        ("d_splits", ctypes.c_int32), ("h_lo", ctypes.c_void_p)]


ALIGN_VIEW_FIELDS = ("sorted_ids", "expert_off", "seg_start", "seg_cnt", "block_expert",
                     "pos_of_pair", "num_padded", "err_count")


class moe_lora_align_ptrs(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in ALIGN_VIEW_FIELDS]


class moe_lora_tune_entry(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in ("rows_per_expert", "H", "I", "E", "r", "L", "block_m")
                + KNOBS]


# An entry's tuned configuration applies to shapes within this distance of
# its key (sum over rows per expert (x4), H, I, E, r, L of |log2 ratio|):
# e.g. a shape with half or twice the entry's rows per expert and the same
# sizes otherwise; farther shapes keep the built-in choice.
TUNE_MAX_DIST = 4.0


def make_shape(T, H, I, E, topk, L, r, block_m=0, lora_scale=1.0, tuning=None,
               max_dist=TUNE_MAX_DIST, **knobs) -> moe_lora_shape:
    """The shape struct (knobs: shrink_splits, shrink_zblocks, down_splits,
    tile_order, expand_mode; 0 = the library's choice).  With a tuning table
    (load_tuning), every field left at 0 is taken from the table's nearest
    entry within max_dist (moe_lora_tune_apply)."""
    s = moe_lora_shape(int(T), int(H), int(I), int(E), int(topk), int(L), int(r), int(block_m),
                       float(lora_scale), *(int(knobs.pop(k, 0)) for k in KNOBS))
    if knobs:
        raise TypeError(f"unknown shape fields {sorted(knobs)}")
    if tuning is not None:
        s = moe_lora_tune_apply(s, tuning, max_dist)
    return s


def load_tuning(path: str = TUNING_PATH):
    """Entries of a tile-configuration table written by ``lora_moe_amd.tune``
    (JSON), as the C array moe_lora_tune_apply reads (knobs missing from an
    entry are 0)."""
    import json
    with open(path) as f:
        doc = json.load(f)
    rows = doc["entries"]
    arr = (moe_lora_tune_entry * max(1, len(rows)))()
    for i, e in enumerate(rows):
        arr[i] = moe_lora_tune_entry(*(int(e.get(n, 0)) for n, _ in moe_lora_tune_entry._fields_))
    return arr, len(rows)


def moe_lora_tune_block_m(shape: moe_lora_shape, tuning, max_dist: float = 0.0) -> int:
    table, n = tuning
    return load_library().moe_lora_tune_block_m(ctypes.byref(shape), table, int(n), float(max_dist))


def moe_lora_tune_apply(shape: moe_lora_shape, tuning, max_dist: float = 0.0) -> moe_lora_shape:
    """A copy of ``shape`` with block_m and the knobs it leaves at 0 taken
    from the nearest table entry."""
    table, n = tuning
    out = moe_lora_shape()
    _check("moe_lora_tune_apply", min(0, load_library().moe_lora_tune_apply(
        ctypes.byref(shape), table, int(n), float(max_dist), ctypes.byref(out))))
    return out


def load_library(path: str = LIB_PATH):
    """Load libmoe_lora.so (raises when it is missing: build it first)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"{path} not found: build the HIP library first "
                           "(python -c 'import __graft_entry__ as g; g.build()')")
    lib = ctypes.CDLL(path)
    vp, sp = ctypes.c_void_p, ctypes.POINTER(moe_lora_shape)
    i32 = ctypes.c_int
    lib.moe_lora_resolve_block_m.argtypes = [sp]
    lib.moe_lora_resolve_block_m.restype = i32
    lib.moe_lora_tune_block_m.argtypes = [sp, ctypes.POINTER(moe_lora_tune_entry), ctypes.c_int32,
                                          ctypes.c_float]
    lib.moe_lora_tune_block_m.restype = i32
    lib.moe_lora_tune_apply.argtypes = [sp, ctypes.POINTER(moe_lora_tune_entry), ctypes.c_int32,
                                        ctypes.c_float, sp]
    lib.moe_lora_tune_apply.restype = i32
    lib.moe_lora_workspace_bytes.argtypes = [sp]
    lib.moe_lora_workspace_bytes.restype = ctypes.c_size_t
    lib.moe_lora_align.argtypes = [sp, vp, vp, vp, ctypes.c_size_t, vp]
    lib.moe_lora_align.restype = i32
    lib.moe_lora_align_timed.argtypes = [sp, vp, vp, vp, ctypes.c_size_t, vp, vp]
    lib.moe_lora_align_timed.restype = i32
    lib.moe_lora_align_view.argtypes = [sp, vp, ctypes.POINTER(moe_lora_align_ptrs)]
    lib.moe_lora_align_view.restype = i32
    lib.moe_lora_route.argtypes = [sp, vp, vp, vp, vp]
    lib.moe_lora_route.restype = i32
    lib.moe_lora_route_align.argtypes = [sp, vp, vp, vp, vp, vp, ctypes.c_size_t, vp]
    lib.moe_lora_route_align.restype = i32
    lib.moe_lora_route_align_timed.argtypes = [sp, vp, vp, vp, vp, vp, ctypes.c_size_t, vp, vp]
    lib.moe_lora_route_align_timed.restype = i32
    lib.moe_lora_workspace_view.argtypes = [sp, vp, ctypes.POINTER(moe_lora_views)]
    lib.moe_lora_workspace_view.restype = i32
    lib.moe_lora_forward.argtypes = [sp] + [vp] * 11 + [ctypes.c_size_t, vp, vp]
    lib.moe_lora_forward.restype = i32
    lib.moe_lora_forward_timed.argtypes = [sp] + [vp] * 11 + [ctypes.c_size_t, vp, vp, vp]
    lib.moe_lora_forward_timed.restype = i32
    lib.moe_lora_forward_noalloc.argtypes = [sp] + [vp] * 11 + [vp]
    lib.moe_lora_forward_noalloc.restype = i32
    lib.moe_lora_device_errors.argtypes = [sp, vp, ctypes.POINTER(ctypes.c_int32), vp]
    lib.moe_lora_device_errors.restype = i32
    lib.moe_lora_status_str.argtypes = [i32]
    lib.moe_lora_status_str.restype = ctypes.c_char_p
    lib.moe_lora_stage_count.argtypes = []
    lib.moe_lora_stage_count.restype = i32
    lib.moe_lora_stage_name.argtypes = [i32]
    lib.moe_lora_stage_name.restype = ctypes.c_char_p
    lib.moe_lora_profiler_create.argtypes = [i32, ctypes.c_uint32, ctypes.POINTER(vp)]
    lib.moe_lora_profiler_create.restype = i32
    lib.moe_lora_profiler_read.argtypes = [vp, ctypes.POINTER(ctypes.c_float), i32,
                                           ctypes.POINTER(ctypes.c_int)]
    lib.moe_lora_profiler_read.restype = i32
    lib.moe_lora_profiler_destroy.argtypes = [vp]
    lib.moe_lora_profiler_destroy.restype = None
    _lib = lib
    return lib


def _check(func: str, code: int):
    if code != MOE_LORA_OK:
        raise MoeLoraError(func, code)


def _ptr(t, name: str):
    """Device address of a contiguous tensor (None -> NULL)."""
    if t is None:
        return None
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    return t.data_ptr()


def layer_operand_specs(shape) -> dict:
    """Expected (shape, dtype name) of every tensor the calls take, from the
    layer sizes in ``shape``."""
    T, H, I, E, k, L, r = shape.T, shape.H, shape.I, shape.E, shape.topk, shape.L, shape.r
    return dict(
        x=((T, H), "bfloat16"), topk_ids=((T, k), "int32"), topk_weights=((T, k), "float32"),
        lora_ids=((T,), "int32"), W_gu=((E, 2 * I, H), "bfloat16"), W_down=((E, H, I), "bfloat16"),
        A_gu=((L, E, r, H), "bfloat16"), B_gu=((L, E, 2 * I, r), "bfloat16"),
        A_down=((L, E, r, I), "bfloat16"), B_down=((L, E, H, r), "bfloat16"),
        y=((T, H), "bfloat16"), logits=((T, E), "float32"))


def check_operands(shape, workspace=None, **tensors) -> None:
    """Raise ValueError unless every given tensor has the dtype and shape the
    kernels assume for ``shape``, is contiguous, and all of them (workspace
    included) are device tensors on one device; the workspace must be a uint8
    tensor of at least moe_lora_workspace_bytes(shape) bytes.  Runs before
    any launch: a wrong dtype (int64 ids from torch.topk, say) or a short
    weight stack would otherwise be read as something else, or past its end."""
    specs = layer_operand_specs(shape)
    devices = set()
    for name, t in tensors.items():
        if t is None:
            raise ValueError(f"{name} is required")
        want_shape, want_dtype = specs[name]
        got_dtype = str(t.dtype).replace("torch.", "")
        if got_dtype != want_dtype:
            raise ValueError(f"{name}: dtype {got_dtype}, expected {want_dtype}")
        if tuple(t.shape) != want_shape:
            raise ValueError(f"{name}: shape {tuple(t.shape)}, expected {want_shape}")
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
        devices.add(t.device)
    if workspace is not None:
        if str(workspace.dtype) != "torch.uint8" or workspace.dim() != 1:
            raise ValueError("workspace must be a 1-D uint8 tensor (alloc_workspace)")
        need = moe_lora_workspace_bytes(shape)
        if need == 0:
            raise MoeLoraError("moe_lora_workspace_bytes", MOE_LORA_EINVAL)
        if workspace.numel() < need:
            raise ValueError(f"workspace holds {workspace.numel()} bytes, the shape needs {need}")
        devices.add(workspace.device)
    for d in devices:
        if d.type != "cuda":
            raise ValueError(f"operands must be device tensors (got one on {d})")
    if len(devices) > 1:
        raise ValueError(f"operands on several devices: {sorted(str(d) for d in devices)}")


def _stream(stream):
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    return getattr(stream, "cuda_stream", stream)


def moe_lora_status_str(code: int) -> str:
    return load_library().moe_lora_status_str(int(code)).decode()


def moe_lora_resolve_block_m(shape: moe_lora_shape) -> int:
    return load_library().moe_lora_resolve_block_m(ctypes.byref(shape))


def moe_lora_workspace_bytes(shape: moe_lora_shape) -> int:
    return int(load_library().moe_lora_workspace_bytes(ctypes.byref(shape)))


def alloc_workspace(shape: moe_lora_shape, device="cuda"):
    import torch
    n = moe_lora_workspace_bytes(shape)
    if n == 0:
        raise MoeLoraError("moe_lora_workspace_bytes", MOE_LORA_EINVAL)
    return torch.empty(n, dtype=torch.uint8, device=device)


def _prof(profiler):
    return None if profiler is None else profiler.handle


def moe_lora_route(shape, logits, topk_ids, topk_weights, stream=None) -> None:
    """Top-k experts and weights of each token from fp32 logits [T, E] into
    topk_ids [T, k] (int32) and topk_weights [T, k] (fp32)."""
    check_operands(shape, logits=logits, topk_ids=topk_ids, topk_weights=topk_weights)
    _check("moe_lora_route", load_library().moe_lora_route(
        ctypes.byref(shape), _ptr(logits, "logits"), _ptr(topk_ids, "topk_ids"),
        _ptr(topk_weights, "topk_weights"), _stream(stream)))


def moe_lora_route_align(shape, logits, lora_ids, topk_ids, topk_weights, workspace,
                         stream=None, profiler=None) -> None:
    """moe_lora_route then moe_lora_align on the routed ids (one kernel for
    small batches)."""
    check_operands(shape, workspace, logits=logits, lora_ids=lora_ids, topk_ids=topk_ids,
                   topk_weights=topk_weights)
    _check("moe_lora_route_align", load_library().moe_lora_route_align_timed(
        ctypes.byref(shape), _ptr(logits, "logits"), _ptr(lora_ids, "lora_ids"),
        _ptr(topk_ids, "topk_ids"), _ptr(topk_weights, "topk_weights"),
        _ptr(workspace, "workspace"), workspace.numel() * workspace.element_size(),
        _stream(stream), _prof(profiler)))


def moe_lora_align(shape, topk_ids, lora_ids, workspace, stream=None, profiler=None) -> None:
    check_operands(shape, workspace, topk_ids=topk_ids, lora_ids=lora_ids)
    _check("moe_lora_align", load_library().moe_lora_align_timed(
        ctypes.byref(shape), _ptr(topk_ids, "topk_ids"), _ptr(lora_ids, "lora_ids"),
        _ptr(workspace, "workspace"), workspace.numel() * workspace.element_size(),
        _stream(stream), _prof(profiler)))


def moe_lora_forward(shape, x, topk_ids, topk_weights, lora_ids, W_gu, W_down, A_gu, B_gu,
                     A_down, B_down, workspace, y, stream=None, profiler=None) -> None:
    check_operands(shape, workspace, x=x, topk_ids=topk_ids, topk_weights=topk_weights,
                   lora_ids=lora_ids, W_gu=W_gu, W_down=W_down, A_gu=A_gu, B_gu=B_gu,
                   A_down=A_down, B_down=B_down, y=y)
    _check("moe_lora_forward", load_library().moe_lora_forward_timed(
        ctypes.byref(shape), _ptr(x, "x"), _ptr(topk_ids, "topk_ids"),
        _ptr(topk_weights, "topk_weights"), _ptr(lora_ids, "lora_ids"), _ptr(W_gu, "W_gu"),
        _ptr(W_down, "W_down"), _ptr(A_gu, "A_gu"), _ptr(B_gu, "B_gu"), _ptr(A_down, "A_down"),
        _ptr(B_down, "B_down"), _ptr(workspace, "workspace"),
        workspace.numel() * workspace.element_size(), _ptr(y, "y"), _stream(stream),
        _prof(profiler)))


def moe_lora_forward_noalloc(shape, x, topk_ids, topk_weights, lora_ids, W_gu, W_down, A_gu, B_gu,
                             A_down, B_down, y, stream=None) -> None:
    """Align + forward with the library's static workspace (for callers that
    cannot allocate); shapes whose workspace exceeds
    MOE_LORA_NOALLOC_WORKSPACE_BYTES raise MoeLoraError (EWORKSPACE)."""
    check_operands(shape, x=x, topk_ids=topk_ids, topk_weights=topk_weights, lora_ids=lora_ids,
                   W_gu=W_gu, W_down=W_down, A_gu=A_gu, B_gu=B_gu, A_down=A_down, B_down=B_down,
                   y=y)
    _check("moe_lora_forward_noalloc", load_library().moe_lora_forward_noalloc(
        ctypes.byref(shape), _ptr(x, "x"), _ptr(topk_ids, "topk_ids"),
        _ptr(topk_weights, "topk_weights"), _ptr(lora_ids, "lora_ids"), _ptr(W_gu, "W_gu"),
        _ptr(W_down, "W_down"), _ptr(A_gu, "A_gu"), _ptr(B_gu, "B_gu"), _ptr(A_down, "A_down"),
        _ptr(B_down, "B_down"), _ptr(y, "y"), _stream(stream)))


def moe_lora_align_view(shape, workspace) -> dict:
    """Device addresses (ints) of the align outputs in ``workspace``."""
    v = moe_lora_align_ptrs()
    _check("moe_lora_align_view", load_library().moe_lora_align_view(
        ctypes.byref(shape), ctypes.c_void_p(workspace if isinstance(workspace, int)
                                             else workspace.data_ptr()), ctypes.byref(v)))
    return {n: getattr(v, n) for n in ALIGN_VIEW_FIELDS}


def moe_lora_workspace_view(shape, workspace) -> moe_lora_views:
    v = moe_lora_views()
    _check("moe_lora_workspace_view", load_library().moe_lora_workspace_view(
        ctypes.byref(shape), _ptr(workspace, "workspace"), ctypes.byref(v)))
    return v


def workspace_tensors(shape, workspace) -> dict:
    """The workspace regions of ``moe_lora_workspace_view`` as torch views of
    ``workspace`` (a uint8 device tensor)."""
    import torch
    v = moe_lora_workspace_view(shape, workspace)
    base = workspace.data_ptr()
    P = shape.T * shape.topk
    NB = shape.E * (shape.L + 1)
    cap, capb = v.cap_rows, v.cap_blocks

    def region(addr, n, dtype):
        nbytes = n * torch.empty((), dtype=dtype).element_size()
        off = addr - base
        return workspace[off:off + nbytes].view(dtype)

    return dict(
        sorted_ids=region(v.sorted_ids, cap, torch.int32),
        expert_off=region(v.expert_off, shape.E + 1, torch.int32),
        seg_start=region(v.seg_start, NB, torch.int32),
        seg_cnt=region(v.seg_cnt, NB, torch.int32),
        block_expert=region(v.block_expert, capb, torch.int32),
        pos_of_pair=region(v.pos_of_pair, P, torch.int32),
        num_padded=region(v.num_padded, 1, torch.int32),
        err_count=region(v.err_count, 1, torch.int32),
        z_gu=region(v.z_gu, cap * shape.r, torch.float32).view(cap, shape.r),
        z_down=region(v.z_down, cap * shape.r, torch.float32).view(cap, shape.r),
        h=region(v.h, cap * shape.I, torch.bfloat16).view(cap, shape.I),
        d=region(v.d, v.d_splits * cap * shape.H, torch.float32).view(v.d_splits, cap, shape.H),
        h_lo=(region(v.h_lo, cap * shape.I, torch.bfloat16).view(cap, shape.I) if v.h_lo else None),
        cap_rows=cap, cap_blocks=capb, block_m=v.block_m, d_splits=v.d_splits)


def moe_lora_device_errors(shape, workspace, stream=None) -> int:
    n = ctypes.c_int32(0)
    _check("moe_lora_device_errors", load_library().moe_lora_device_errors(
        ctypes.byref(shape), _ptr(workspace, "workspace"), ctypes.byref(n), _stream(stream)))
    return int(n.value)


def moe_lora_stage_count() -> int:
    return load_library().moe_lora_stage_count()


def moe_lora_stage_name(i: int) -> str:
    return load_library().moe_lora_stage_name(int(i)).decode()


class Profiler:
    """A caller-owned stage-timing recorder (moe_lora_profiler_create): pass
    it as ``profiler=`` to align / route_align / forward; ``read()`` waits
    for the recorded events and returns the summed milliseconds per stage
    name and the number of recorded calls."""

    def __init__(self, max_calls: int, stages=None):
        mask = 0xFFFFFFFF
        if stages is not None:
            names = [moe_lora_stage_name(i) for i in range(moe_lora_stage_count())]
            mask = 0
            for st in stages:
                mask |= 1 << names.index(st)
        h = ctypes.c_void_p()
        _check("moe_lora_profiler_create", load_library().moe_lora_profiler_create(
            int(max_calls), mask, ctypes.byref(h)))
        self.handle = h

    def read(self) -> tuple[dict, int]:
        n = moe_lora_stage_count()
        arr = (ctypes.c_float * n)()
        calls = ctypes.c_int(0)
        _check("moe_lora_profiler_read", load_library().moe_lora_profiler_read(
            self.handle, arr, n, ctypes.byref(calls)))
        return {moe_lora_stage_name(i): float(arr[i]) for i in range(n)}, int(calls.value)

    def close(self) -> None:
        if self.handle:
            load_library().moe_lora_profiler_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def fused_moe_lora(x, topk_ids, topk_weights, lora_ids, W_gu, W_down, A_gu, B_gu, A_down, B_down,
                   lora_scale=1.0, block_m=0, workspace=None, y=None, stream=None):
    """Align + forward on the current stream; returns y [T, H] (bf16).

    x [T,H] bf16; topk_ids [T,k] int32; topk_weights [T,k] fp32; lora_ids [T]
    int32; W_gu [E,2I,H]; W_down [E,H,I]; A_gu [L,E,r,H]; B_gu [L,E,2I,r];
    A_down [L,E,r,I]; B_down [L,E,H,r] (all bf16)."""
    import torch
    for name, t, nd in (("x", x, 2), ("topk_ids", topk_ids, 2), ("W_gu", W_gu, 3), ("A_gu", A_gu, 4)):
        if t.dim() != nd:
            raise ValueError(f"{name}: {t.dim()} dimensions, expected {nd}")
    T, H = x.shape
    E, twoI, _ = W_gu.shape
    L, _, r, _ = A_gu.shape
    shape = make_shape(T, H, twoI // 2, E, topk_ids.shape[1], L, r, block_m, lora_scale)
    check_operands(shape, x=x, topk_ids=topk_ids, topk_weights=topk_weights, lora_ids=lora_ids,
                   W_gu=W_gu, W_down=W_down, A_gu=A_gu, B_gu=B_gu, A_down=A_down, B_down=B_down)
    if workspace is None:
        workspace = alloc_workspace(shape, x.device)
    if y is None:
        y = torch.empty((T, H), dtype=torch.bfloat16, device=x.device)
    moe_lora_align(shape, topk_ids, lora_ids, workspace, stream)
    moe_lora_forward(shape, x, topk_ids, topk_weights, lora_ids, W_gu, W_down, A_gu, B_gu, A_down,
                     B_down, workspace, y, stream)
    return y


__all__ = [n for n in dir() if n.startswith("moe_lora") or n in (
    "make_shape", "alloc_workspace", "workspace_tensors", "fused_moe_lora", "load_library",
    "MoeLoraError", "Profiler", "check_operands", "layer_operand_specs")]
