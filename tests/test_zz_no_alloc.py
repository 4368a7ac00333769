"""moe_lora_forward_noalloc (align + forward with the library's static
workspace, for callers that cannot allocate) against moe_lora_align +
moe_lora_forward on a caller workspace: two calls in a row, the second with
fewer tokens, each within the layer tolerance of the existing entry point's
output and of the fp64 reference."""
import ctypes

import numpy as np
import pytest
import torch

import synth
from gpu_common import compare, log, oracle_tokens, run_gpu, sample_tokens

pytestmark = pytest.mark.gpu


def noalloc(lm, shape, dev, y):
    lib = lm.load_library()
    args = [dev[n].data_ptr() for n in ("x", "topk_ids", "topk_weights", "lora_ids", "W_gu", "W_down",
                                        "A_gu", "B_gu", "A_down", "B_down")]
    return lib.moe_lora_forward_noalloc(ctypes.byref(shape), *args, y.data_ptr(),
                                        torch.cuda.current_stream().cuda_stream)


def test_noalloc_matches_workspace_path():
    import lora_moe_amd as lm
    wl = synth.WORKLOADS[3]  # 256 tokens: a 51 MB workspace, inside the 64 MB array
    dev_full, inp_full = synth.device_inputs(wl, touched_only=True, keep_host=True)
    for T in (wl.T, 100):  # the second call with a smaller input
        dev = dict(dev_full)
        for n in ("x", "topk_ids", "topk_weights", "lora_ids"):
            dev[n] = dev_full[n][:T].contiguous()
        wlT = synth.Workload(wl.name, T=T, H=wl.H, I=wl.I, E=wl.E, topk=wl.topk, L=wl.L, r=wl.r)
        shape = lm.make_shape(T, wl.H, wl.I, wl.E, wl.topk, wl.L, wl.r, 0, wl.scale)
        assert lm.moe_lora_workspace_bytes(shape) <= lm.MOE_LORA_NOALLOC_WORKSPACE_BYTES
        log(f"noalloc: T={T}")
        y = torch.full((T, wl.H), float("nan"), dtype=torch.bfloat16, device="cuda")
        assert noalloc(lm, shape, dev, y) == lm.MOE_LORA_OK
        torch.cuda.synchronize()
        got = y.float().cpu().numpy().astype(np.float64)
        want, _, _ = run_gpu(dev, wlT)
        compare(got, want, f"noalloc vs align + forward, T={T}")
        log(f"noalloc T={T}: bit-identical to the workspace path: {bool(np.array_equal(got, want))}")
        toks = sample_tokens(T, 32)
        inp = synth.Inputs(wlT, inp_full.x[:T], inp_full.topk_ids[:T], inp_full.topk_weights[:T],
                           inp_full.lora_ids[:T], inp_full.W_gu, inp_full.W_down, inp_full.A_gu,
                           inp_full.B_gu, inp_full.A_down, inp_full.B_down)
        compare(got[toks], oracle_tokens(inp, toks), f"noalloc vs reference, T={T}")


def test_noalloc_refuses_a_workspace_too_large():
    import lora_moe_amd as lm
    wl = synth.WORKLOADS[4]
    shape = lm.make_shape(wl.T, wl.H, wl.I, wl.E, wl.topk, wl.L, wl.r, 0, wl.scale)
    assert lm.moe_lora_workspace_bytes(shape) > lm.MOE_LORA_NOALLOC_WORKSPACE_BYTES
    lib = lm.load_library()
    buf = torch.zeros(64, dtype=torch.uint8, device="cuda")
    p = buf.data_ptr()
    assert lib.moe_lora_forward_noalloc(ctypes.byref(shape), *([p] * 11), None) == lm.MOE_LORA_EWORKSPACE
