"""Two layers in flight at once on two streams, each with its own workspace
(the library keeps no per-call global state): both match their results
computed alone."""
import numpy as np
import pytest
import torch

import synth
from gpu_common import log, to_device

pytestmark = pytest.mark.gpu


def run(lm, wl, dev, ws, y, stream, bm):
    shape = lm.make_shape(wl.T, wl.H, wl.I, wl.E, wl.topk, wl.L, wl.r, bm, wl.scale)
    lm.moe_lora_align(shape, dev["topk_ids"], dev["lora_ids"], ws, stream)
    lm.moe_lora_forward(shape, dev["x"], dev["topk_ids"], dev["topk_weights"], dev["lora_ids"],
                        dev["W_gu"], dev["W_down"], dev["A_gu"], dev["B_gu"], dev["A_down"],
                        dev["B_down"], ws, y, stream)


def test_two_streams_two_workspaces():
    import lora_moe_amd as lm
    a = synth.Workload("stream-a", T=96, H=512, I=384, E=8, topk=2, L=4, r=16,
                       lora_mode="uniform_with_none", seed=11)
    b = synth.Workload("stream-b", T=300, H=256, I=512, E=16, topk=4, L=6, r=32,
                       lora_mode="uniform_with_none", seed=12)
    jobs = []
    for wl, bm in ((a, 16), (b, 128)):
        dev = to_device(synth.make_inputs(wl))
        shape = lm.make_shape(wl.T, wl.H, wl.I, wl.E, wl.topk, wl.L, wl.r, bm, wl.scale)
        ws = lm.alloc_workspace(shape)
        y = torch.empty((wl.T, wl.H), dtype=torch.bfloat16, device="cuda")
        jobs.append((wl, bm, dev, ws, y))
    # alone, one after the other on the current stream
    alone = []
    for wl, bm, dev, ws, y in jobs:
        run(lm, wl, dev, ws, y, torch.cuda.current_stream(), bm)
        torch.cuda.synchronize()
        alone.append(y.float().cpu().numpy())
    # together: both streams wait for the current one, then run interleaved
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    for s in streams:
        s.wait_stream(torch.cuda.current_stream())
    for rep in range(3):
        for (wl, bm, dev, ws, y), s in zip(jobs, streams):
            y.zero_()
        torch.cuda.synchronize()
        for _ in range(2):
            for (wl, bm, dev, ws, y), s in zip(jobs, streams):
                run(lm, wl, dev, ws, y, s, bm)
        torch.cuda.synchronize()
        for i, (wl, bm, dev, ws, y) in enumerate(jobs):
            got = y.float().cpu().numpy()
            d = float(np.max(np.abs(got - alone[i])))
            log(f"streams rep {rep} {wl.name}: max |together - alone| {d:.3e}")
            # the split-K shrink adds with atomics: equal up to fp32 ordering
            assert np.allclose(got, alone[i], rtol=1e-2, atol=1e-2)
