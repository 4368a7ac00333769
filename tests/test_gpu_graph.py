"""The layer captured in a HIP graph (launch gaps removed for decode): the
eager run and every replay, with eager work and synchronisations between
replays, match the fp64 reference."""
import numpy as np
import pytest
import torch

import synth
from gpu_common import compare, log, oracle_tokens, to_device

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("n,routed", [(1, False), (1, True), (2, False)])
def test_graph_replays_match_reference(n, routed):
    import lora_moe_amd as lm
    wl = synth.WORKLOADS[n]
    if n == 1:
        inp = synth.make_inputs(wl)
        dev = to_device(inp)
    else:
        dev, inp = synth.device_inputs(wl, touched_only=True, keep_host=True)
    shape = lm.make_shape(wl.T, wl.H, wl.I, wl.E, wl.topk, wl.L, wl.r, 0, wl.scale)
    ws = lm.alloc_workspace(shape)
    y = torch.empty((wl.T, wl.H), dtype=torch.bfloat16, device="cuda")
    ids = torch.empty_like(dev["topk_ids"])
    w = torch.empty_like(dev["topk_weights"])
    logits = torch.full((wl.T, wl.E), -1e30, dtype=torch.float32, device="cuda")
    logits.scatter_(1, dev["topk_ids"].long(), torch.log(dev["topk_weights"].clamp_min(1e-30)))

    def step(stream):
        if routed:
            lm.moe_lora_route_align(shape, logits, dev["lora_ids"], ids, w, ws, stream)
            tid, tw = ids, w
        else:
            lm.moe_lora_align(shape, dev["topk_ids"], dev["lora_ids"], ws, stream)
            tid, tw = dev["topk_ids"], dev["topk_weights"]
        lm.moe_lora_forward(shape, dev["x"], tid, tw, dev["lora_ids"], dev["W_gu"], dev["W_down"],
                            dev["A_gu"], dev["B_gu"], dev["A_down"], dev["B_down"], ws, y, stream)

    step(torch.cuda.current_stream())  # eager (also sets kernel attributes before capture)
    torch.cuda.synchronize()
    if routed:  # the reference layer on the reference router's choice
        import oracle
        rids, rw = oracle.Oracle().route(logits.cpu().numpy(), wl.topk)
        assert np.array_equal(ids.cpu().numpy(), rids)
        inp.topk_ids[:] = rids
        inp.topk_weights[:] = rw.astype(np.float32)
    ref = oracle_tokens(inp, None)
    compare(y.float().cpu().numpy().astype(np.float64), ref, f"workload {n} routed={routed} eager")

    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            step(s)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    for rep in range(4):
        y.zero_()  # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        y_g = y.float().cpu().numpy().astype(np.float64)
        log(f"workload {n} routed={routed} replay {rep}")
        compare(y_g, ref, f"workload {n} routed={routed} replay {rep}")
