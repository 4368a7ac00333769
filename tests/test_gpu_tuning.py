"""The layer at the configuration the shipped tuning table picks matches the
fp64 reference: for a shape near a table entry but not in it, for a shape
far from every entry (the pick leaves the library's own choice), and at full
size for every entry whose stored knobs differ from the library's own
choice."""
import json

import numpy as np
import pytest

import synth
from test_gpu_parity import full_check

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("n,T,near", [(3, 192, True), (1, None, False)])
def test_layer_at_tuned_block_m(n, T, near):
    """GPT-OSS-like at 192 tokens (24 rows per expert against the entry's 32)
    takes that entry's block_m; the tiny shape is beyond the pick's distance
    and keeps block_m 0, which the library resolves itself."""
    import lora_moe_amd as lm
    table = lm.load_tuning()
    inp = synth.make_inputs(n, T=T)
    wl = inp.wl
    shape = lm.make_shape(wl.T, wl.H, wl.I, wl.E, wl.topk, wl.L, wl.r, 0, wl.scale, tuning=table)
    if near:
        entries = json.load(open(lm.TUNING_PATH))["entries"]
        entry = next(e for e in entries if e["workload"] == synth.WORKLOADS[n].name)
        assert shape.block_m == entry["block_m"]
    else:
        assert shape.block_m == 0
    bm = lm.moe_lora_resolve_block_m(shape)
    assert bm in (16, 32, 64, 128, 192, 256)
    full_check(inp, shape.block_m, f"workload {n} T={wl.T} at tuned block_m {bm}")


def test_tune_sweep_writes_a_valid_table(tmp_path):
    """The offline sweep runs end to end on the small workload and writes a
    table that the pick reads back to its own best block_m."""
    import json
    import lora_moe_amd as lm
    from lora_moe_amd import tune
    out = tmp_path / "table.json"
    assert tune.main(["--workloads", "1", "--iters", "3", "--warmup", "1", "--out", str(out)]) == 0
    doc = json.loads(out.read_text())
    (e,) = doc["entries"]
    assert e["workload"] == "tiny" and e["block_m"] in (16, 32, 64, 128, 192, 256)
    assert min(e["ms"], key=e["ms"].get) == str(e["block_m"])
    wl = synth.WORKLOADS[1]
    shape = lm.make_shape(wl.T, wl.H, wl.I, wl.E, wl.topk, wl.L, wl.r, 0, wl.scale,
                          tuning=lm.load_tuning(str(out)))
    assert shape.block_m == e["block_m"]


def tuned_entries():
    import lora_moe_amd as lm
    doc = json.load(open(lm.TUNING_PATH))
    return [e["workload"] for e in doc["entries"] if any(e.get(k, 0) for k in lm.KNOBS)]


@pytest.mark.parametrize("name", tuned_entries())
def test_full_size_at_tuned_configuration(name):
    """A shape whose tuned knobs beat the built-in choice in the sweep, run at
    that configuration at full size against the reference (every token)."""
    import torch

    import lora_moe_amd as lm
    from gpu_common import compare, compare_delta, log, oracle_tokens
    wl = next(w for w in synth.WORKLOADS.values() if w.name == name)
    shape = lm.make_shape(wl.T, wl.H, wl.I, wl.E, wl.topk, wl.L, wl.r, 0, wl.scale, tuning=lm.load_tuning())
    knobs = {k: getattr(shape, k) for k in lm.KNOBS}
    assert any(knobs.values())
    log(f"{name} at the tuned configuration: block_m {shape.block_m} {knobs}")
    dev, inp = synth.device_inputs(wl, touched_only=True, keep_host=True)

    def run(lids):
        ws = lm.alloc_workspace(shape)
        y = torch.empty((wl.T, wl.H), dtype=torch.bfloat16, device="cuda")
        lm.moe_lora_align(shape, dev["topk_ids"], lids, ws)
        lm.moe_lora_forward(shape, dev["x"], dev["topk_ids"], dev["topk_weights"], lids, dev["W_gu"],
                            dev["W_down"], dev["A_gu"], dev["B_gu"], dev["A_down"], dev["B_down"], ws, y)
        torch.cuda.synchronize()
        return y.float().cpu().numpy().astype(np.float64)

    y = run(dev["lora_ids"])
    ref = oracle_tokens(inp, None)
    compare(y, ref, f"{name} tuned")
    y0 = run(torch.full_like(dev["lora_ids"], -1))
    ref0 = oracle_tokens(inp, None, lora_ids=np.full_like(inp.lora_ids, -1))
    compare(y0, ref0, f"{name} tuned, no adapters")
    compare_delta(y, y0, ref, ref0, f"{name} tuned")
