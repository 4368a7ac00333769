"""The layer at the block_m the shipped tile-configuration table picks
matches the fp64 reference, for a shape in the table's range but not in it."""
import pytest

import synth
from test_gpu_parity import full_check

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("n", [1])
def test_layer_at_tuned_block_m(n):
    import lora_moe_amd as lm
    table = lm.load_tuning()
    wl = synth.WORKLOADS[n]
    shape = lm.make_shape(wl.T, wl.H, wl.I, wl.E, wl.topk, wl.L, wl.r, 0, wl.scale, tuning=table)
    assert shape.block_m in (16, 32, 64, 128, 192, 256)
    full_check(synth.make_inputs(wl), shape.block_m, f"workload {n} at tuned block_m {shape.block_m}")


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
