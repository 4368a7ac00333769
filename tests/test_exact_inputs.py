"""The small-integer inputs of the bit-exact GPU test (exact_inputs.py) do
what that test assumes: the fp64 reference's output lies within the SiLU's
rounding of multiples of 16 that bf16 represents exactly, and most of it is
non-zero (CPU only)."""
import numpy as np
import pytest

import exact_inputs
import oracle
import pins


@pytest.fixture(scope="module")
def orc():
    oracle.build(force=False)
    return oracle.Oracle()


@pytest.mark.parametrize("shape", sorted(exact_inputs.SHAPES))
def test_exact_inputs_premise(orc, shape):
    inp = exact_inputs.make(shape=shape)
    x = pins.f64(inp.x)
    assert np.all(x[:, 0] == exact_inputs.GATE)
    assert np.all(np.abs(x[:, 1:]) <= 1)
    for lids in (None, np.full_like(inp.lora_ids, -1)):
        y = pins.run(orc, inp) if lids is None else pins.run(orc, inp, lora_ids=lids)
        ye = exact_inputs.exact(y)
        assert np.max(np.abs(y - ye)) < 1e-9              # multiples of 16 up to the SiLU's rounding
        assert np.array_equal(exact_inputs.bf16_round(ye), ye)  # and bf16 holds them exactly
        assert np.mean(ye != 0) > 0.8
    # the adapters change the output (the exact comparison covers the LoRA path)
    y0 = pins.run(orc, inp, lora_ids=np.full_like(inp.lora_ids, -1))
    assert np.mean(pins.run(orc, inp) != y0) > 0.5
