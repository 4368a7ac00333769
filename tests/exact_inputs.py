"""Small-integer layer inputs whose every intermediate is exact on the GPU.

With integer bf16 inputs and sparse {-1, 0, 1} weights, every sum the layer
forms is an integer well inside fp32's 24-bit range, so the GPU's result does
not depend on summation order, K splits or atomics, and can be compared with
the fp64 reference bit for bit.  Two choices make the rest exact:

  * the gate half of W_gu picks x[:, 0] = 32 (and B_gu's gate rows are zero),
    so every gate value is 32 and silu(32) = 32 / (1 + e^-32) rounds to 32 in
    fp32; h = silu(gate) * up = 32 * up is then exact in bf16;
  * both top-k weights are 1/2, so y = (d1 + d2) / 2 with d a multiple of 32
    is exact in bf16 while its integer part needs at most 8 significant bits.

Only the SiLU keeps the fp64 reference off these values (by a relative
1e-14); `exact` takes its output back to them.  The construction
is checked on the CPU (test_exact_inputs.py) before the GPU test relies on it.
"""
from __future__ import annotations

from dataclasses import replace

import numpy as np

import synth

# Tiny routing (8 experts, top-2, 4 adapters and the no-adapter id) at a K
# deep enough for split-K shrinks: H = 1024 gives the gate_up shrink 16 K
# steps, I = 512 the down shrink 8.
EXACT_WL = replace(synth.WORKLOADS[1], name="exact-int", H=1024, I=512, r=16)
GATE = 32.0


def _sparse_pm1(rng, shape, per_row):
    """{-1, 0, 1} matrix (last axis = row) with `per_row` nonzeros per row."""
    out = np.zeros(shape, dtype=np.float32)
    flat = out.reshape(-1, shape[-1])
    for row in flat:
        idx = rng.choice(shape[-1], size=per_row, replace=False)
        row[idx] = rng.choice([-1.0, 1.0], size=per_row)
    return out


# shapes of the bit-exact test: K multiple of 64 and rank 16; then K with a
# remainder (1000 = 15*64 + 40, 520 = 8*64 + 8) and a rank that is not a
# multiple of 16 (24), which exercise the masked K tails and rank columns;
# rank 64, where the tiled GEMMs can run the expand as extra K stages
SHAPES = {"even": dict(H=1024, I=512, r=16), "ragged": dict(H=1000, I=520, r=24),
          "rank64": dict(H=1024, I=512, r=64)}


def make(seed: int = 5, shape: str = "even") -> synth.Inputs:
    """The workload's routing and adapter ids, with integer data and weights."""
    wl = replace(EXACT_WL, **SHAPES[shape])
    base = synth.make_inputs(wl)
    rng = np.random.default_rng(seed)
    T, H, I, E, L, r = wl.T, wl.H, wl.I, wl.E, wl.L, wl.r
    x = rng.choice([-1.0, 0.0, 1.0], size=(T, H)).astype(np.float32)
    x[:, 0] = GATE
    W_gu = np.zeros((E, 2 * I, H), np.float32)
    W_gu[:, :I, 0] = 1.0                                 # gate = x[:, 0]
    W_gu[:, I:, 1:] = _sparse_pm1(rng, (E, I, H - 1), 3)  # up: |up| <= 3
    A_gu = np.zeros((L, E, r, H), np.float32)
    A_gu[..., 1:] = _sparse_pm1(rng, (L, E, r, H - 1), 3)  # |z_gu| <= 3
    B_gu = np.zeros((L, E, 2 * I, r), np.float32)
    B_gu[:, :, I:, :] = _sparse_pm1(rng, (L, E, I, r), 1)  # up LoRA: |.| <= 3
    W_down = _sparse_pm1(rng, (E, H, I), 2)                # d / 32: |.| <= 12
    A_down = _sparse_pm1(rng, (L, E, r, I), 2)             # z_d / 32: |.| <= 12
    B_down = _sparse_pm1(rng, (L, E, H, r), 1)             # LoRA d / 32: |.| <= 12
    w = np.full(base.topk_weights.shape, 0.5, np.float32)
    b = synth.to_bf16
    return synth.Inputs(replace(wl, scale=1.0), x=b(x), topk_ids=base.topk_ids, topk_weights=w,
                        lora_ids=base.lora_ids, W_gu=b(W_gu), W_down=b(W_down), A_gu=b(A_gu),
                        B_gu=b(B_gu), A_down=b(A_down), B_down=b(B_down))


# d is a multiple of 32 (h = 32 * up, integer weights) and y = (d1 + d2) / 2
STEP = 16.0


def exact(y: np.ndarray) -> np.ndarray:
    """The exact layer output from the fp64 reference's: its nearest multiple
    of STEP (the reference is off only by the SiLU's 1e-14 relative, which
    leaves residues of ~1e-15 where the exact output is 0)."""
    return np.round(np.asarray(y, np.float64) / STEP) * STEP


def bf16_round(y: np.ndarray) -> np.ndarray:
    """fp64 values -> the nearest bf16 values (through fp32), as fp64."""
    return synth.bf16_to_f64(synth.to_bf16(np.asarray(y, np.float64).astype(np.float32)))
