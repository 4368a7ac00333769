"""The seeded input generator (CPU only): determinism, distribution, routing."""
import numpy as np

import synth


def test_normal_moments_and_determinism():
    k = synth.stream_key(0, 4, 1, 0)
    a = synth.normal(k, 400_000)
    assert abs(a.mean()) < 0.01 and abs(a.std() - 1.0) < 0.01
    np.testing.assert_array_equal(a, synth.normal(k, 400_000))
    b = synth.normal(synth.stream_key(0, 4, 2, 0), 1000)
    assert not np.allclose(a[:1000], b)
    # a prefix of a longer stream is the shorter stream
    np.testing.assert_array_equal(synth.normal(k, 999), a[:999])


def test_bf16_rounding_is_rne():
    rng = np.random.default_rng(1)
    f = rng.standard_normal(100_000).astype(np.float32)
    f[:4] = [1.00390625, 1.01171875, -1.00390625, 0.0]  # ties: round to even
    u = f.view(np.uint32).astype(np.uint64)
    want = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)
    np.testing.assert_array_equal(synth.to_bf16(f), want)
    assert synth.bf16_to_f64(synth.to_bf16([1.00390625]))[0] == 1.0
    assert synth.bf16_to_f64(synth.to_bf16([1.01171875]))[0] == 1.015625


def test_workload_inputs_shapes_and_router():
    inp = synth.make_inputs(1)
    wl = inp.wl
    assert inp.x.shape == (wl.T, wl.H) and inp.W_gu.shape == (wl.E, 2 * wl.I, wl.H)
    assert inp.B_down.shape == (wl.L, wl.E, wl.H, wl.r)
    np.testing.assert_allclose(inp.topk_weights.sum(1), 1.0, rtol=1e-6)
    assert np.all(np.diff(inp.topk_weights, axis=1) <= 0), "weights follow logit order"
    for row in inp.topk_ids:
        assert len(set(row.tolist())) == wl.topk
    assert inp.lora_ids.min() >= -1 and inp.lora_ids.max() < wl.L
    w = synth.bf16_to_f64(inp.W_gu)
    assert abs(w.std() - 0.02) < 0.001


def test_router_ties_go_to_lower_index():
    ids, w = synth.route(np.array([[1.0, 3.0, 3.0, 0.0]]), 2)
    assert ids.tolist() == [[1, 2]]
    np.testing.assert_allclose(w, [[0.5, 0.5]])


def test_adapter_id_modes():
    wl4 = synth.WORKLOADS[4]
    ids = synth.adapter_ids(wl4)
    assert (ids == -1).sum() == int(0.2 * wl4.T)
    ids3 = synth.adapter_ids(synth.WORKLOADS[3])
    counts = np.bincount(ids3, minlength=16)
    assert counts[0] > counts[1] > counts[4] and ids3.min() >= 0
