"""Seeded random layer shapes and kernel configurations against the fp64
oracle (needs an MI355X).

Sizes, ranks, adapter counts, adapter-id mixes, routing skew, block_m and
every kernel knob are drawn together, so that combinations no targeted test
names (an expand as K stages on a 192-row tile beside a K remainder, 70
adapters on the thin ring, a single expert at block_m 256, ...) still meet
the tolerance |gpu - ref| <= 1e-2 + 1e-2*|ref|, with and without adapters.
The shapes are small: the oracle takes milliseconds per case."""
import numpy as np
import pytest

import synth
from gpu_common import compare, compare_delta, log, oracle_tokens, run_gpu, to_device

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

N_CASES = 128


def draw(i):
    """Case i: a Workload, its block_m and kernel knobs (all valid for the ABI)."""
    rng = np.random.default_rng(1000 + i)
    E = int(rng.integers(1, 17))
    k = int(rng.integers(1, min(E, 4) + 1))
    T = int(rng.integers(1, 300))
    H = int(rng.integers(1, 80)) * 8
    I = int(rng.integers(1, 80)) * 8
    L = int(rng.choice([1, 2, 3, 8, 31, 64, 65, 70]))
    r = int(rng.integers(1, 17)) * 8
    bm = int(rng.choice([0, 16, 32, 64, 128, 192, 256]))
    mode = str(rng.choice(["uniform", "uniform_with_none", "zipf", "none_fraction"]))
    zb = [d for d in (0, 1, 2, 4) if d == 0 or (r % d == 0 and (r // d) % 8 == 0)]
    knobs = {"expand_mode": int(rng.integers(0, 3)), "tile_order": int(rng.integers(0, 3)),
             "shrink_splits": int(rng.choice([0, 0, 1, 2, 4, 16])), "shrink_zblocks": int(rng.choice(zb)),
             "down_splits": int(rng.choice([0, 0, 1, 3]))}
    wl = synth.Workload(f"random-{i}", T=T, H=H, I=I, E=E, topk=k, L=L, r=r, lora_mode=mode,
                        none_fraction=0.2 if mode == "none_fraction" else 0.0,
                        bias_std=float(rng.choice([0.0, 2.0])), seed=2000 + i)
    return wl, bm, knobs


@pytest.fixture(scope="module", autouse=True)
def need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import lora_moe_amd as lm
    lm.load_library()


@pytest.mark.parametrize("i", range(N_CASES))
def test_random_shape(i):
    import lora_moe_amd as lm
    wl, bm, knobs = draw(i)
    shape = lm.make_shape(wl.T, wl.H, wl.I, wl.E, wl.topk, wl.L, wl.r, bm, wl.scale, **knobs)
    assert lm.moe_lora_workspace_bytes(shape) > 0, (wl, bm, knobs)
    what = (f"case {i}: T={wl.T} H={wl.H} I={wl.I} E={wl.E} k={wl.topk} L={wl.L} r={wl.r} "
            f"{wl.lora_mode} bias={wl.bias_std} bm={bm} {knobs}")
    log(what)
    inp = synth.make_inputs(wl)
    dev = to_device(inp)
    y, shape, ws = run_gpu(dev, wl, bm, knobs=knobs)
    assert lm.moe_lora_device_errors(shape, ws) == 0, what
    ref = oracle_tokens(inp, None)
    compare(y, ref, what)
    if (inp.lora_ids >= 0).any():
        none = torch.full_like(dev["lora_ids"], -1)
        y0, _, _ = run_gpu(dev, wl, bm, lora_ids=none, workspace=ws, knobs=knobs)
        ref0 = oracle_tokens(inp, None, lora_ids=np.full_like(inp.lora_ids, -1))
        compare(y0, ref0, what + " (no adapters)")
        compare_delta(y, y0, ref, ref0, what)


N_LARGE = 16


def draw_large(i):
    """Larger case i: thousands of tokens, so experts span several row tiles
    (weight reuse across tiles, the interleaved tile order's rounding, thin
    last tiles), checked on sampled tokens."""
    rng = np.random.default_rng(5000 + i)
    E = int(rng.integers(2, 33))
    k = int(rng.integers(1, min(E, 8) + 1))
    T = int(rng.integers(1000, 8193))
    H = int(rng.integers(8, 65)) * 8
    I = int(rng.integers(8, 65)) * 8
    L = int(rng.choice([4, 8, 16]))
    r = int(rng.choice([16, 32, 64, 128]))
    bm = int(rng.choice([0, 64, 128, 192, 256]))
    mode = str(rng.choice(["uniform", "uniform_with_none", "zipf", "none_fraction"]))
    knobs = {"expand_mode": int(rng.integers(0, 3)), "tile_order": int(rng.integers(0, 3))}
    wl = synth.Workload(f"random-large-{i}", T=T, H=H, I=I, E=E, topk=k, L=L, r=r, lora_mode=mode,
                        none_fraction=0.2 if mode == "none_fraction" else 0.0,
                        bias_std=float(rng.choice([0.0, 1.0, 2.0])), seed=6000 + i)
    return wl, bm, knobs


@pytest.mark.parametrize("i", range(N_LARGE))
def test_random_large_shape(i):
    import lora_moe_amd as lm
    from gpu_common import sample_tokens
    wl, bm, knobs = draw_large(i)
    shape = lm.make_shape(wl.T, wl.H, wl.I, wl.E, wl.topk, wl.L, wl.r, bm, wl.scale, **knobs)
    assert lm.moe_lora_workspace_bytes(shape) > 0, (wl, bm, knobs)
    what = (f"large case {i}: T={wl.T} H={wl.H} I={wl.I} E={wl.E} k={wl.topk} L={wl.L} r={wl.r} "
            f"{wl.lora_mode} bias={wl.bias_std} bm={lm.moe_lora_resolve_block_m(shape)} {knobs}")
    log(what)
    inp = synth.make_inputs(wl, touched_only=True)
    dev = to_device(inp)
    y, shape, ws = run_gpu(dev, wl, bm, knobs=knobs)
    assert lm.moe_lora_device_errors(shape, ws) == 0, what
    toks = sample_tokens(wl.T, 256, seed=i)
    ref = oracle_tokens(inp, toks)
    compare(y[toks], ref, what)
    none = torch.full_like(dev["lora_ids"], -1)
    y0, _, _ = run_gpu(dev, wl, bm, lora_ids=none, workspace=ws, knobs=knobs)
    ref0 = oracle_tokens(inp, toks, lora_ids=np.full_like(inp.lora_ids, -1))
    compare(y0[toks], ref0, what + " (no adapters)")
    if (inp.lora_ids[toks] >= 0).any():
        compare_delta(y[toks], y0[toks], ref, ref0, what)


N_DENSE = 16


def draw_dense(i):
    """Dense case i: one expert and at most 32 pairs (one row tile), where
    the gate_up spreads its ceil(I / 8) column groups evenly over the
    workgroups; I up to 6000 gives 1 to 3 groups per workgroup, ragged."""
    rng = np.random.default_rng(13000 + i)
    k = 1
    T = int(rng.integers(1, 33))
    H = int(rng.integers(1, 65)) * 8
    I = int(rng.integers(1, 751)) * 8
    L = int(rng.choice([1, 3, 8]))
    r = int(rng.choice([8, 16, 32, 64]))
    bm = int(rng.choice([0, 32]))
    mode = str(rng.choice(["uniform", "uniform_with_none"]))
    wl = synth.Workload(f"random-dense-{i}", T=T, H=H, I=I, E=1, topk=k, L=L, r=r, lora_mode=mode,
                        seed=14000 + i)
    return wl, bm


@pytest.mark.parametrize("i", range(N_DENSE))
def test_random_dense(i):
    import lora_moe_amd as lm
    wl, bm = draw_dense(i)
    what = f"dense case {i}: T={wl.T} H={wl.H} I={wl.I} L={wl.L} r={wl.r} {wl.lora_mode} bm={bm}"
    log(what)
    inp = synth.make_inputs(wl)
    dev = to_device(inp)
    y, shape, ws = run_gpu(dev, wl, bm)
    assert lm.moe_lora_device_errors(shape, ws) == 0, what
    ref = oracle_tokens(inp, None)
    compare(y, ref, what)


N_ALIGN = 64


def draw_align(i):
    """Align case i: sizes on both sides of the single-workgroup path's 1024
    pairs, skewed routing, duplicate experts in a token and invalid ids."""
    rng = np.random.default_rng(9000 + i)
    E = int(rng.integers(1, 301))
    L = int(rng.integers(1, min(61, 14336 // E)))
    k = int(rng.integers(1, min(E, 8) + 1))
    T = int(rng.choice([int(rng.integers(1, 129)), int(rng.integers(129, 6001))]))
    bm = int(rng.choice([16, 32, 64, 128, 192, 256]))
    hot = rng.random() < 0.5
    ids = rng.integers(0, E, (T, k))
    if hot:  # most pairs on one expert
        ids = np.where(rng.random((T, k)) < 0.6, int(rng.integers(0, E)), ids)
    bad = rng.random((T, k)) < 0.02
    ids = np.where(bad, rng.choice([-1, E, E + 7, -100], (T, k)), ids).astype(np.int32)
    lids = rng.integers(-1, L, T)
    lids = np.where(rng.random(T) < 0.02, rng.choice([L, -2, 999], T), lids).astype(np.int32)
    return T, k, E, L, bm, ids, lids


@pytest.mark.parametrize("i", range(N_ALIGN))
def test_random_align(i):
    from test_gpu_parity import check_align_exact
    T, k, E, L, bm, ids, lids = draw_align(i)
    check_align_exact(T, k, E, L, bm, ids, lids, f"random align {i}")


N_ROUTE = 48


def draw_route(i):
    """Router case i: expert counts on both sides of the router's 512-expert
    path, k up to 64, ties, skewed biases and scattered non-finite logits."""
    rng = np.random.default_rng(11000 + i)
    E = int(rng.choice([int(rng.integers(1, 513)), int(rng.integers(513, 1025))]))
    k = int(rng.integers(1, min(E, 64) + 1))
    T = int(rng.integers(1, 400))
    key = synth.stream_key(12000 + i, 0, T, E)
    if rng.random() < 0.3:  # a coarse grid: many equal logits per token
        lg = np.floor(synth.uniform(key, T * E) * 4.0) - 2.0
    else:
        lg = synth.normal(key, T * E) + rng.choice([0.0, 2.0]) * np.tile(synth.normal(
            synth.stream_key(12000 + i, 1, T, E), E), T)
    lg = np.asarray(lg, np.float64).reshape(T, E).astype(np.float32)
    if rng.random() < 0.3:
        bad = rng.random((T, E)) < 0.05
        lg = np.where(bad, rng.choice([np.nan, np.inf, -np.inf], (T, E)).astype(np.float32), lg)
        for t in rng.integers(0, T, 3):  # rows with fewer finite logits than k: -1 slots
            keep = rng.permutation(E)[:int(rng.integers(0, k))]
            row = np.full(E, rng.choice([np.nan, -np.inf]), np.float32)
            row[keep] = lg[t, keep]
            lg[t] = row
    L = int(rng.integers(1, 9))
    lids = rng.integers(-1, L, T).astype(np.int32)
    bm = int(rng.choice([16, 32, 64, 128, 256]))
    return np.ascontiguousarray(lg), k, L, lids, bm


@pytest.mark.parametrize("i", range(N_ROUTE))
def test_random_route(i):
    """The router alone and the fused router + align: ids bit-exact and
    weights within 1e-6 of the fp64 reference, the align's outputs bit-exact
    against the reference align on the reference ids."""
    import lora_moe_amd as lm
    import oracle
    from gpu_common import gpu_views
    lg, k, L, lids, bm = draw_route(i)
    T, E = lg.shape
    what = f"random route {i}: T={T} E={E} k={k} L={L} bm={bm}"
    log(what)
    o = oracle.Oracle()
    rids, rw = o.route(lg, k)
    shape = lm.make_shape(T, 64, 64, E, k, L, 8, bm)
    ids = torch.empty((T, k), dtype=torch.int32, device="cuda")
    w = torch.empty((T, k), dtype=torch.float32, device="cuda")
    dlg = torch.from_numpy(lg).cuda()
    lm.moe_lora_route(shape, dlg, ids, w)
    torch.cuda.synchronize()
    assert np.array_equal(ids.cpu().numpy(), rids), what
    wg = w.cpu().numpy()
    assert np.all(np.isfinite(wg)) and float(np.max(np.abs(wg - rw))) <= 1e-6, what
    ws = lm.alloc_workspace(shape)
    ids.fill_(-7)
    w.zero_()
    lm.moe_lora_route_align(shape, dlg, torch.from_numpy(lids).cuda(), ids, w, ws)
    torch.cuda.synchronize()
    assert np.array_equal(ids.cpu().numpy(), rids), what + " (fused)"
    assert float(np.max(np.abs(w.cpu().numpy() - rw))) <= 1e-6, what + " (fused)"
    got = gpu_views(shape, ws)
    want = o.align(T, k, E, L, got["block_m"], rids, lids, got["cap_rows"], got["cap_blocks"])
    for name in ("sorted_ids", "expert_off", "seg_start", "seg_cnt", "block_expert", "pos_of_pair"):
        assert np.array_equal(got[name], want[name]), f"{what}: {name} differs"
    assert got["num_padded"] == want["num_padded"] and got["err_count"] == want["err_count"], what
