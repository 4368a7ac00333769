"""Parity of the HIP path with the fp64 CPU reference (needs an MI355X).

Align outputs are compared bit-exactly; layer outputs element-wise within
|gpu - ref| <= 1e-2 + 1e-2*|ref| (bf16 inputs, fp32 accumulation), plus a
relative-L2 bound and an adapter-delta check (the element-wise tolerance alone
cannot see a dropped adapter on the small shapes)."""
from dataclasses import replace

import numpy as np
import pytest

import synth
from gpu_common import (compare, compare_delta, gpu_views, log, oracle_tokens, run_gpu, sample_tokens,
                        shape_for, to_device)

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module", autouse=True)
def need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import lora_moe_amd as lm
    lm.load_library()


# ------------------------------------------------------------------ align

def align_gpu(T, k, E, L, bm, ids, lids):
    import lora_moe_amd as lm
    shape = lm.make_shape(T, 64, 64, E, k, L, 8, bm)
    ws = lm.alloc_workspace(shape)
    lm.moe_lora_align(shape, torch.from_numpy(np.ascontiguousarray(ids, np.int32)).cuda(),
                      torch.from_numpy(np.ascontiguousarray(lids, np.int32)).cuda(), ws)
    torch.cuda.synchronize()
    return gpu_views(shape, ws), lm.moe_lora_device_errors(shape, ws)


def check_align_exact(T, k, E, L, bm, ids, lids, what):
    import oracle
    log(f"align {what}: T={T} k={k} E={E} L={L} bm={bm}")
    got, errs = align_gpu(T, k, E, L, bm, ids, lids)
    want = oracle.Oracle().align(T, k, E, L, bm, ids, lids, got["cap_rows"], got["cap_blocks"])
    assert got["num_padded"] == want["num_padded"], what
    assert got["err_count"] == want["err_count"] == errs, what
    for n in ("sorted_ids", "expert_off", "seg_start", "seg_cnt", "block_expert", "pos_of_pair"):
        np.testing.assert_array_equal(got[n], want[n], err_msg=f"{what}: {n}")


@pytest.mark.parametrize("n", [1, 2, 3, 4, 5, 6])
@pytest.mark.parametrize("bm", [16, 64, 192, 256])
def test_align_bitexact_workloads(n, bm):
    wl = synth.WORKLOADS[n]
    ids, _ = synth.make_routing(wl)
    lids = synth.adapter_ids(wl)
    check_align_exact(wl.T, wl.topk, wl.E, wl.L, bm, ids, lids, f"workload {n}")


def test_align_adversarial():
    import pins
    for name, T, k, E, L, bm, ids, lids in pins.align_cases():
        if T == 0:
            continue
        for b in sorted({16, 32, 128} | ({bm} if bm in (16, 32, 64, 128, 192, 256) else set())):
            check_align_exact(T, k, E, L, b, ids, lids, f"{name} bm={b}")
    rng = np.random.default_rng(9)
    # many chunks, one hot expert, ragged P
    T, k, E, L = 3001, 3, 40, 5
    ids = np.where(rng.random((T, k)) < 0.7, 7, rng.integers(0, E, (T, k))).astype(np.int32)
    lids = rng.integers(-1, L, T).astype(np.int32)
    check_align_exact(T, k, E, L, 64, ids, lids, "hot expert, 18 chunks")
    check_align_exact(1, 1, 1, 1, 16, np.zeros((1, 1), np.int32), np.zeros(1, np.int32), "T=1")


def test_align_deterministic():
    wl = synth.WORKLOADS[4]
    ids, _ = synth.make_routing(wl)
    lids = synth.adapter_ids(wl)
    a, _ = align_gpu(wl.T, wl.topk, wl.E, wl.L, 64, ids, lids)
    b, _ = align_gpu(wl.T, wl.topk, wl.E, wl.L, 64, ids, lids)
    for n in ("sorted_ids", "pos_of_pair", "block_expert"):
        np.testing.assert_array_equal(a[n], b[n])


# ------------------------------------------------------------------ layer, small shapes

def full_check(inp, block_m=0, what="", scale=None, errors=0, knobs=None):
    import lora_moe_amd as lm
    if scale is not None:
        inp = synth.Inputs(replace(inp.wl, scale=scale), **{k: v for k, v in inp.arrays().items()})
    wl = inp.wl
    log(f"layer {what}: T={wl.T} H={wl.H} I={wl.I} E={wl.E} k={wl.topk} L={wl.L} r={wl.r} bm={block_m} {knobs or ''}")
    dev = to_device(inp)
    y, shape, ws = run_gpu(dev, wl, block_m, knobs=knobs)
    # the invalid ids the align met
    assert lm.moe_lora_device_errors(shape, ws) == errors, what
    ref = oracle_tokens(inp, None)
    compare(y, ref, what)
    if (inp.lora_ids >= 0).any():
        none = torch.full_like(dev["lora_ids"], -1)
        y0, _, _ = run_gpu(dev, wl, block_m, lora_ids=none, workspace=ws, knobs=knobs)
        ref0 = oracle_tokens(inp, None, lora_ids=np.full_like(inp.lora_ids, -1))
        compare(y0, ref0, what + " (no adapters)")
        compare_delta(y, y0, ref, ref0, what)
    return y, ref


@pytest.mark.parametrize("I", [1024, 1000])
@pytest.mark.parametrize("bm", [0, 32])
def test_dense_split_k(I, bm):
    """One expert (a dense multi-LoRA layer): the streaming down GEMM splits K
    (I / 128 splits here, the last one with the K remainder when I = 1000) and
    the combine adds the partial slabs."""
    import lora_moe_amd as lm
    wl = synth.Workload("dense", T=20, H=256, I=I, E=1, topk=1, L=3, r=16,
                        lora_mode="uniform_with_none")
    shape = lm.make_shape(wl.T, wl.H, wl.I, wl.E, wl.topk, wl.L, wl.r, bm, wl.scale)
    ws = lm.alloc_workspace(shape)
    assert lm.workspace_tensors(shape, ws)["d_splits"] == I // 128
    full_check(synth.make_inputs(wl), bm, f"dense I={I} bm={bm}")


@pytest.mark.parametrize("bm", [0, 16, 32, 64, 128, 192, 256])
def test_tiny_workload(bm):
    inp = synth.make_inputs(1)
    full_check(inp, bm, f"tiny bm={bm}")


def test_tiny_scale_and_seed():
    inp = synth.make_inputs(1, seed=3)
    full_check(inp, 0, "tiny seed 3 scale 0.5", scale=0.5)


@pytest.mark.parametrize("T,I", [(32, 25600), (32, 4104), (7, 200)])
def test_dense_balanced_gate_up(T, I):
    """One expert whose pairs fit one 32-row tile: the gate_up spreads its
    ceil(I / 8) column groups evenly over the workgroups (12-13 each at I =
    25600, 2-3 at 4104, one each at 200), the wavefronts past a workgroup's
    share idle."""
    wl = synth.Workload("dense-bal", T=T, H=512, I=I, E=1, topk=1, L=3, r=16,
                        lora_mode="uniform_with_none")
    full_check(synth.make_inputs(wl), 32, f"dense balanced T={T} I={I}")


@pytest.mark.parametrize("bm", [0, 64, 128, 192, 256])
@pytest.mark.parametrize("H,I,r", [(104, 104, 8), (104, 1000, 24), (1000, 104, 16), (2880, 2880, 64),
                                   (256, 512, 128), (64, 40, 8), (24, 16, 8)])
def test_ragged_tails(H, I, r, bm):
    """K and N tails (the pages' K = 100 vs BLOCK_SIZE_K = 64 example, here
    104 = 64 + 40) and every rank family, on both GEMM families (block_m 128
    selects the LDS-tiled one)."""
    wl = synth.Workload("tail", T=37, H=H, I=I, E=5, topk=2, L=3, r=r,
                        lora_mode="uniform_with_none")
    full_check(synth.make_inputs(wl), bm, f"tails H={H} I={I} r={r} bm={bm}")


def test_edge_cases():
    base = synth.Workload("edge", T=50, H=256, I=128, E=6, topk=3, L=3, r=16,
                          lora_mode="uniform_with_none")
    # every token without adapter
    inp = synth.make_inputs(replace(base, lora_mode="none"))
    full_check(inp, 0, "no adapters")
    # one token
    full_check(synth.make_inputs(replace(base, T=1)), 0, "T=1")
    # every token on the same three experts with the same adapter
    inp = synth.make_inputs(replace(base, lora_mode="uniform"))
    inp.topk_ids[:] = np.array([2, 4, 0], np.int32)
    inp.lora_ids[:] = 1
    full_check(inp, 16, "three hot buckets")
    # invalid expert and adapter ids are dropped / treated as none and counted
    inp = synth.make_inputs(base)
    inp.topk_ids[3, 1] = 99
    inp.topk_ids[7, 0] = -2
    inp.lora_ids[5] = 17
    inp.lora_ids[9] = -4
    y, ref = full_check(inp, 0, "invalid ids", errors=4)
    import lora_moe_amd as lm
    dev = to_device(inp)
    _, shape, ws = run_gpu(dev, inp.wl)
    assert lm.moe_lora_device_errors(shape, ws) == 4


@pytest.mark.parametrize("bm", [0, 32, 64, 128, 192, 256])
def test_routing_extremes(bm):
    """Every token to every expert (topk = E), and every token to one expert
    (several row tiles of one expert, the others untouched)."""
    base = synth.Workload("extreme", T=300, H=256, I=128, E=4, topk=4, L=3, r=16,
                          lora_mode="uniform_with_none")
    full_check(synth.make_inputs(base), bm, f"topk = E bm={bm}")
    one = replace(base, T=700, E=8, topk=1)
    inp = synth.make_inputs(one)
    inp.topk_ids[:] = 5
    inp.topk_weights[:] = 1.0
    full_check(inp, bm, f"one expert bm={bm}")


@pytest.mark.parametrize("H,I", [(256, 256), (264, 200)])
def test_thin_tiles(H, I):
    """block_m 256 with experts of exactly 1, 30, 64, 65, 200, 256, 300 and 513
    rows: row tiles with at most 64 real rows (an expert's only tile, or the
    last of 300 and 513) run on the tiled GEMM's thin ring when K is a
    multiple of 64 in both GEMMs (H = I = 256), and on the full ring
    otherwise (H = 264, I = 200); 65 and 200 rows and the full tiles always
    take the full ring."""
    counts = [1, 30, 64, 65, 200, 256, 300, 513]
    wl = synth.Workload("thin", T=sum(counts), H=H, I=I, E=8, topk=1, L=4, r=16,
                        lora_mode="uniform_with_none", seed=6)
    inp = synth.make_inputs(wl)
    ids = np.repeat(np.arange(len(counts), dtype=np.int32), counts)
    np.random.default_rng(6).shuffle(ids)
    inp.topk_ids[:, 0] = ids
    inp.topk_weights[:] = 1.0
    full_check(inp, 256, f"thin tiles H={H} I={I}")


@pytest.mark.parametrize("r,mode", [(16, 1), (64, 1), (64, 2)])
def test_thin_tiles_192(r, mode):
    """block_m 192 with experts of 1, 96, 97, 127, 128, 129, 160, 192, 300
    and 320 rows: tiles with at most 128 real rows (an expert's only tile,
    or the last of 300 and 320 with 108 and 128) run on the 192 x 256
    tile's thin ring of 128-row stages, the others on the full ring; rank 16
    runs the register expand inside the loop (whose item loads the thin loop
    issues before the stage's copies), rank 64 the register or the stage
    form."""
    counts = [1, 96, 97, 127, 128, 129, 160, 192, 300, 320]
    wl = synth.Workload("thin192", T=sum(counts), H=256, I=256, E=len(counts), topk=1, L=5, r=r,
                        lora_mode="uniform_with_none", seed=15)
    inp = synth.make_inputs(wl)
    ids = np.repeat(np.arange(len(counts), dtype=np.int32), counts)
    np.random.default_rng(15).shuffle(ids)
    inp.topk_ids[:, 0] = ids
    inp.topk_weights[:] = 1.0
    full_check(inp, 192, f"thin tiles 192 r={r} expand_mode={mode}", knobs=dict(expand_mode=mode))


def _expand_case(case):
    """Workloads for the two forms of the tiled GEMMs' expand: (inputs, block_m)."""
    if case == "thin":  # experts of 1 .. 513 rows at block_m 256, rank 64
        counts = [1, 30, 64, 65, 200, 256, 300, 513]
        wl = synth.Workload("expand-thin", T=sum(counts), H=256, I=256, E=8, topk=1, L=4, r=64,
                            lora_mode="uniform_with_none", seed=7)
        inp = synth.make_inputs(wl)
        ids = np.repeat(np.arange(len(counts), dtype=np.int32), counts)
        np.random.default_rng(7).shuffle(ids)
        inp.topk_ids[:, 0] = ids
        inp.topk_weights[:] = 1.0
        return inp, 256
    if case == "r128":  # two 64-rank stages per segment
        wl = synth.Workload("expand-r128", T=300, H=256, I=512, E=4, topk=2, L=5, r=128,
                            lora_mode="uniform_with_none", seed=8)
        return synth.make_inputs(wl), 192
    if case in ("L64", "L65"):  # one lane per adapter: 64 is the last the stage form takes
        wl = synth.Workload("expand-" + case, T=700, H=256, I=256, E=2, topk=1, L=int(case[1:]), r=64,
                            lora_mode="uniform_with_none", seed=9)
        return synth.make_inputs(wl), 256
    if case.startswith("rank"):  # ranks below 64 share a stage (8 / (r / 8) segments), 72 spills into a second
        wl = synth.Workload("expand-" + case, T=400, H=256, I=256, E=3, topk=2, L=9, r=int(case[4:]),
                            lora_mode="uniform_with_none", seed=11)
        return synth.make_inputs(wl), 128
    # gate_up K = 264 has a remainder (register expand), down K = 256 does not
    wl = synth.Workload("expand-uneven", T=200, H=264, I=256, E=4, topk=2, L=3, r=64,
                        lora_mode="uniform_with_none", seed=10)
    return synth.make_inputs(wl), 128


@pytest.mark.parametrize("mode", [1, 2])
@pytest.mark.parametrize("case", ["thin", "r128", "L64", "L65", "uneven", "rank8", "rank16", "rank24",
                                  "rank40", "rank72"])
def test_expand_forms(case, mode):
    """The tiled GEMMs' expand as extra K stages through the LDS ring
    (expand_mode 2, taken where L <= 64 and K is a multiple of 64) and from
    registers (expand_mode 1) both match the oracle: thin row tiles, 128 ranks
    (two stages per segment), 64 adapters with a segment each in a tile (64
    expand stages behind 4 K stages) and 65 (the register form runs), a
    gate_up K with a remainder beside a down K without one, and ranks that
    share a stage between segments (8, 16, 24 with two chunks unused, 40 with
    three) or leave a second stage nearly empty (72)."""
    inp, bm = _expand_case(case)
    full_check(inp, bm, f"expand {case}", knobs=dict(expand_mode=mode))


def test_expert_weights_past_2gb():
    """An expert whose gate_up weights take 2 GB (2I x H x 2 bytes = 2^31)
    cannot be addressed through the LDS-tiled GEMM's buffer resources; at
    block_m 256 its gate_up runs on the streaming kernel in 32-row tiles
    (the down GEMM, I >= 4096, takes h as hi + lo on the same kernel).
    3 GB of weights, four tokens."""
    wl = synth.Workload("big-w", T=4, H=16384, I=32768, E=1, topk=1, L=2, r=16,
                        lora_mode="uniform_with_none", seed=12)
    full_check(synth.make_inputs(wl), 256, "expert weights past 2 GB")


@pytest.mark.parametrize("mode", [1, 2])
@pytest.mark.parametrize("bm", [64, 128, 192, 256])
def test_expand_forms_exact(bm, mode):
    """Both expand forms at rank 64 give the exact small-integer layer bit for
    bit (at block_m 256 the tiny routing's tiles run on the thin ring)."""
    import lora_moe_amd as lm
    import exact_inputs
    inp = exact_inputs.make(shape="rank64")
    wl = inp.wl
    log(f"exact integers rank 64, bm={bm} expand_mode={mode}")
    dev = to_device(inp)
    y, shape, ws = run_gpu(dev, wl, bm, knobs=dict(expand_mode=mode))
    assert lm.moe_lora_device_errors(shape, ws) == 0
    want = exact_inputs.exact(oracle_tokens(inp, None))
    bad = np.argwhere(y != want)
    assert bad.size == 0, f"{len(bad)} outputs differ, first {bad[:3].tolist()}"


@pytest.mark.parametrize("T,E,L", [(200, 4, 100), (600, 64, 200)])
@pytest.mark.parametrize("bm", [0, 32, 64, 128, 192, 256])
def test_more_than_64_adapters(T, E, L, bm):
    """L > 64 adapters: the tiled expand scans adapter ids 64 at a time; the
    align's (expert, slot) table has E x (L + 1) buckets (12864 at E = 64,
    L = 200, with P = 1200 pairs: the multi-kernel align)."""
    wl = synth.Workload("many-adapters", T=T, H=256, I=384, E=E, topk=2, L=L, r=16,
                        lora_mode="uniform_with_none")
    full_check(synth.make_inputs(wl), bm, f"T={T} E={E} L={L} bm={bm}")


def test_shrink_stage_matches_reference():
    """z = x A for every adapter row, against the reference's shrink output."""
    import lora_moe_amd as lm
    import oracle
    inp = synth.make_inputs(1)
    wl = inp.wl
    dev = to_device(inp)
    _, shape, ws = run_gpu(dev, wl)
    t = lm.workspace_tensors(shape, ws)
    zg = t["z_gu"].cpu().numpy()
    pos = t["pos_of_pair"].cpu().numpy()
    o = oracle.Oracle()
    checked = 0
    for tok in range(wl.T):
        if inp.lora_ids[tok] < 0:
            continue
        for j in range(wl.topk):
            st = o.pair((wl.T, wl.H, wl.I, wl.E, wl.topk, wl.L, wl.r), inp.x, inp.topk_ids,
                        inp.lora_ids, inp.W_gu, inp.W_down, inp.A_gu, inp.B_gu, inp.A_down,
                        inp.B_down, tok, j, scale=wl.scale)
            got = zg[pos[tok * wl.topk + j]]
            np.testing.assert_allclose(got, st["zg"], rtol=1e-4, atol=1e-4)
            checked += 1
    assert checked > 20


@pytest.mark.parametrize("shape", ["even", "ragged"])
@pytest.mark.parametrize("bm", [0, 16, 32, 64, 128, 192, 256])
def test_exact_small_integer_layer(bm, shape):
    """Small-integer inputs make every intermediate exact (exact_inputs.py):
    the layer output must equal the exact values the fp64 reference gives
    (exact_inputs.exact) bit for bit, with and without adapters, in every GEMM family and through the
    split-K shrinks' atomics."""
    import lora_moe_amd as lm
    import exact_inputs
    inp = exact_inputs.make(shape=shape)
    wl = inp.wl
    log(f"exact integers ({shape}) bm={bm}: T={wl.T} H={wl.H} I={wl.I} E={wl.E} k={wl.topk} L={wl.L} r={wl.r}")
    dev = to_device(inp)
    y, shape, ws = run_gpu(dev, wl, bm)
    assert lm.moe_lora_device_errors(shape, ws) == 0
    want = exact_inputs.exact(oracle_tokens(inp, None))
    bad = np.argwhere(y != want)
    assert bad.size == 0, f"{len(bad)} outputs differ, first {bad[:3].tolist()}: {y[tuple(bad[0])]} vs {want[tuple(bad[0])]}"
    none = torch.full_like(dev["lora_ids"], -1)
    y0, _, _ = run_gpu(dev, wl, bm, lora_ids=none, workspace=ws)
    want0 = exact_inputs.exact(oracle_tokens(inp, None, lora_ids=np.full_like(inp.lora_ids, -1)))
    assert np.array_equal(y0, want0)
    assert not np.array_equal(y, y0)


# ------------------------------------------------------------------ full-size workloads

def full_size_tokens(n, wl, inp, shape, ws):
    """Tokens the reference checks at full size: every token of workloads 2,
    3, 4 and 6; for the DeepSeek-like one 256 seeded tokens plus the tokens
    of the hot expert's first and last row tiles and of every expert whose
    rows fit one tile (from the align outputs of the run under test)."""
    if n != 5:
        return np.arange(wl.T, dtype=np.int32)
    v = gpu_views(shape, ws)
    bm, P = v["block_m"], wl.T * wl.topk
    eoff, sorted_ids = v["expert_off"], v["sorted_ids"]
    counts = np.bincount(inp.topk_ids.reshape(-1), minlength=wl.E)
    hot = int(np.argmax(counts))
    pick = set(sample_tokens(wl.T, 256).tolist())
    first = sorted_ids[eoff[hot]:eoff[hot] + bm]
    last_tile = eoff[hot] + (counts[hot] - 1) // bm * bm
    last = sorted_ids[last_tile:eoff[hot + 1]]
    for rows in (first[:8], first[-8:], last[:8], last[last < P][-8:]):
        pick |= {int(p) // wl.topk for p in rows if p < P}
    single = [e for e in range(wl.E) if 0 < counts[e] <= bm]
    for e in single[:16]:
        pr = sorted_ids[eoff[e]]
        pick.add(int(pr) // wl.topk)
    log(f"workload 5: hot expert {hot} ({counts[hot]} rows, tiles {eoff[hot]}..{eoff[hot + 1]}), "
        f"{len(single)} single-tile experts, {len(pick)} tokens")
    return np.array(sorted(pick), dtype=np.int32)


@pytest.mark.parametrize("n", [2, 3, 4, 5, 6])
def test_workload_full_size(n):
    """The benchmarked launch configuration at full size against the
    reference: every token of workloads 2-4 and 6, a few hundred chosen
    tokens of the DeepSeek-like one (its reference costs seconds per hundred
    tokens); the stated tolerance everywhere."""
    import lora_moe_amd as lm
    wl = synth.WORKLOADS[n]
    log(f"workload {n} ({wl.name}): generating on device")
    dev, inp = synth.device_inputs(wl, touched_only=True, keep_host=True)
    y, shape, ws = run_gpu(dev, wl)
    assert lm.moe_lora_device_errors(shape, ws) == 0
    toks = full_size_tokens(n, wl, inp, shape, ws)
    ref = oracle_tokens(inp, toks)
    compare(y[toks], ref, f"workload {n}, {len(toks)} tokens")
    none = torch.full_like(dev["lora_ids"], -1)
    y0, _, _ = run_gpu(dev, wl, lora_ids=none, workspace=ws)
    ref0 = oracle_tokens(inp, toks, lora_ids=np.full_like(inp.lora_ids, -1))
    compare(y0[toks], ref0, f"workload {n} (no adapters)")
    compare_delta(y[toks], y0[toks], ref, ref0, f"workload {n}")
    assert np.all(np.isfinite(y))
    del dev, ws
    torch.cuda.empty_cache()


@pytest.mark.parametrize("bm", [0, 16, 32, 64, 128, 256])
def test_deep_intermediate_hi_lo(bm):
    """I >= 4096: h reaches the down GEMM as bf16 hi + lo (the streaming
    kernel, whatever block_m) -- the lo part is written and is the remainder
    of h, and the layer meets the stated tolerance."""
    import lora_moe_amd as lm
    wl = synth.Workload("deep", T=40, H=512, I=4104, E=3, topk=2, L=3, r=16,
                        lora_mode="uniform_with_none", seed=4)
    inp = synth.make_inputs(wl)
    full_check(inp, bm, f"deep I={wl.I} bm={bm}")
    dev = to_device(inp)
    _, shape, ws = run_gpu(dev, wl, bm)
    t = lm.workspace_tensors(shape, ws)
    assert t["h_lo"] is not None
    pos = t["pos_of_pair"].cpu().numpy()
    rows = pos[pos >= 0]
    hi = t["h"][torch.from_numpy(rows).cuda().long()].float()
    lo = t["h_lo"][torch.from_numpy(rows).cuda().long()].float()
    # lo is what rounding h to bf16 left: at most half an ulp of hi
    ulp = torch.where(hi != 0, hi.abs() * 2.0 ** -7, torch.full_like(hi, 2.0 ** -126))
    assert bool((lo.abs() <= 0.5 * ulp + 1e-30).all())
    assert float(lo.abs().max()) > 0


def test_forward_needs_its_own_align():
    """Each forward follows an align of its own (the align clears the split-K
    shrink accumulators): align + forward twice on one workspace gives the
    reference both times, at a decode shape whose shrinks split K."""
    import lora_moe_amd as lm
    wl = synth.Workload("forward-rule", T=16, H=2048, I=512, E=8, topk=2, L=4, r=16,
                        lora_mode="uniform_with_none", seed=8)
    inp = synth.make_inputs(wl)
    dev = to_device(inp)
    ref = oracle_tokens(inp, None)
    shape = shape_for(wl)
    ws = lm.alloc_workspace(shape)
    for rep in range(2):
        y, _, _ = run_gpu(dev, wl, workspace=ws)
        compare(y, ref, f"align + forward, call {rep}")


@pytest.mark.parametrize("bm,knobs", [
    (16, dict(shrink_splits=1)), (16, dict(shrink_splits=8, shrink_zblocks=2)), (32, dict(down_splits=3)),
    (64, dict(shrink_splits=4, tile_order=2)), (128, dict(shrink_zblocks=1, tile_order=2)),
    (192, dict(shrink_splits=2, shrink_zblocks=2, tile_order=1)), (256, dict(tile_order=1, shrink_splits=16)),
    (256, dict(tile_order=2))])
def test_kernel_knobs(bm, knobs):
    """Non-default kernel configurations (shrink K splits and z column blocks,
    down-GEMM K splits, tiled-GEMM workgroup order) give the same layer."""
    wl = synth.Workload("knobs", T=150, H=1024, I=512, E=6, topk=2, L=3, r=16,
                        lora_mode="uniform_with_none", seed=21)
    inp = synth.make_inputs(wl)
    import lora_moe_amd as lm
    shape = lm.make_shape(wl.T, wl.H, wl.I, wl.E, wl.topk, wl.L, wl.r, bm, wl.scale, **knobs)
    log(f"knobs bm={bm} {knobs}")
    dev = to_device(inp)
    ws = lm.alloc_workspace(shape)
    y = torch.empty((wl.T, wl.H), dtype=torch.bfloat16, device="cuda")
    lm.moe_lora_align(shape, dev["topk_ids"], dev["lora_ids"], ws)
    lm.moe_lora_forward(shape, dev["x"], dev["topk_ids"], dev["topk_weights"], dev["lora_ids"], dev["W_gu"],
                        dev["W_down"], dev["A_gu"], dev["B_gu"], dev["A_down"], dev["B_down"], ws, y)
    torch.cuda.synchronize()
    compare(y.float().cpu().numpy().astype(np.float64), oracle_tokens(inp, None), f"knobs bm={bm} {knobs}")
