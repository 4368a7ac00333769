"""Pins of the fp64 reference against facts fixed by the pages and by mathematics.

Each ``pin_*`` takes an ``oracle.Oracle`` and raises AssertionError when the
reference disagrees.  They are run on the shipped reference by
``test_oracle_pins.py`` and on deliberately broken copies of it by
``test_oracle_mutants.py`` (each broken copy must fail at least one pin).

What pins what:
  * worked examples in ``golden/worked_examples.json`` -- closed forms by hand;
  * E=1, k=1 reduces to a dense SwiGLU MLP, computed here with numpy matmuls;
  * one adapter = base layer with merged weights W + s*B*A (associativity of
    y = xW + xAB), and the same per (token, expert) pair in the general case;
  * invariances: token permutation, top-k slot order, adapter relabelling,
    expert relabelling, x = 0, B = 0, A = 0, no-adapter id, weight linearity;
  * the align against a comparison sort of the keys and hand-worked examples;
  * the router against a sort on (-logit, expert), scipy's softmax, hand-worked
    examples in ``golden/router_examples.json`` and its invariances.
"""
from __future__ import annotations

import json
import math
import os
from dataclasses import replace

import numpy as np

import synth

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")

RTOL = 1e-11


def close(a, b, rtol=RTOL, what=""):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    scale = max(1.0, float(np.max(np.abs(b))) if b.size else 1.0)
    err = float(np.max(np.abs(a - b))) if a.size else 0.0
    assert err <= rtol * scale, f"{what}: max |diff| {err:.3e} > {rtol:.1e} * {scale:.3e}"


def shape_of(wl):
    return (wl.T, wl.H, wl.I, wl.E, wl.topk, wl.L, wl.r)


def run(orc, inp, scale=None, **repl):
    """Reference output for ``inp`` with some arrays replaced."""
    a = inp.arrays()
    a.update(repl)
    wl = inp.wl
    T = a["x"].shape[0]
    shape = (T, wl.H, wl.I, wl.E, a["topk_ids"].shape[1], wl.L, wl.r)
    return orc.layer(shape, a["x"], a["topk_ids"], a["topk_weights"], a["lora_ids"], a["W_gu"],
                     a["W_down"], a["A_gu"], a["B_gu"], a["A_down"], a["B_down"],
                     scale=wl.scale if scale is None else scale, nthreads=2)


# Small workloads: several experts and adapters, a no-adapter id, non-trivial
# SiLU range (weights std 0.3 so gate values are O(1)).
PIN_WL = synth.Workload("pin", T=7, H=24, I=16, E=3, topk=2, L=3, r=4,
                        lora_mode="uniform_with_none", w_std=0.3, scale=0.5, seed=11)


def pin_inputs(**kw):
    return synth.make_inputs(replace(PIN_WL, **kw))


def silu(v):
    return v / (1.0 + np.exp(-v))


def dense_swiglu(x, Wg_u, Wd):
    """Textbook SwiGLU MLP with numpy matmuls: (silu(x Wg) * (x Wu)) Wd,
    where Wg_u stacks [gate; up] rows ([2I, H]) and Wd is [H, I]."""
    I = Wd.shape[1]
    gu = x @ Wg_u.T
    return (silu(gu[:, :I]) * gu[:, I:]) @ Wd.T


def f64(u):
    return synth.bf16_to_f64(u)


# ---------------------------------------------------------------- layer pins

def pin_worked_examples(orc):
    data = json.load(open(os.path.join(GOLDEN, "worked_examples.json")))
    env = {"exp": math.exp, "__builtins__": {}}
    for ex in data["examples"]:
        L, E, r, I, H = ex["L"], ex["E"], ex["r"], ex["I"], ex["H"]
        shape = (ex["T"], H, I, E, ex["topk"], L, r)
        b = synth.to_bf16
        y = orc.layer(shape, b(ex["x"]), np.array(ex["topk_ids"], np.int32),
                      np.array(ex["topk_weights"], np.float32), np.array(ex["lora_ids"], np.int32),
                      b(ex["W_gu"]), b(ex["W_down"]), b(ex["A_gu"]), b(ex["B_gu"]),
                      b(ex["A_down"]), b(ex["B_down"]), scale=ex["scale"], nthreads=1)
        want = np.array([[eval(s, env) for s in row] for row in ex["expected"]], dtype=np.float64)
        close(y, want, 1e-13, ex["name"])


def pin_dense_swiglu_no_adapter(orc):
    inp = pin_inputs(E=1, topk=1, lora_mode="none", T=5)
    inp.topk_weights[:] = 1.0
    y = run(orc, inp)
    want = dense_swiglu(f64(inp.x), f64(inp.W_gu[0]), f64(inp.W_down[0]))
    close(y, want, what="E=1 k=1 dense SwiGLU")


def pin_dense_swiglu_merged_adapter(orc):
    """One adapter on every token == base layer with W + s*B*A on both projections."""
    inp = pin_inputs(E=1, topk=1, L=1, lora_mode="uniform", T=5)
    inp.topk_weights[:] = 1.0
    s = inp.wl.scale
    Wg = f64(inp.W_gu[0]) + s * f64(inp.B_gu[0, 0]) @ f64(inp.A_gu[0, 0])
    Wd = f64(inp.W_down[0]) + s * f64(inp.B_down[0, 0]) @ f64(inp.A_down[0, 0])
    want = dense_swiglu(f64(inp.x), Wg, Wd)
    close(run(orc, inp), want, what="merged-weight identity")


def merged_moe(inp, scale):
    """Every (token, slot) pair as a dense SwiGLU MLP with its expert's weights
    merged with its adapter (W + s*B*A), weighted and summed over slots."""
    wl = inp.wl
    x = f64(inp.x)
    y = np.zeros((x.shape[0], wl.H))
    for t in range(x.shape[0]):
        l = int(inp.lora_ids[t])
        for j in range(inp.topk_ids.shape[1]):
            e = int(inp.topk_ids[t, j])
            if not (0 <= e < wl.E):
                continue
            Wg = f64(inp.W_gu[e])
            Wd = f64(inp.W_down[e])
            if 0 <= l < wl.L:
                Wg = Wg + scale * f64(inp.B_gu[l, e]) @ f64(inp.A_gu[l, e])
                Wd = Wd + scale * f64(inp.B_down[l, e]) @ f64(inp.A_down[l, e])
            y[t] += float(inp.topk_weights[t, j]) * dense_swiglu(x[t:t + 1], Wg, Wd)[0]
    return y


def pin_moe_merged_per_pair(orc):
    inp = pin_inputs()
    assert set(inp.lora_ids.tolist()) >= {-1}, "fixture should include no-adapter tokens"
    close(run(orc, inp), merged_moe(inp, inp.wl.scale), what="per-pair merged weights")


def pin_moe_merged_scale_one(orc):
    inp = pin_inputs(scale=1.0, seed=12, T=5)
    close(run(orc, inp), merged_moe(inp, 1.0), what="per-pair merged weights, s=1")


def pin_no_adapter_paths(orc):
    """lora = -1, B = 0 or A = 0 all reduce to the base layer."""
    inp = pin_inputs()
    base = run(orc, inp, lora_ids=np.full_like(inp.lora_ids, -1))
    zB = dict(B_gu=np.zeros_like(inp.B_gu), B_down=np.zeros_like(inp.B_down))
    zA = dict(A_gu=np.zeros_like(inp.A_gu), A_down=np.zeros_like(inp.A_down))
    close(run(orc, inp, **zB), base, 0.0, "B=0")
    close(run(orc, inp, **zA), base, 0.0, "A=0")
    # adapter ids outside [-1, L) are treated as no adapter
    bad = inp.lora_ids.copy()
    bad[0], bad[1] = inp.wl.L, -7
    ref = inp.lora_ids.copy()
    ref[0], ref[1] = -1, -1
    close(run(orc, inp, lora_ids=bad), run(orc, inp, lora_ids=ref), 0.0, "invalid adapter ids")
    # the LoRA must change the output when present
    assert np.max(np.abs(run(orc, inp) - base)) > 1e-3, "adapters have no effect"


def pin_zero_input(orc):
    inp = pin_inputs()
    y = run(orc, inp, x=np.zeros_like(inp.x))
    assert np.all(y == 0.0), "x = 0 must give y = 0 exactly"


def pin_token_permutation(orc):
    inp = pin_inputs()
    perm = np.array([3, 0, 6, 1, 5, 2, 4])
    y = run(orc, inp)
    yp = run(orc, inp, x=inp.x[perm], topk_ids=inp.topk_ids[perm],
             topk_weights=inp.topk_weights[perm], lora_ids=inp.lora_ids[perm])
    close(yp, y[perm], 1e-14, "token permutation")


def pin_slot_order(orc):
    inp = pin_inputs()
    y = run(orc, inp)
    yr = run(orc, inp, topk_ids=inp.topk_ids[:, ::-1].copy(),
             topk_weights=inp.topk_weights[:, ::-1].copy())
    close(yr, y, 1e-13, "top-k slot order")


def pin_adapter_relabel(orc):
    inp = pin_inputs()
    L = inp.wl.L
    sig = np.array([2, 0, 1])  # new id of old adapter l is sig[l]
    inv = np.argsort(sig)
    relab = dict(A_gu=inp.A_gu[inv], B_gu=inp.B_gu[inv], A_down=inp.A_down[inv],
                 B_down=inp.B_down[inv],
                 lora_ids=np.where(inp.lora_ids >= 0, sig[np.clip(inp.lora_ids, 0, L - 1)], -1)
                 .astype(np.int32))
    close(run(orc, inp, **relab), run(orc, inp), 1e-14, "adapter relabelling")


def pin_expert_relabel(orc):
    inp = pin_inputs()
    sig = np.array([1, 2, 0])
    inv = np.argsort(sig)
    relab = dict(W_gu=inp.W_gu[inv], W_down=inp.W_down[inv], A_gu=inp.A_gu[:, inv],
                 B_gu=inp.B_gu[:, inv], A_down=inp.A_down[:, inv], B_down=inp.B_down[:, inv],
                 topk_ids=sig[inp.topk_ids].astype(np.int32))
    close(run(orc, inp, **relab), run(orc, inp), 1e-14, "expert relabelling")


def pin_weight_linearity(orc):
    """The top-k weights enter linearly: y(w1) + y(w2) = y(w1 + w2); a zero
    weight removes the pair; an out-of-range expert id removes it too."""
    inp = pin_inputs()
    w1 = (np.round(inp.topk_weights * 1024) / 1024).astype(np.float32)
    w2 = (np.arange(w1.size).reshape(w1.shape) / 8.0 - 1.0).astype(np.float32)
    s = (w1.astype(np.float64) + w2).astype(np.float32)
    assert np.all(s.astype(np.float64) == w1.astype(np.float64) + w2), "need exact sums"
    close(run(orc, inp, topk_weights=s),
          run(orc, inp, topk_weights=w1) + run(orc, inp, topk_weights=w2), 1e-13, "linearity")
    w0 = w1.copy()
    w0[:, 1] = 0
    bad = inp.topk_ids.copy()
    bad[:, 1] = np.array([inp.wl.E, -1, 99, inp.wl.E, -3, 7, 3])
    close(run(orc, inp, topk_ids=bad, topk_weights=w1), run(orc, inp, topk_weights=w0), 0.0,
          "dropped pairs")


def pin_pair_stages(orc):
    """Intermediates of one pair against the stage definitions with numpy:
    g = W_gu x + s B_gu (A_gu x); h = silu(g[:I]) g[I:]; d = W_down h + s B_down (A_down h)."""
    inp = pin_inputs()
    wl = inp.wl
    t = int(np.flatnonzero(inp.lora_ids >= 0)[0])
    for j in range(wl.topk):
        e, l = int(inp.topk_ids[t, j]), int(inp.lora_ids[t])
        st = orc.pair(shape_of(wl), inp.x, inp.topk_ids, inp.lora_ids, inp.W_gu, inp.W_down,
                      inp.A_gu, inp.B_gu, inp.A_down, inp.B_down, t, j, scale=wl.scale)
        x = f64(inp.x[t])
        zg = f64(inp.A_gu[l, e]) @ x
        g = f64(inp.W_gu[e]) @ x + wl.scale * f64(inp.B_gu[l, e]) @ zg
        h = silu(g[:wl.I]) * g[wl.I:]
        zd = f64(inp.A_down[l, e]) @ h
        d = f64(inp.W_down[e]) @ h + wl.scale * f64(inp.B_down[l, e]) @ zd
        for name, want in (("zg", zg), ("g", g), ("h", h), ("zd", zd), ("d", d)):
            close(st[name], want, what=f"stage {name}")


LAYER_PINS = [pin_worked_examples, pin_dense_swiglu_no_adapter, pin_dense_swiglu_merged_adapter,
              pin_moe_merged_per_pair, pin_moe_merged_scale_one, pin_no_adapter_paths,
              pin_zero_input, pin_token_permutation, pin_slot_order, pin_adapter_relabel,
              pin_expert_relabel, pin_weight_linearity, pin_pair_stages]


# ---------------------------------------------------------------- align pins

def align_by_comparison_sort(T, k, E, L, bm, topk_ids, lora_ids):
    """The align contract by a comparison sort of (expert, slot, p) keys."""
    ids = np.asarray(topk_ids).reshape(-1)
    P = T * k
    keys = []
    err = sum(1 for t in range(T) if not (-1 <= lora_ids[t] < L))
    for p in range(P):
        e = int(ids[p])
        if not (0 <= e < E):
            err += 1
            continue
        l = int(lora_ids[p // k])
        s = l if 0 <= l < L else L
        keys.append((e, s, p))
    keys.sort()
    rows, expert_off, seg_start, seg_cnt, block_expert = [], [0], [], [], []
    for e in range(E):
        mine = [kk for kk in keys if kk[0] == e]
        for s in range(L + 1):
            seg = [kk for kk in mine if kk[1] == s]
            # rows already holds the runs of experts < e, so len(rows) is this run's start
            seg_start.append(len(rows) + sum(1 for kk in mine if kk[1] < s))
            seg_cnt.append(len(seg))
        run_ = [kk[2] for kk in mine]
        while len(run_) % bm:
            run_.append(P)
        block_expert += [e] * (len(run_) // bm)
        rows += run_
        expert_off.append(len(rows))
    pos = [-1] * P
    for i, p in enumerate(rows):
        if p < P:
            pos[p] = i
    return dict(sorted_ids=np.array(rows, np.int32), expert_off=np.array(expert_off, np.int32),
                seg_start=np.array(seg_start, np.int32), seg_cnt=np.array(seg_cnt, np.int32),
                block_expert=np.array(block_expert, np.int32), pos_of_pair=np.array(pos, np.int32),
                num_padded=len(rows), err_count=err)


def check_align(got, want, P, bm, what=""):
    n = want["num_padded"]
    assert got["num_padded"] == n, f"{what}: num_padded {got['num_padded']} != {n}"
    assert got["err_count"] == want["err_count"], f"{what}: err_count"
    np.testing.assert_array_equal(got["sorted_ids"][:n], want["sorted_ids"][:n], err_msg=what)
    assert np.all(got["sorted_ids"][n:] == P), f"{what}: sentinel beyond num_padded"
    for name in ("expert_off", "seg_start", "seg_cnt", "pos_of_pair"):
        np.testing.assert_array_equal(got[name], want[name], err_msg=f"{what}: {name}")
    nb = n // bm
    np.testing.assert_array_equal(got["block_expert"][:nb], want["block_expert"][:nb],
                                  err_msg=f"{what}: block_expert")
    assert np.all(got["block_expert"][nb:] == -1), f"{what}: unused blocks must be -1"


def align_cases():
    """(name, T, k, E, L, block_m, topk_ids, lora_ids) including adversarial ones."""
    rng = np.random.default_rng(5)
    cases = []
    for (T, k, E, L, bm) in ((9, 2, 4, 3, 4), (33, 3, 5, 2, 8), (16, 4, 16, 4, 16), (1, 1, 2, 1, 16),
                             (0, 2, 3, 2, 16), (40, 2, 3, 1, 32)):
        ids = np.array([rng.permutation(E)[:k] for _ in range(T)], dtype=np.int32).reshape(T, k)
        lids = rng.integers(-1, L, size=T).astype(np.int32)
        cases.append((f"rand_T{T}_E{E}_bm{bm}", T, k, E, L, bm, ids, lids))
    # all pairs to one expert and one adapter
    cases.append(("one_bucket", 20, 1, 4, 2, 16, np.full((20, 1), 2, np.int32), np.zeros(20, np.int32)))
    # every token without adapter
    ids = np.stack([rng.permutation(6)[:2] for _ in range(25)]).astype(np.int32)
    cases.append(("all_no_adapter", 25, 2, 6, 3, 8, ids, np.full(25, -1, np.int32)))
    # invalid expert and adapter ids
    ids = rng.integers(-2, 6, size=(30, 2)).astype(np.int32)
    lids = rng.integers(-3, 5, size=30).astype(np.int32)
    cases.append(("invalid_ids", 30, 2, 4, 3, 4, ids, lids))
    return cases


def pin_align_examples(orc):
    data = json.load(open(os.path.join(GOLDEN, "align_examples.json")))
    for ex in data["examples"]:
        T, k, E, L, bm = ex["T"], ex["topk"], ex["E"], ex["L"], ex["block_m"]
        got = orc.align(T, k, E, L, bm, np.array(ex["topk_ids"], np.int32),
                        np.array(ex["lora_ids"], np.int32))
        w = ex["expected"]
        n = w["num_padded"]
        assert got["num_padded"] == n, ex["name"]
        assert got["err_count"] == w["err_count"], ex["name"]
        np.testing.assert_array_equal(got["sorted_ids"][:n], w["sorted_ids_prefix"], ex["name"])
        assert np.all(got["sorted_ids"][n:] == T * k), ex["name"]
        for name in ("expert_off", "seg_start", "seg_cnt", "pos_of_pair"):
            np.testing.assert_array_equal(got[name], w[name], err_msg=f"{ex['name']}: {name}")
        np.testing.assert_array_equal(got["block_expert"][:n // bm], w["block_expert_prefix"])
        assert np.all(got["block_expert"][n // bm:] == -1)


def pin_align_comparison_sort(orc):
    for name, T, k, E, L, bm, ids, lids in align_cases():
        got = orc.align(T, k, E, L, bm, ids, lids)
        want = align_by_comparison_sort(T, k, E, L, bm, ids, lids)
        check_align(got, want, T * k, bm, name)


def pin_align_invariants(orc):
    for name, T, k, E, L, bm, ids, lids in align_cases():
        got = orc.align(T, k, E, L, bm, ids, lids)
        P = T * k
        n = got["num_padded"]
        off = got["expert_off"]
        assert np.all(off % bm == 0) and off[-1] == n, name
        srt = got["sorted_ids"][:n]
        real = srt[srt < P]
        valid = [p for p in range(P) if 0 <= ids.reshape(-1)[p] < E]
        assert sorted(real.tolist()) == valid, f"{name}: not a permutation of valid pairs"
        assert got["seg_cnt"].sum() == len(valid), name
        for e in range(E):
            run_ = srt[off[e]:off[e + 1]]
            assert np.all(ids.reshape(-1)[run_[run_ < P]] == e), f"{name}: wrong expert in run"


ALIGN_PINS = [pin_align_examples, pin_align_comparison_sort, pin_align_invariants]


# ------------------------------------------------------------------ router

def route_by_sorting(logits, k):
    """Top-k by sorting (expert, logit) pairs on (-logit, expert) -- an
    independent statement of "largest first, ties to the lower index" -- and
    the weights from scipy's softmax over the chosen logits.  Non-finite
    logits are left out of the sort; slots past the finite ones get -1 and
    weight 0."""
    from scipy.special import softmax
    T, E = logits.shape
    ids = np.full((T, k), -1, np.int32)
    w = np.zeros((T, k))
    for t in range(T):
        fin = [e for e in range(E) if np.isfinite(logits[t, e])]
        order = sorted(fin, key=lambda e: (-float(logits[t, e]), e))[:k]
        ids[t, :len(order)] = order
        if order:
            w[t, :len(order)] = softmax(logits[t, order].astype(np.float64))
    return ids, w


def router_cases():
    rng = np.random.default_rng(7)
    cases = []
    for T, E, k in [(5, 8, 2), (4, 16, 4), (3, 6, 6), (6, 32, 8), (2, 5, 1)]:
        lg = rng.standard_normal((T, E)).astype(np.float32)
        cases.append((f"normal T={T} E={E} k={k}", lg, k))
    # ties: logits on a coarse grid
    lg = rng.integers(-2, 3, size=(8, 10)).astype(np.float32)
    cases.append(("grid ties", lg, 3))
    # non-finite logits scattered among finite ones, and rows with fewer
    # finite logits than k
    lg = rng.standard_normal((6, 9)).astype(np.float32)
    lg[rng.random((6, 9)) < 0.3] = np.nan
    lg[0, 2] = np.inf
    lg[1, 4] = -np.inf
    lg[2, :7] = -np.inf
    lg[3, :] = np.nan
    cases.append(("non-finite", lg, 4))
    return cases


def pin_router_examples(orc):
    data = json.load(open(os.path.join(GOLDEN, "router_examples.json")))
    for ex in data["examples"]:
        ids, w = orc.route(np.array([[float(v) for v in row] for row in ex["logits"]], np.float32), ex["k"])
        assert ids.tolist() == ex["ids"], f"{ex['name']}: ids {ids.tolist()}"
        close(w, np.array(ex["weights"]), rtol=ex.get("weights_rtol", 1e-14), what=ex["name"])


def pin_router_sorting(orc):
    for name, lg, k in router_cases():
        ids, w = orc.route(lg, k)
        ids2, w2 = route_by_sorting(lg, k)
        assert np.array_equal(ids, ids2), f"{name}: ids differ from the sorted order"
        close(w, w2, rtol=1e-13, what=name)


def pin_router_invariants(orc):
    rng = np.random.default_rng(11)
    lg = rng.standard_normal((6, 12)).astype(np.float32)
    k = 4
    ids, w = orc.route(lg, k)
    # weights sum to one; full softmax renormalised over the chosen experts
    assert np.allclose(w.sum(axis=1), 1.0, rtol=0, atol=1e-14)
    full = np.exp(lg.astype(np.float64) - lg.max(axis=1, keepdims=True))
    full /= full.sum(axis=1, keepdims=True)
    sel = np.take_along_axis(full, ids.astype(np.int64), axis=1)
    close(w, sel / sel.sum(axis=1, keepdims=True), rtol=1e-13, what="renormalised softmax")
    # weights are non-increasing along the slots
    assert np.all(np.diff(w, axis=1) <= 1e-15)
    # a shift of a token's logits by a power of two changes nothing
    ids_s, w_s = orc.route(lg + np.float32(4.0), k)
    assert np.array_equal(ids, ids_s)
    close(w, w_s, rtol=1e-6, what="shift")
    # relabelling experts relabels the choice (distinct logits here)
    perm = rng.permutation(12)
    ids_p, w_p = orc.route(lg[:, perm], k)
    assert np.array_equal(perm[ids_p], ids), "expert relabelling"
    close(w, w_p, rtol=1e-14, what="relabel")
    # k = E: every expert once, weights = the full softmax in that order
    ids_a, w_a = orc.route(lg, 12)
    assert all(sorted(r) == list(range(12)) for r in ids_a.tolist())
    close(w_a, np.take_along_axis(full, ids_a.astype(np.int64), axis=1), rtol=1e-13, what="k=E")


ROUTER_PINS = [pin_router_examples, pin_router_sorting, pin_router_invariants]
ALL_PINS = LAYER_PINS + ALIGN_PINS + ROUTER_PINS
