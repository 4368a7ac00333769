"""Router (top-k + weights from logits) and the fused router + align on the
GPU against the fp64 reference: expert ids bit-exact, weights to 1e-6."""
import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_common import compare, gpu_views, log, oracle_tokens

pytestmark = pytest.mark.gpu


def logits_for(T, E, seed, ties=False, bias_std=0.0):
    key = synth.stream_key(seed, 0, T, E)
    if ties:  # a coarse grid: many equal logits per token
        lg = np.floor(synth.uniform(key, T * E) * 5.0) - 2.0
    else:
        lg = synth.normal(key, T * E)
        if bias_std > 0:
            lg = lg.reshape(T, E) + synth.normal(synth.stream_key(seed, 1, T, E), E, 0.0, bias_std)[None, :]
    return np.ascontiguousarray(np.asarray(lg, np.float64).reshape(T, E).astype(np.float32))


def gpu_route(lg, k, L=1):
    import lora_moe_amd as lm
    T, E = lg.shape
    shape = lm.make_shape(T, 8, 8, E, k, L, 8)
    ids = torch.empty((T, k), dtype=torch.int32, device="cuda")
    w = torch.empty((T, k), dtype=torch.float32, device="cuda")
    lm.moe_lora_route(shape, torch.from_numpy(lg).cuda(), ids, w)
    torch.cuda.synchronize()
    return ids.cpu().numpy(), w.cpu().numpy()


CASES = [  # T, E, k, ties, bias
    (64, 8, 2, False, 0.0), (33, 256, 8, False, 2.0), (17, 128, 1, False, 0.0),
    (40, 10, 3, True, 0.0), (9, 80, 64, False, 0.0), (12, 700, 6, False, 0.0),
    (7, 700, 5, True, 0.0), (5, 4, 4, True, 0.0), (1, 1, 1, False, 0.0),
]


@pytest.mark.parametrize("T,E,k,ties,bias", CASES)
def test_router_matches_reference(T, E, k, ties, bias):
    lg = logits_for(T, E, seed=T * 1000 + E, ties=ties, bias_std=bias)
    log(f"router T={T} E={E} k={k} ties={ties}")
    ids, w = gpu_route(lg, k)
    rids, rw = oracle.Oracle().route(lg, k)
    assert np.array_equal(ids, rids), f"ids differ in {int((ids != rids).sum())} slots"
    err = float(np.max(np.abs(w - rw)))
    log(f"router T={T} E={E} k={k}: ids exact, max |dw| {err:.2e}")
    assert err <= 1e-6


def nonfinite_logits(T, E, seed):
    lg = logits_for(T, E, seed=seed)
    lg[0, 3] = np.nan
    lg[1, :] = -np.inf
    lg[1, 7] = 0.5            # one finite logit: slot 0 gets it, the rest -1
    lg[2, 0] = np.inf         # +inf is not chosen either
    lg[3, :] = np.nan         # nothing eligible
    lg[4, ::2] = np.inf
    return lg


@pytest.mark.parametrize("E", [16, 200])
def test_router_nonfinite_matches_reference(E):
    """Non-finite logits (NaN, +inf, -inf) are never chosen; slots without a
    finite logit get -1 and weight 0: ids bit-exact and weights within 1e-6
    of the reference, every weight finite."""
    k = 3
    lg = nonfinite_logits(8, E, seed=5)
    ids, w = gpu_route(lg, k)
    rids, rw = oracle.Oracle().route(lg, k)
    assert rids[1].tolist() == [7, -1, -1] and rids[3].tolist() == [-1, -1, -1]
    assert 0 not in rids[2].tolist()
    assert np.array_equal(ids, rids), f"ids {ids.tolist()} vs {rids.tolist()}"
    assert np.all(np.isfinite(w))
    assert float(np.max(np.abs(w - rw))) <= 1e-6


def test_route_align_nonfinite_matches_reference():
    """The same through the fused router + align kernel (one thread per
    token): the -1 slots are dropped and counted by the align."""
    import lora_moe_amd as lm
    T, E, k, L = 8, 16, 3, 2
    lg = nonfinite_logits(T, E, seed=6)
    lids = np.zeros(T, np.int32)
    shape = lm.make_shape(T, 64, 64, E, k, L, 8, 16)
    ws = lm.alloc_workspace(shape)
    ids = torch.empty((T, k), dtype=torch.int32, device="cuda")
    w = torch.empty((T, k), dtype=torch.float32, device="cuda")
    lm.moe_lora_route_align(shape, torch.from_numpy(lg).cuda(), torch.from_numpy(lids).cuda(), ids, w, ws)
    torch.cuda.synchronize()
    o = oracle.Oracle()
    rids, rw = o.route(lg, k)
    assert np.array_equal(ids.cpu().numpy(), rids)
    wg = w.cpu().numpy()
    assert np.all(np.isfinite(wg)) and float(np.max(np.abs(wg - rw))) <= 1e-6
    got = gpu_views(shape, ws)
    want = o.align(T, k, E, L, 16, rids, lids, got["cap_rows"], got["cap_blocks"])
    for name in ("sorted_ids", "expert_off", "pos_of_pair"):
        assert np.array_equal(got[name], want[name]), name
    assert got["err_count"] == want["err_count"] == int((rids < 0).sum())


@pytest.mark.parametrize("T,E,k,L,bm", [(16, 8, 2, 8, 16), (32, 64, 8, 5, 32), (100, 64, 8, 5, 32), (300, 32, 4, 16, 128),
                                        (2048, 128, 8, 32, 256)])
def test_route_align_matches_reference(T, E, k, L, bm):
    """The fused call (one kernel while T*k <= 256, router kernel first beyond)
    against the reference router followed by the reference align."""
    import lora_moe_amd as lm
    lg = logits_for(T, E, seed=77 + T)
    lids = synth.adapter_ids(synth.Workload("r", T=T, H=8, I=8, E=E, topk=k, L=L, r=8,
                                            lora_mode="uniform_with_none"))
    shape = lm.make_shape(T, 64, 64, E, k, L, 8, bm)
    ws = lm.alloc_workspace(shape)
    ids = torch.empty((T, k), dtype=torch.int32, device="cuda")
    w = torch.empty((T, k), dtype=torch.float32, device="cuda")
    lm.moe_lora_route_align(shape, torch.from_numpy(lg).cuda(), torch.from_numpy(lids).cuda(), ids, w, ws)
    torch.cuda.synchronize()
    o = oracle.Oracle()
    rids, rw = o.route(lg, k)
    assert np.array_equal(ids.cpu().numpy(), rids)
    assert float(np.max(np.abs(w.cpu().numpy() - rw))) <= 1e-6
    got = gpu_views(shape, ws)
    want = o.align(T, k, E, L, got["block_m"], rids, lids, got["cap_rows"], got["cap_blocks"])
    for name in ("sorted_ids", "expert_off", "seg_start", "seg_cnt", "block_expert", "pos_of_pair"):
        assert np.array_equal(got[name], want[name]), f"{name} differs"
    assert got["num_padded"] == want["num_padded"] and got["err_count"] == want["err_count"]
    log(f"route_align T={T} E={E} k={k} bm={bm}: bit-exact")


def test_layer_from_logits():
    """Router + align + forward against the reference layer on the reference
    router's ids and weights."""
    import lora_moe_amd as lm
    wl = synth.WORKLOADS[1]
    inp = synth.make_inputs(wl)
    lg = logits_for(wl.T, wl.E, seed=3)
    shape = lm.make_shape(wl.T, wl.H, wl.I, wl.E, wl.topk, wl.L, wl.r, 0, wl.scale)
    ws = lm.alloc_workspace(shape)
    ids = torch.empty((wl.T, wl.topk), dtype=torch.int32, device="cuda")
    w = torch.empty((wl.T, wl.topk), dtype=torch.float32, device="cuda")
    lids = torch.from_numpy(inp.lora_ids).cuda()
    y = torch.empty((wl.T, wl.H), dtype=torch.bfloat16, device="cuda")
    lm.moe_lora_route_align(shape, torch.from_numpy(lg).cuda(), lids, ids, w, ws)

    def u16(name):
        return torch.from_numpy(np.ascontiguousarray(getattr(inp, name)).view(np.int16)).cuda().view(torch.bfloat16)

    lm.moe_lora_forward(shape, u16("x"), ids, w, lids, u16("W_gu"), u16("W_down"), u16("A_gu"), u16("B_gu"),
                        u16("A_down"), u16("B_down"), ws, y)
    torch.cuda.synchronize()
    rids, rw = oracle.Oracle().route(lg, wl.topk)
    inp.topk_ids[:] = rids
    inp.topk_weights[:] = rw.astype(np.float32)
    ref = oracle_tokens(inp, None)
    compare(y.float().cpu().numpy(), ref, "layer from logits")
