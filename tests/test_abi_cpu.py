"""The C-ABI library on the CPU: it loads, exports every declared symbol, and
its host-side checks return the documented codes without touching a GPU."""
import ctypes
import os
import re

import pytest

import lora_moe_amd as lm
import synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def declared_functions():
    names = set()
    for fn in os.listdir(os.path.join(ROOT, "include")):
        if fn.endswith(".h"):
            src = open(os.path.join(ROOT, "include", fn)).read()
            src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
            names |= set(re.findall(r"\b(moe_lora_\w+)\s*\(", src))
    return sorted(names)


@pytest.fixture(scope="module")
def lib():
    return lm.load_library()


def test_exports_every_declared_symbol(lib):
    names = declared_functions()
    assert len(names) >= 10
    missing = [n for n in names if not hasattr(lib, n)]
    assert not missing, missing


def test_status_strings(lib):
    assert lm.moe_lora_status_str(0) == "ok"
    assert "workspace" in lm.moe_lora_status_str(lm.MOE_LORA_EWORKSPACE)
    assert lm.moe_lora_status_str(-99) == "unknown status"


def shape_of(wl, bm=0):
    return lm.make_shape(wl.T, wl.H, wl.I, wl.E, wl.topk, wl.L, wl.r, bm, wl.scale)


@pytest.mark.parametrize("n", [1, 2, 3, 4, 5, 6])
def test_workspace_and_block_m(lib, n):
    wl = synth.WORKLOADS[n]
    s = shape_of(wl)
    bm = lm.moe_lora_resolve_block_m(s)
    # the built-in choice: 16-row streaming tiles at <= 16 rows per expert,
    # 32-row ones for the dense layer, 64 x 128 tiles at ~32 rows per expert
    # (GPT-OSS-like), 192 x 256 at ~128 (Qwen3-MoE-like), 256 x 256 at ~256
    assert bm == {1: 16, 2: 16, 3: 64, 4: 192, 5: 256, 6: 32}[n]
    ws = lm.moe_lora_workspace_bytes(s)
    P = wl.T * wl.topk
    cap = P + wl.E * (bm - 1)
    # at least the intermediates h (bf16) and d (fp32) for every row
    assert ws >= cap * (2 * wl.I + 4 * wl.H)
    s2 = shape_of(wl, 64)
    assert lm.moe_lora_resolve_block_m(s2) == 64


def test_block_m_heuristic_boundaries(lib):
    """The built-in block_m at each edge of its rows-per-expert ranges (64
    experts top-8: T = 8 * rows gives T * 8 / 64 = rows per expert; H = 2048
    gives the tiled grids enough column tiles), and the streaming fallback for
    a single expert."""
    want = {16: 16, 17: 32, 24: 32, 25: 64, 48: 64, 49: 128, 95: 128, 96: 192, 144: 192,
            145: 256, 1000: 256}
    for rows, bm in want.items():
        s = lm.make_shape(8 * rows, 2048, 768, 64, 8, 4, 16)
        assert lm.moe_lora_resolve_block_m(s) == bm, rows
    # one expert with wide weights: 40 column tiles of 128 < 512 -> streaming
    assert lm.moe_lora_resolve_block_m(lm.make_shape(200, 5120, 25600, 1, 1, 8, 16)) == 32


def test_bad_shapes(lib):
    good = dict(T=4, H=64, I=32, E=4, topk=2, L=2, r=8)
    cases = [
        (dict(T=-1), lm.MOE_LORA_EINVAL), (dict(H=0), lm.MOE_LORA_EINVAL),
        (dict(topk=5), lm.MOE_LORA_EINVAL), (dict(L=0), lm.MOE_LORA_EINVAL),
        (dict(block_m=48), lm.MOE_LORA_EINVAL), (dict(block_m=96), lm.MOE_LORA_EINVAL), (dict(H=60), lm.MOE_LORA_EALIGN),
        (dict(I=36), lm.MOE_LORA_EALIGN), (dict(r=12), lm.MOE_LORA_EUNSUPPORTED),
        (dict(r=136), lm.MOE_LORA_EUNSUPPORTED), (dict(E=8000, L=2), lm.MOE_LORA_EUNSUPPORTED),
    ]
    for over, code in cases:
        args = dict(good, **over)
        s = lm.make_shape(**args)
        assert lm.moe_lora_resolve_block_m(s) == code, over
        assert lm.moe_lora_workspace_bytes(s) == 0, over
        rc = lib.moe_lora_align(ctypes.byref(s), None, None, None, 0, None)
        assert rc == code, over


def test_size_limits(lib):
    """The index-width limits, each met alone: one under it is accepted, at
    it refused with EUNSUPPORTED (x rows and the intermediate rows are read
    through 32-bit byte offsets, one expert's weights through 32-bit element
    offsets; cap = T*topk + 255*E rows)."""
    small = dict(E=1, topk=1, L=1, r=8)
    pairs = [  # (accepted, refused)
        (dict(T=(1 << 24) - 1, H=64, I=8), dict(T=1 << 24, H=64, I=8)),          # T*H*2 vs 2^31
        (dict(T=1, H=32768, I=65528), dict(T=1, H=32768, I=65536)),            # 2*I*H vs 2^32
        (dict(T=(1 << 26) - 256, H=8, I=16), dict(T=(1 << 26) - 255, H=8, I=16)),  # cap*I*2 vs 2^31
    ]
    for ok, bad in pairs:
        assert lm.moe_lora_workspace_bytes(lm.make_shape(**dict(small, **ok))) > 0, ok
        s = lm.make_shape(**dict(small, **bad))
        assert lm.moe_lora_resolve_block_m(s) == lm.MOE_LORA_EUNSUPPORTED, bad
        assert lm.moe_lora_workspace_bytes(s) == 0, bad
    # more pairs than 2^30
    s = lm.make_shape(**dict(small, T=(1 << 26) + 1, H=8, I=8, E=16, topk=16))
    assert lm.moe_lora_resolve_block_m(s) == lm.MOE_LORA_EUNSUPPORTED


def test_null_and_workspace_checks_do_not_launch(lib):
    s = lm.make_shape(4, 64, 32, 4, 2, 2, 8)
    need = lm.moe_lora_workspace_bytes(s)
    buf = ctypes.create_string_buffer(64)
    p = ctypes.addressof(buf)
    p16 = (p + 15) // 16 * 16
    assert lib.moe_lora_align(ctypes.byref(s), None, p16, p16, need, None) == lm.MOE_LORA_EINVAL
    assert lib.moe_lora_align(ctypes.byref(s), p16, p16, p16, need - 1, None) == lm.MOE_LORA_EWORKSPACE
    assert lib.moe_lora_align(ctypes.byref(s), p16, p16, p16 + 4, need, None) == lm.MOE_LORA_EALIGN
    args = [p16] * 11
    assert lib.moe_lora_forward(ctypes.byref(s), *args, need - 1, p16, None) == lm.MOE_LORA_EWORKSPACE
    bad = list(args)
    bad[4] = p16 + 2  # W_gu misaligned
    assert lib.moe_lora_forward(ctypes.byref(s), *bad[:10], p16, need, bad[10], None) == lm.MOE_LORA_EALIGN
    bad = list(args)
    bad[0] = None
    assert lib.moe_lora_forward(ctypes.byref(s), *bad[:10], p16, need, bad[10], None) == lm.MOE_LORA_EINVAL
    # T = 0 is a no-op that succeeds without any device call
    s0 = lm.make_shape(0, 64, 32, 4, 2, 2, 8)
    assert lib.moe_lora_align(ctypes.byref(s0), None, None, None, 0, None) == 0
    n = ctypes.c_int32(7)
    assert lib.moe_lora_device_errors(ctypes.byref(s0), p16, ctypes.byref(n), None) == 0
    assert n.value == 0


def test_view_offsets_are_aligned_and_disjoint(lib):
    wl = synth.WORKLOADS[3]
    s = shape_of(wl)
    v = lm.moe_lora_workspace_view(s, type("T", (), {
        "is_cuda": True, "is_contiguous": lambda self: True, "data_ptr": lambda self: 1 << 20})())
    addrs = sorted(getattr(v, n) for n in ("sorted_ids", "expert_off", "seg_start", "seg_cnt",
                                            "block_expert", "pos_of_pair", "z_gu", "z_down", "h", "d"))
    assert all(a % 256 == 0 for a in addrs)
    assert len(set(addrs)) == len(addrs)
    assert v.d - (1 << 20) + v.cap_rows * wl.H * 4 <= lm.moe_lora_workspace_bytes(s)


# ------------------------------------------------------------------ tuning table

def _entry(rows, H, I, E, r, L, bm):
    return lm.moe_lora_tune_entry(rows, H, I, E, r, L, bm)


def test_tune_pick_nearest_and_fallbacks(lib):
    """moe_lora_tune_block_m: nearest entry by the weighted log2 distance,
    the built-in choice when the table is empty, too far or invalid, and the
    shape's own block_m when it is set."""
    decode = lm.make_shape(16, 4096, 11008, 8, 2, 8, 32)       # 4 rows per expert
    prefill = lm.make_shape(8192, 7168, 2048, 256, 8, 8, 64)   # 256 rows per expert
    table = (lm.moe_lora_tune_entry * 3)(_entry(4, 4096, 11008, 8, 32, 8, 64),
                                         _entry(256, 7168, 2048, 256, 64, 8, 128),
                                         _entry(300, 7168, 2048, 256, 64, 8, 256))
    t = (table, 3)
    assert lm.moe_lora_tune_block_m(decode, t) == 64
    assert lm.moe_lora_tune_block_m(prefill, t) == 128          # exact key beats the near one
    builtin = lm.moe_lora_resolve_block_m(decode)
    assert lm.moe_lora_tune_block_m(decode, (table, 0)) == builtin
    # rows_per_expert counts four times: 4 -> 8 rows is distance 4
    far = (lm.moe_lora_tune_entry * 1)(_entry(8, 4096, 11008, 8, 32, 8, 128))
    assert lm.moe_lora_tune_block_m(decode, (far, 1), 3.5) == builtin
    assert lm.moe_lora_tune_block_m(decode, (far, 1), 4.5) == 128
    assert lm.moe_lora_tune_block_m(decode, (far, 1), 0.0) == 128
    # invalid entries are skipped
    bad = (lm.moe_lora_tune_entry * 2)(_entry(4, 4096, 11008, 8, 32, 8, 48),
                                       _entry(0, 4096, 11008, 8, 32, 8, 32))
    assert lm.moe_lora_tune_block_m(decode, (bad, 2)) == builtin
    # a set block_m wins; an invalid shape returns its status
    assert lm.moe_lora_tune_block_m(lm.make_shape(16, 4096, 11008, 8, 2, 8, 32, 128), t) == 128
    assert lm.moe_lora_tune_block_m(lm.make_shape(16, 4096, 11008, 8, 2, 8, 7), t) == lm.MOE_LORA_EUNSUPPORTED
    # make_shape consults the table only when block_m is 0
    assert lm.make_shape(16, 4096, 11008, 8, 2, 8, 32, tuning=t).block_m == 64
    assert lm.make_shape(16, 4096, 11008, 8, 2, 8, 32, 32, tuning=t).block_m == 32


def test_committed_tuning_table_is_valid(lib):
    """The shipped table loads, its entries are complete and valid, and each
    entry picks its own block_m for the workload it was swept on."""
    import json
    doc = json.load(open(lm.TUNING_PATH))
    assert doc["arch"] == "gfx950" and doc["entries"]
    table = lm.load_tuning()
    byname = {w.name: w for w in synth.WORKLOADS.values()}
    for e in doc["entries"]:
        assert e["block_m"] in (16, 32, 64, 128, 192, 256)
        assert str(e["block_m"]) in e["ms"] and min(e["ms"], key=e["ms"].get) == str(e["block_m"])
        wl = byname[e["workload"]]
        shape = lm.make_shape(wl.T, wl.H, wl.I, wl.E, wl.topk, wl.L, wl.r, 0, wl.scale, tuning=table)
        assert shape.block_m == e["block_m"]
        for k in lm.KNOBS:
            assert getattr(shape, k) == e.get(k, 0), (e["workload"], k)
            if e.get(k, 0):  # a stored knob beat the library's own choice in the sweep
                assert k in e["knob_ms"] and str(e[k]) in e["knob_ms"][k]


# ------------------------------------------------------------------ views, operand checks, h hi + lo

FAKE_BASE = 1 << 20


def _fake_ws():
    return type("T", (), {"is_cuda": True, "is_contiguous": lambda self: True,
                          "data_ptr": lambda self: FAKE_BASE})()


@pytest.mark.parametrize("n", [1, 3, 5])
def test_align_view_matches_workspace_view(lib, n):
    """moe_lora_align_view (host only) points at the same align regions as
    moe_lora_workspace_view, and refuses a null workspace or output."""
    s = shape_of(synth.WORKLOADS[n])
    v = lm.moe_lora_workspace_view(s, _fake_ws())
    a = lm.moe_lora_align_view(s, FAKE_BASE)
    for name in lm.ALIGN_VIEW_FIELDS:
        assert a[name] == getattr(v, name), name
    assert lib.moe_lora_align_view(ctypes.byref(s), None, ctypes.byref(lm.moe_lora_align_ptrs())) == \
        lm.MOE_LORA_EINVAL
    assert lib.moe_lora_align_view(ctypes.byref(s), FAKE_BASE, None) == lm.MOE_LORA_EINVAL
    bad = lm.make_shape(4, 64, 32, 4, 2, 2, 12)
    assert lib.moe_lora_align_view(ctypes.byref(bad), FAKE_BASE, ctypes.byref(lm.moe_lora_align_ptrs())) == \
        lm.MOE_LORA_EUNSUPPORTED


@pytest.mark.parametrize("I,split", [(2048, False), (4088, False), (4096, True), (25600, True)])
def test_h_lo_region_from_4096(lib, I, split):
    """From I = 4096 on the workspace holds h's bf16 remainder beside h."""
    s = lm.make_shape(32, 512, I, 4, 2, 2, 16)
    v = lm.moe_lora_workspace_view(s, _fake_ws())
    assert bool(v.h_lo) == split
    if split:
        assert v.h_lo % 256 == 0 and v.h_lo >= v.h + v.cap_rows * I * 2
        assert v.d >= v.h_lo + v.cap_rows * I * 2


def test_operand_checks_refuse_before_launch():
    """Wrong dtypes, shapes, non-contiguous or host tensors are refused with
    ValueError before anything is launched (CPU tensors: the device check
    comes last, so dtype and shape errors are seen first)."""
    torch = pytest.importorskip("torch")
    T, H, I, E, k, L, r = 6, 64, 32, 4, 2, 3, 8
    shape = lm.make_shape(T, H, I, E, k, L, r)
    bf = torch.bfloat16
    ok = dict(x=torch.zeros(T, H, dtype=bf), topk_ids=torch.zeros(T, k, dtype=torch.int32),
              topk_weights=torch.zeros(T, k), lora_ids=torch.zeros(T, dtype=torch.int32),
              W_gu=torch.zeros(E, 2 * I, H, dtype=bf), W_down=torch.zeros(E, H, I, dtype=bf),
              A_gu=torch.zeros(L, E, r, H, dtype=bf), B_gu=torch.zeros(L, E, 2 * I, r, dtype=bf),
              A_down=torch.zeros(L, E, r, I, dtype=bf), B_down=torch.zeros(L, E, H, r, dtype=bf))
    ws = torch.zeros(lm.moe_lora_workspace_bytes(shape), dtype=torch.uint8)
    y = torch.zeros(T, H, dtype=bf)

    def forward(**over):
        a = dict(ok, **over)
        lm.moe_lora_forward(shape, a["x"], a["topk_ids"], a["topk_weights"], a["lora_ids"], a["W_gu"],
                            a["W_down"], a["A_gu"], a["B_gu"], a["A_down"], a["B_down"], ws, y)

    cases = [
        (dict(topk_ids=ok["topk_ids"].long()), "topk_ids: dtype int64"),      # torch.topk's dtype
        (dict(lora_ids=ok["lora_ids"].long()), "lora_ids: dtype int64"),
        (dict(topk_weights=ok["topk_weights"].half()), "topk_weights: dtype float16"),
        (dict(x=ok["x"].float()), "x: dtype float32"),
        (dict(W_down=torch.zeros(E, H, I - 8, dtype=bf)), "W_down: shape"),
        (dict(B_gu=torch.zeros(L, E, I, r, dtype=bf)), "B_gu: shape"),
        (dict(B_down=torch.zeros(L - 1, E, H, r, dtype=bf)), "B_down: shape"),
        (dict(x=torch.zeros(H, T, dtype=bf).t()), "x must be contiguous"),
        ({}, "device tensors"),
    ]
    for over, msg in cases:
        with pytest.raises(ValueError, match=msg):
            forward(**over)
    with pytest.raises(ValueError, match="topk_ids: dtype int64"):
        lm.moe_lora_align(shape, ok["topk_ids"].long(), ok["lora_ids"], ws)
    with pytest.raises(ValueError, match="workspace holds"):
        lm.moe_lora_align(shape, ok["topk_ids"], ok["lora_ids"], ws[:16])
    with pytest.raises(ValueError, match="dtype int64"):
        lm.fused_moe_lora(ok["x"], ok["topk_ids"].long(), ok["topk_weights"], ok["lora_ids"],
                          ok["W_gu"], ok["W_down"], ok["A_gu"], ok["B_gu"], ok["A_down"], ok["B_down"])
    with pytest.raises(ValueError, match="logits: shape"):
        lm.moe_lora_route(shape, torch.zeros(T, E + 1), ok["topk_ids"], ok["topk_weights"])


def test_kernel_knob_validation(lib):
    """Kernel configuration fields: 0 or an allowed value, else EINVAL; the
    down-GEMM K split shows in the workspace view (streaming family only)."""
    base = dict(T=40, H=256, I=512, E=4, topk=2, L=2, r=32)
    ok = [dict(shrink_splits=64), dict(shrink_zblocks=4), dict(shrink_zblocks=2), dict(down_splits=8), dict(down_splits=64),
          dict(tile_order=2), dict(expand_mode=1), dict(expand_mode=2)]
    bad = [dict(shrink_splits=65), dict(shrink_splits=-1), dict(shrink_zblocks=3), dict(shrink_zblocks=8),
           dict(down_splits=65), dict(tile_order=3), dict(expand_mode=3), dict(expand_mode=-1)]
    for k in ok:
        assert lm.moe_lora_workspace_bytes(lm.make_shape(**base, **k)) > 0, k
    for k in bad:
        s = lm.make_shape(**base, **k)
        assert lm.moe_lora_resolve_block_m(s) == lm.MOE_LORA_EINVAL, k
        assert lm.moe_lora_workspace_bytes(s) == 0, k
    v = lm.moe_lora_workspace_view(lm.make_shape(**base, block_m=16, down_splits=3), _fake_ws())
    assert v.d_splits == 3
    v = lm.moe_lora_workspace_view(lm.make_shape(**base, block_m=128, down_splits=3), _fake_ws())
    assert v.d_splits == 1  # the tiled down GEMM does not split K
    with pytest.raises(TypeError):
        lm.make_shape(**base, no_such_knob=1)


def test_tune_apply_fills_knobs(lib):
    """moe_lora_tune_apply copies block_m and the knobs of the nearest entry
    into the fields the shape leaves at 0."""
    decode = lm.make_shape(16, 4096, 11008, 8, 2, 8, 32)
    table = (lm.moe_lora_tune_entry * 1)(lm.moe_lora_tune_entry(4, 4096, 11008, 8, 32, 8, 16, 4, 2, 3, 0, 1))
    out = lm.moe_lora_tune_apply(decode, (table, 1))
    assert (out.block_m, out.shrink_splits, out.shrink_zblocks, out.down_splits, out.tile_order,
            out.expand_mode) == (16, 4, 2, 3, 0, 1)
    own = lm.make_shape(16, 4096, 11008, 8, 2, 8, 32, shrink_splits=7)
    assert lm.moe_lora_tune_apply(own, (table, 1)).shrink_splits == 7
    assert lm.make_shape(16, 4096, 11008, 8, 2, 8, 32, tuning=(table, 1)).down_splits == 3
    # an entry whose knobs do not fit the shape leaves it unchanged (r = 8: 2 z blocks invalid)
    small = lm.make_shape(16, 4096, 11008, 8, 2, 8, 8)
    t2 = (lm.moe_lora_tune_entry * 1)(lm.moe_lora_tune_entry(4, 4096, 11008, 8, 8, 8, 16, 0, 2, 0, 0))
    assert lm.moe_lora_tune_apply(small, (t2, 1)).shrink_zblocks == 0
