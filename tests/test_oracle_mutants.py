"""Plant plausible mistakes in copies of the fp64 reference (CPU only) and
check that every copy fails at least one pin.  This shows the pins can tell a
correct reference from a wrong one: a dropped term, a wrong sign, a transposed
operand, a wrong index or a wrong sort order each get caught."""
import os

import pytest

import oracle
import pins

SRC = open(os.path.join(os.path.dirname(oracle.__file__), "moe_lora_oracle.c")).read()

# (name, text in the reference, replacement)
MUTANTS = [
    ("drop_gate_up_lora", "g[n] += P->s * acc;", "g[n] += 0.0 * acc;"),
    ("drop_down_lora", "d[m] += P->s * acc;", "d[m] += 0.0 * acc;"),
    ("ignore_scale_gate_up", "g[n] += P->s * acc;", "g[n] += acc;"),
    ("ignore_scale_down", "d[m] += P->s * acc;", "d[m] += acc;"),
    ("transpose_B_gu", "acc += zg[q] * bf(B[(size_t)n * r + q]);",
     "acc += zg[q] * bf(B[(size_t)q * 2 * I + n]);"),
    ("transpose_B_down", "acc += zd[q] * bf(B[(size_t)m * r + q]);",
     "acc += zd[q] * bf(B[(size_t)q * H + m]);"),
    ("transpose_W_down", "acc += h[i] * bf(Wd[(size_t)m * I + i]);",
     "acc += h[i] * bf(Wd[(size_t)i * H + m]);"),
    ("swap_gate_up", "h[i] = silu(g[i]) * g[I + i];", "h[i] = silu(g[I + i]) * g[i];"),
    ("silu_sign", "return v / (1.0 + exp(-v));", "return v / (1.0 + exp(v));"),
    ("sigmoid_not_silu", "return v / (1.0 + exp(-v));", "return 1.0 / (1.0 + exp(-v));"),
    ("ignore_topk_weight", "yr[m] += w * d[m];", "yr[m] += d[m];"),
    ("slab_index_e_l", "const uint16_t* A = P->A_gu + ((size_t)l * E + e) * r * H;",
     "const uint16_t* A = P->A_gu + ((size_t)e * P->L + l) * r * H;"),
    ("down_slab_wrong_expert", "const uint16_t* B = P->B_down + ((size_t)l * E + e) * H * r;",
     "const uint16_t* B = P->B_down + ((size_t)l * E + (e + 1) % E) * H * r;"),
    ("none_means_adapter0", "return (l >= 0 && l < P->L) ? l : -1;",
     "return (l >= 0 && l < P->L) ? l : 0;"),
    ("shrink_skips_first", "for (int i = 0; i < H; ++i) acc += bf(xr[i]) * bf(A[(size_t)q * H + i]);",
     "for (int i = 1; i < H; ++i) acc += bf(xr[i]) * bf(A[(size_t)q * H + i]);"),
    ("down_shrink_uses_gate", "for (int i = 0; i < I; ++i) acc += h[i] * bf(A[(size_t)q * I + i]);",
     "for (int i = 0; i < I; ++i) acc += g[i] * bf(A[(size_t)q * I + i]);"),
    ("clamp_bad_expert", "return (e >= 0 && e < P->E) ? e : -1;",
     "return e < 0 ? 0 : (e >= P->E ? P->E - 1 : e);"),
    # align
    ("align_reverse_order", "for (int p = 0; p < P; ++p) {\n    int e = topk_ids[p];\n    if (e < 0 || e >= E) { pos_of_pair[p] = -1; continue; }",
     "for (int p = P - 1; p >= 0; --p) {\n    int e = topk_ids[p];\n    if (e < 0 || e >= E) { pos_of_pair[p] = -1; continue; }"),
    ("align_none_slot_first", "int s = (l >= 0 && l < L) ? l : L;\n    int pos",
     "int s = (l >= 0 && l < L) ? l + 1 : 0;\n    int pos"),
    ("align_no_padding", "int pad = (n_e + block_m - 1) / block_m * block_m;", "int pad = n_e;"),
    ("align_wrong_sentinel", "for (int i = 0; i < cap_rows; ++i) sorted_ids[i] = P;",
     "for (int i = 0; i < cap_rows; ++i) sorted_ids[i] = -1;"),
    ("align_no_lora_errors", "if (!(l >= -1 && l < L)) errs++;", "if (0) errs++;"),
    ("align_block_expert_unset", "block_expert[b] = -1;\n", "block_expert[b] = 0;\n"),
    # router
    ("router_ties_to_higher", "if (best < 0 || (double)lg[e] > (double)lg[best]) best = e;",
     "if (best < 0 || (double)lg[e] >= (double)lg[best]) best = e;"),
    ("router_smallest_first", "if (best < 0 || (double)lg[e] > (double)lg[best]) best = e;",
     "if (best < 0 || (double)lg[e] < (double)lg[best]) best = e;"),
    ("router_full_softmax", "for (int j = 0; j < nch; ++j) sum += exp((double)lg[id[j]] - m);",
     "for (int j = 0; j < E; ++j) sum += exp((double)lg[j] - m);"),
    ("router_unnormalised", "wt[j] = j < nch ? exp((double)lg[id[j]] - m) / sum : 0.0;",
     "wt[j] = j < nch ? exp((double)lg[id[j]] - m) : 0.0;"),
    ("router_chooses_nonfinite", "if (taken[e] || !isfinite(lg[e])) continue;",
     "if (taken[e] || isnan(lg[e])) continue;"),
]


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_mutant_is_caught(tmp_path, name, old, new):
    assert SRC.count(old) == 1, f"mutation site for {name} not found exactly once"
    src = tmp_path / f"{name}.c"
    src.write_text(SRC.replace(old, new))
    so = oracle.compile_to(str(tmp_path / f"lib{name}.so"), str(src))
    orc = oracle.Oracle(so)
    caught = []
    for pin in pins.ALL_PINS:
        try:
            pin(orc)
        except (AssertionError, ValueError, MemoryError) as exc:  # noqa: PERF203
            caught.append((pin.__name__, str(exc).splitlines()[0][:80] if str(exc) else ""))
    assert caught, f"mutant {name} passed every pin"
