"""The oracle's pins catch plausible mistakes.

Each case copies the oracle's C source, plants one plausible mistake by text
substitution, builds the copy into a temporary library on the CPU, swaps it in
for the real one and runs the pin tests. At least one pin must fail for every
mutant; the unmodified source must pass them all.
"""
import ctypes as C
import os

import pytest

import oracle
from oracle import build as obuild
import test_oracle_ffn as F
import test_oracle_route_group as R

SRC = obuild.SRC

MUTANTS = {
    "tie_to_higher_index": ("    return a < b;\n}\n\n/* Top-k", "    return a > b;\n}\n\n/* Top-k"),
    "gate_sum_drops_a_term": ("for (int j = 0; j < k; ++j) sum +=", "for (int j = 1; j < k; ++j) sum +="),
    "group_not_stable": ("for (int f = 0; f < A_routed; ++f) {          /* ascending",
                         "for (int f = A_routed - 1; f >= 0; --f) {          /* ascending"),
    "code_bit_order_reversed": ("(codes[8 * b + j / 4] >> (2 * (j % 4)))",
                                "(codes[8 * b + j / 4] >> (2 * (3 - j % 4)))"),
    "code_byte_index": ("codes[8 * b + j / 4]", "codes[8 * b + j / 8]"),
    "affine_offset_dropped": ("w[32 * b + j] = d * (acc_t)q + m;", "w[32 * b + j] = d * (acc_t)q;"),
    "high_bit_weight": ("& 1) << 2;", "& 1) << 1;"),
    "silu_sign": ("exp(-(double)z)", "exp((double)z)"),
    "swiglu_operands_swapped": ("h[r] = silu(g) * u;", "h[r] = silu(u) * g;"),
    "gate_uses_up_scales": ("dm + 2 * bg, H, wrow);", "dm + 2 * bu, H, wrow);"),
    "combine_ignores_gates": ("yt[c] += gate * o[c];", "yt[c] += o[c];"),
    "shared_expert_dropped": ("int n_terms = k + (has_shared ? 1 : 0);", "int n_terms = k;"),
    "down_rows_strided_wrong": ("size_t bd = dn0 + (size_t)r * bpr_d;",
                                "size_t bd = dn0 + (size_t)r * bpr_gu % (3 * bpr_d);"),
}

# (callable, args) pins to run against a mutant
PINS = [
    (R.test_topk_ties_go_to_lower_index, ()),
    (R.test_all_equal_logits, ()),
    (R.test_gates_equal_full_softmax_renormalised, ()),
    (R.test_gates_closed_form_two_experts, ()),
    (R.test_grouping_invariants, (1024, 512, 10, 1)),
    (F.test_dequant_constant_cases, ("f64",)),
    (F.test_dequant_planted_code, (5,)),
    (F.test_dequant_planted_code, (30,)),
    (F.test_dequant_blocks_use_their_own_scale, ()),
    (F.test_expert_forward_matches_matrices, ()),
    (F.test_constant_weights_closed_form, ()),
    (F.test_layer_matches_dense_f64, (F.small_cfg(2),)),
    (F.test_layer_matches_dense_f64, (F.small_cfg(3),)),
]


def run_pins():
    failed = []
    for fn, args in PINS:
        try:
            fn(*args)
        except AssertionError:
            failed.append(fn.__name__)
        except Exception as exc:  # a crash in a mutant also counts as caught
            failed.append(f"{fn.__name__}:{type(exc).__name__}")
    return failed


@pytest.fixture
def swap_lib(monkeypatch, tmp_path):
    def load(src_text: str):
        src = tmp_path / "mut.c"
        src.write_text(src_text)
        lib = obuild.build(src=str(src), lib=str(tmp_path / "libmut.so"))
        monkeypatch.setattr(oracle, "_lib", oracle.bind(C.CDLL(os.path.abspath(lib))))
    return load


def test_unmodified_source_passes_all_pins(swap_lib):
    swap_lib(open(SRC).read())
    assert run_pins() == []


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name, swap_lib):
    text = open(SRC).read()
    old, new = MUTANTS[name]
    assert text.count(old) == 1, f"mutation anchor for {name} not unique"
    swap_lib(text.replace(old, new))
    assert run_pins(), f"no pin caught mutant {name}"
