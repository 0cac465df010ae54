"""The oracle's pins must catch plausible mistakes.

Each case plants one mistake in a copy of oracle.c (on the CPU, in a temporary
directory), builds it, and runs the pin tests against that copy: at least one
pin must fail.  The shipped oracle is untouched.
"""
import os
import subprocess
import tempfile

import pytest

import oracle
from tests import test_oracle_balance as B
from tests import test_oracle_fp8 as Q
from tests import test_oracle_ffn as F
from tests import test_oracle_permute as P
from tests import test_oracle_selection as S
from tests import test_oracle_sigmoid as G
from tests import test_oracle_v4 as V

SRC = os.path.join(os.path.dirname(oracle.__file__), "oracle.c")

MUTANTS = {
    "group score from the best expert twice": ("gscore[g] = score[best] + score[second];",
                                               "gscore[g] = score[best] + score[best];"),
    "routed scaling factor dropped": ("w[j] = (L->renorm ? s / sum : s) * L->scale;",
                                      "w[j] = (L->renorm ? s / sum : s);"),
    "ties to the higher index": ("return va > vb || (va == vb && ia < ib);",
                                 "return va > vb || (va == vb && ia > ib);"),
    "silu applied to the up projection": ("hbuf[i] = g * sigmoid64(g) * u;", "hbuf[i] = u * sigmoid64(u) * g;"),
    "down projection transposed": ("acc += elem(wd, L->dtype, n * I + i) * hbuf[i];",
                                   "acc += elem(wd, L->dtype, i * H + n) * hbuf[i];"),
    "shared expert not added": ("for (int64_t n = 0; n < H; ++n) o[n] += y[n];",
                                "for (int64_t n = 0; n < H; ++n) o[n] += 0.0 * y[n];"),
    "capacity off by one": ("if (count[e] < cap) {\n          idx[t * k + got++] = e;",
                            "if (count[e] <= cap) {\n          idx[t * k + got++] = e;"),
    "drop mode re-routes the overflow": ("  } else if (L->drop_tokens) {", "  } else if (0) {"),
    "drop mode lets one token too many in": ("if (count[e] < cap) {\n          count[e] += 1;",
                                             "if (count[e] <= cap) {\n          count[e] += 1;"),
    "drop mode keeps the dropped gate": ("idx[t * k + j] = -1;\n          w[t * k + j] = 0.0;",
                                         "idx[t * k + j] = -1;"),
    "unnormalised softmax over the selection": ("w[j] = (L->renorm ? p / z_sel : p / z_all) * L->scale;",
                                                "w[j] = (L->renorm ? p / z_sel : p / z_sel) * L->scale;"),
    "strided groups": ("if (kept[e / gsz]) order[n_allowed++] = e;", "if (kept[e % G]) order[n_allowed++] = e;"),
    "ln2 low part dropped": ("r = fmaf(-n, EXP32_LN2_LO, r);", "r = r;"),
    "logit bias ignored": ("if (logit_bias) acc += (double)logit_bias[e];", "(void)logit_bias;"),
    "gates from the biased score": ("double s = gate_score64(L, logit[idx[j]]);\n      w[j]",
                                    "double s = gate_score64(L, logit[idx[j]]) + 0.01 * j;\n      w[j]"),
    "log1p series not doubled": ("float z2 = z + z;", "float z2 = z;"),
    "softplus without its linear part": ("float sp = (l > 0.0f ? l : 0.0f) + log1p32_unit(u);",
                                         "float sp = 0.0f + log1p32_unit(u);"),
    "sqrt(softplus) without the clamp": ("  if (a > 80.0f) a = 80.0f;\n  float u", "  float u"),
    "sqrt(softplus) gates from the sigmoid": (
        "return L->scoring == 2 ? sqrtsoftplus64((double)l) : sigmoid64((double)l);",
        "return sigmoid64((double)l);"),
    "sqrt(softplus) selection without the square root": (
        "float s = L->scoring == 1 ? oracle_sigmoid32(logit[e]) : oracle_sqrtsoftplus32(logit[e]);",
        "float s = L->scoring == 1 ? oracle_sigmoid32(logit[e]) : logit[e];"),
    "hash table read transposed": ("e = tid2eid[id * k + j];", "e = tid2eid[j * vocab + id];"),
    "hash routing keeps repeated entries": ("if (tid2eid[id * k + i] == e) e = -1;", "if (0) e = -1;"),
    "hash routing reads negative ids as row 0": ("const int64_t id = token_ids[t];",
                                                 "const int64_t id = token_ids[t] < 0 ? 0 : token_ids[t];"),
    "hash drop mode lets one token too many in": ("if (held[e] >= cap) {", "if (held[e] > cap) {"),
    "fp8 tile scale rounded down": ("int p = E - 8 + (M > 1.75 ? 1 : 0);", "int p = E - 8;"),
    "fp8 rounding truncates": ("const double q = nearbyint(a / spacing);", "const double q = floor(a / spacing);"),
    "e4m3 subnormals one binade low": ("ldexp((double)m, -9) : ldexp((double)(8 + m), e - 10);",
                                       "ldexp((double)m, -10) : ldexp((double)(8 + m), e - 10);"),
    "fp8 weight scale of the first column block only": (
        "oracle_e8m0_value(scales[(row / 128) * (cols / 128) + col / 128]);",
        "oracle_e8m0_value(scales[(row / 128) * (cols / 128)]);"),
    "fp8 h not quantised": (
        "acc += fp8_weight(wd, sd, I, n, i) * oracle_e4m3_value(hcodes[i]) * oracle_e8m0_value(hscales[i / 128]);",
        "acc += fp8_weight(wd, sd, I, n, i) * (double)hbuf[i];"),
    "fp8 x not quantised": ("xq[h] = oracle_e4m3_value(xc[h]) * oracle_e8m0_value(xs[h / 128]);", "xq[h] = xf[h];"),
    "fp8 quantised zero loses its sign": ("if (r == 0.0) return sign;", "if (r == 0.0) return 0;"),
    "group limit keeps one group too many": ("for (int i = 0; i < L->topk_group; ++i) kept[gid[i]] = 1;",
                                             "for (int i = 0; i <= L->topk_group && i < G; ++i) kept[gid[i]] = 1;"),
    "permutation in descending token order": ("for (int e = 0; e < E; ++e) fill[e] = offsets[e];\n  for (int64_t t = 0; t < T; ++t) {",
                                              "for (int e = 0; e < E; ++e) fill[e] = offsets[e];\n  for (int64_t t = T - 1; t >= 0; --t) {"),
    "balancing pushes experts at the mean": ("if (N > 0 && scaled > N) {", "if (N > 0 && scaled >= N) {"),
    "balancing with the sign reversed": ("bias[e] = bias[e] - gamma;", "bias[e] = bias[e] + gamma;"),
    "entropy in bits": ("if (p > 0.0) ent -= p * log(p);", "if (p > 0.0) ent -= p * log2(p);"),
    "expert gate weight ignored": ("for (int64_t n = 0; n < H; ++n) o[n] += w[t * k + j] * y[n];",
                                   "for (int64_t n = 0; n < H; ++n) o[n] += y[n];"),
}

PINS = [
    G.test_exp32_within_2ulp_of_double_exp, G.test_sigmoid32_closed_forms,
    S.test_group_whose_best_expert_is_global_max_but_pair_sum_loses_is_dropped,
    S.test_bias_changes_selection_but_not_gates, S.test_sigmoid_gates_closed_form,
    S.test_softmax_gates_closed_form, S.test_ties_go_to_lower_index, S.test_softmax_gates_match_library_softmax,
    S.test_v3_gates_sum_to_scaling_factor, S.test_router_logits_are_the_fp32_rounded_matmul_plus_bias,
    lambda: S.test_capacity_matches_sequential_simulation(8, 1, 1, 2, 1.0, "softmax"),
    S.test_drop_mode_hand_example,
    lambda: S.test_drop_mode_is_the_unlimited_top_k_minus_late_assignments(8, 1, 1, 2, 0.75, "softmax"),
    lambda: S.test_selection_matches_exhaustive_enumeration(16, 4, 2, 3, "sigmoid"),
    P.test_hand_example,
    V.test_sqrtsoftplus32_within_2ulp_of_double, V.test_sqrtsoftplus32_closed_forms,
    V.test_without_bias_selection_is_the_top_k_of_the_logits, V.test_gates_closed_form,
    V.test_bias_changes_selection_but_not_gates, V.test_hash_routing_hand_example,
    V.test_hash_routing_follows_the_table_whatever_the_logits,
    V.test_hash_routing_drop_mode_keeps_the_first_c_assignments,
    Q.test_e4m3_decode_hand_values, Q.test_quantize_hand_tiles,
    lambda: Q.test_quantize_matches_torch_rounding_and_minimal_scale(0),
    Q.test_fp8_layer_matches_block_expansion_with_library_rounding,
    Q.test_fp8_layer_with_exact_inputs_is_the_bf16_layer_up_to_h_rounding,
    B.test_loads_at_the_mean_keep_their_bias, B.test_random_loads_against_library_entropy_and_float32_steps,
    F.test_swiglu_closed_form_with_selection_matrices, F.test_single_expert_layer_is_a_dense_swiglu_ffn,
    F.test_identical_experts_factor_out, F.test_empty_slots_are_skipped_and_bf16_inputs_are_exact,
]


def _first_failing_pin():
    for pin in PINS:
        try:
            pin()
        except (AssertionError, ValueError):
            return pin
    return None


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_planted_mistake_is_caught(name, tmp_path):
    old, new = MUTANTS[name]
    src = open(SRC).read()
    assert src.count(old) == 1, "mutation anchor must match exactly once"
    path = tmp_path / "oracle_mutant.c"
    path.write_text(src.replace(old, new))
    lib = tmp_path / "liboracle_mutant.so"
    subprocess.check_call(["gcc", "-O2", "-fPIC", "-shared", "-fopenmp", "-ffp-contract=off", "-std=gnu11",
                           "-o", str(lib), str(path), "-lm"])
    oracle.use_library(str(lib))
    try:
        assert _first_failing_pin() is not None, "no pin caught: " + name
    finally:
        oracle.use_library(None)


def test_unmodified_oracle_passes_every_pin():
    assert _first_failing_pin() is None
