"""Plant plausible mistakes in a copy of the oracle and check that the pins catch each one.

Every mutant is the oracle source with one small edit (a dropped term, a wrong
sign or index, a flipped comparison), compiled into a temporary library.  The
pin tests of ``test_oracle_pins`` are then run against it; at least one of
them must fail.  This runs on the CPU only.
"""
import os
import subprocess
import tempfile

import pytest

import oracle
from tests import test_oracle_filter_pins as fpins
from tests import test_oracle_pins as pins
from tests import test_oracle_tree_pins as tpins

SRC = oracle.oracle.SRC

MUTANTS = {
    "residual_abs_instead_of_max": ("w[v] = diff > 0.0 ? diff : 0.0;", "w[v] = diff > 0.0 ? diff : -diff;"),
    "residual_sign_flipped": ("double diff = prob(&rp, &sp[k], v) - prob(&rq, &sq[k], v);",
                              "double diff = prob(&rq, &sq[k], v) - prob(&rp, &sp[k], v);"),
    "accept_non_strict": ("if (!(u < ai)) { k = i; break; }", "if (!(u <= ai)) { k = i; break; }"),
    "no_break_at_first_reject": ("if (!(u < ai)) { k = i; break; }", "if (!(u < ai)) { k = i; }"),
    "ratio_inverted": ("double ratio = px / qx;", "double ratio = qx / px;"),
    "no_fallback": ("if (Z == 0.0) { /* fallback to p_k */", "if (0) { /* fallback to p_k */"),
    "argmax_last_tie": ("if (z > bz) { /* strict", "if (z >= bz) { /* strict"),
    "temperature_ignored": ("if (z >= st.tau) st.s += exp((z - st.m) / T);", "if (z >= st.tau) st.s += exp((z - st.m));"),
    "inverse_cdf_non_strict": ("if (target < acc) {", "if (target <= acc) {"),
    "inverse_cdf_unnormalised": ("double target = u * Z;", "double target = u;"),
    "bonus_from_previous_row": ("row_t rp = target_row(a->target, dt, gamma, V, b, k);\n        if (k < g) {",
                                "row_t rp = target_row(a->target, dt, gamma, V, b, k < g ? k : (k > 0 ? k - 1 : 0));\n        if (k < g) {"),
    "greedy_uses_draft_row": ("row_t r = target_row(a->target, dt, gamma, V, b, i);\n            tmax[i]",
                              "row_t r = (i < g) ? draft_row(a->draft, dt, gamma, V, b, i) : target_row(a->target, dt, gamma, V, b, i);\n            tmax[i]"),
    "draft_row_shifted": ("row_t rq = draft_row(a->draft, dt, gamma, V, b, i);\n            double px",
                          "row_t rq = draft_row(a->draft, dt, gamma, V, b, i + 1 < g ? i + 1 : i);\n            double px"),
    "topk_off_by_one": ("double tau_k = use_k ? zs[top_k - 1] : -INFINITY;",
                        "double tau_k = use_k ? zs[top_k] : -INFINITY;"),
    "topp_over_full_mass": ("if (zs[v] >= tau_k) Fk += exp", "if (1) Fk += exp"),
    "draft_rows_unfiltered": ("sq[i] = softmax_stats(&r, T, tk, tp);", "sq[i] = softmax_stats(&r, T, 0, 1.0);"),
    "prob_ignores_cut": ("if (z < st->tau) return 0.0;", "if (0) return 0.0;"),
    "sum_ignores_cut": ("if (z >= st.tau) st.s += exp((z - st.m) / T);", "st.s += exp((z - st.m) / T);"),
    "topp_first_group_kept_only": ("if (cum >= target) {", "if (1) {"),
    "tree_residual_not_updated": ("cur[v] = d > 0.0 ? d : 0.0;\n                Z += cur[v];",
                                  "Z += d > 0.0 ? d : 0.0;"),
    "tree_residual_from_p": ("double d = cur[v] - q[v];", "double d = p[v] - q[v];"),
    "tree_target_row_shifted": ("row_t rp = {a->target, dt, ((size_t)b * (size_t)(Nmax + 1) + (size_t)pos) * (size_t)V, V};",
                                "row_t rp = {a->target, dt, ((size_t)b * (size_t)(Nmax + 1) + (size_t)(pos > 0 ? pos - 1 : 0)) * (size_t)V, V};"),
    "tree_last_sibling_first": ("for (int n = pos; n < N && hit < 0; ++n) {", "for (int n = N - 1; n >= pos && hit < 0; --n) {"),
    "cdf_band_in_probability_units": ("if (m < BAND) flags |= 2;", "if (m * Zrep < BAND) flags |= 2;"),
    "cdf_band_normalised_only": ("else if (m * Zrep < BAND) flags |= 16;", "else if (0) flags |= 16;"),
    "tree_greedy_no_descent": ("if (parent[n] == pos - 1 && token[n] == am) { hit = n; break; }",
                               "if (parent[n] == -1 && token[n] == am) { hit = n; break; }"),
}

PIN_TESTS = [
    (pins.test_t1_exact_enumeration_position0, {}),
    (pins.test_t1_exact_enumeration_later_position, {}),
    (pins.test_t1_bonus_marginal, {}),
    (pins.test_t1_exact_integration_random_distributions, {"seed": 0, "T": 0.6}),
    (pins.test_t2_accepted_run_law_and_expected_tokens, {"gamma": 3}),
    (pins.test_t3_greedy_worked_example, {}),
    (pins.test_t4_library_cross_checks, {"dtype": "f32"}),
    (pins.test_t4_argmax_matches_numpy_with_ties, {}),
    (pins.test_t5_u_zero_accepts_and_strict_comparison, {}),
    (pins.test_t5_zero_residual_mass_falls_back_to_p, {}),
    (pins.test_t5_inverse_cdf_is_strict_at_exact_breakpoints, {}),
    (pins.test_t5_identical_rows_accept_everything, {}),
    (pins.test_flag_bits_normalised_band_and_probability_units, {"side": 1.0}),
    (fpins.test_f1_filter_matches_brute_force_definition, {"coarse": True}),
    (fpins.test_f2_exact_integration_gives_filtered_target, {"seed": 0, "top_k": 6, "top_p": 0.9}),
    (fpins.test_f4_three_token_top_p_cut, {}),
    (fpins.test_f4_ties_at_the_top_k_cut_are_kept, {}),
    (tpins.test_tr1_chain_is_the_linear_method, {"dtype": "f32", "T": 1.0}),
    (tpins.test_tr2_exact_integration_first_token_is_p, {"m": 3, "seed": 0}),
    (tpins.test_tr3_sibling_order_and_residual_chain, {}),
    (tpins.test_tr4_greedy_tree, {}),
]


class _MutantOracle:
    """Same call surface as the ``oracle`` package, bound to a mutant build."""

    def __init__(self, lib):
        self._lib = lib

    def spec_verify(self, *a, **k):
        return oracle.spec_verify(*a, lib=self._lib, **k)

    def run_workload(self, w, trace=True):
        return oracle.run_workload(w, trace=trace, lib=self._lib)

    def spec_verify_tree(self, *a, **k):
        return oracle.spec_verify_tree(*a, lib=self._lib, **k)


def test_mutation_sources_apply():
    src = open(SRC).read()
    for name, (old, new) in MUTANTS.items():
        assert src.count(old) == 1, name


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_mutant(name, tmp_path):
    old, new = MUTANTS[name]
    src = open(SRC).read()
    assert src.count(old) == 1
    msrc = tmp_path / "mutant.c"
    msrc.write_text(src.replace(old, new))
    lib_path = str(tmp_path / f"libmutant_{name}.so")
    oracle.build(src=str(msrc), out=lib_path)
    mo = _MutantOracle(oracle.load(lib_path))
    caught = []
    for fn, kw in PIN_TESTS:
        try:
            fn(mo, **kw)
        except (AssertionError, ValueError, IndexError):
            caught.append(fn.__name__)
    assert caught, f"mutant {name} survived every pin"
