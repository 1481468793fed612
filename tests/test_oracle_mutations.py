"""The oracle's pins must catch plausible mistakes.

Each mutation below plants one slip in a copy of oracle/oracle.c (on the
CPU, in a temporary directory), builds it, and runs the pin suite
(tests/test_oracle.py) against it in a subprocess; the suite must fail.
"""
import os
import subprocess
import sys

import pytest

import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "oracle.c")

MUTATIONS = {
    "accept_with_less_equal": ("if (n == d && !((double)u_accept[b * K + k] < ratio))",
                               "if (n == d && !((double)u_accept[b * K + k] <= ratio))"),
    "residual_sign_flipped": ("double d = p[v] - q[v];", "double d = q[v] - p[v];"),
    "bonus_from_row_K": ("row_ptr(target, dtype, b * (K + 1) + d, V),\n                                     NULL",
                         "row_ptr(target, dtype, b * (K + 1) + K, V),\n                                     NULL"),
    "temperature_dropped": ("S += exp((logit_at(row, dtype, v) - M) / T);",
                            "S += exp((logit_at(row, dtype, v) - M));"),
    "inverse_cdf_greater_equal": ("if (acc > target) return v;", "if (acc >= target) return v;"),
    "argmax_highest_index_on_ties": ("if (z > bv) { bv = z; best = v; }", "if (z >= bv) { bv = z; best = v; }"),
    "last_rejection_not_first": ("if (n == d && !((double)u_accept", "if (!((double)u_accept"),
    "dcut_tie_reversed": ("return (a->flat < b->flat) ? -1 : (a->flat > b->flat);",
                          "return (a->flat > b->flat) ? -1 : (a->flat < b->flat);"),
    "dcut_no_floor": ("depth_out[b] = Kb > 0 ? 1 : 0;", "depth_out[b] = 0;"),
    "residual_no_fallback": ("if (R == 0.0) {\n        memcpy(r, p,", "if (R < 0.0) {\n        memcpy(r, p,"),
    "greedy_bonus_from_row_n_plus_1": ("b * (K + 1) + n, V), dtype, V);\n    for (int32_t k = 0; k <= K; ++k) out_row[k] = -1;",
                                       "b * (K + 1) + (n < d ? n + 1 : n), V), dtype, V);\n    for (int32_t k = 0; k <= K; ++k) out_row[k] = -1;"),
    "confidence_not_inverse": ("(float)(1.0 / S)", "(float)(S)"),
    # early-exit verification
    "ee_accept_with_less_equal": ("if (!((double)u_accept[b * K + k] < ratio)) { n = k; break; }",
                                  "if (!((double)u_accept[b * K + k] <= ratio)) { n = k; break; }"),
    "ee_sampled_reads_past_stop": ("if (!((double)u_accept[b * K + k] < ratio)) { n = k; break; }",
                                   "if (!((double)u_accept[b * K + k] < ratio) && n == d) n = k;"),
    "ee_greedy_reads_past_stop": ("if ((int64_t)tok[k] != g) { n = k; emit = g; break; }",
                                  "if ((int64_t)tok[k] != g && n == d) { n = k; emit = g; }"),
    "ee_greedy_bonus_row_unchecked": ("if (row_check(zr, dtype, V) != ROW_OK) bad = 1;\n                else emit",
                                      "if (0) bad = 1;\n                else emit"),
    "ee_draw_uniform_unchecked": ("if (!bad && bad_uniform(u_sample[b])) bad = 1;", "if (0) bad = 1;"),
    # temperature range and large logits
    "softmax_without_max_shift": ("    double M = -INFINITY;\n    for (int64_t v = 0; v < V; ++v) {\n"
                                  "        double z = logit_at(row, dtype, v);\n        if (z > M) M = z;\n    }",
                                  "    double M = 0.0;"),
    "temperature_floor_1e_6": ("(T > 0.0f && isfinite(T))", "(T >= 1e-6f && isfinite(T))"),
    # cost-aware D-cut
    "cost_segment_start_shifted": ("return tcost[above - 1] + w * (tcost[above] - tcost[above - 1]);",
                                   "return tcost[above] + w * (tcost[above] - tcost[above - 1]);"),
    "cost_bid_ties_to_largest_depth": ("if (d == 1 || v > value[b])", "if (d == 1 || v >= value[b])"),
    "cost_offer_lowest_value_first": ("(best < 0 || value[b] > value[best])", "(best < 0 || value[b] < value[best])"),
    "cost_unfit_bid_ends_offer": ("        if (spent + c <= max_verify) {\n            spent = spent + c;",
                                  "        if (!(spent + c <= max_verify)) break;\n        {\n            spent = spent + c;"),
}


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_mutation_is_caught(name, tmp_path):
    old, new = MUTATIONS[name]
    src = open(SRC).read()
    assert src.count(old) == 1, f"mutation anchor for {name} not found exactly once"
    mutated = tmp_path / "oracle_mut.c"
    mutated.write_text(src.replace(old, new))
    lib = oracle.compile_to(str(mutated), str(tmp_path / "liboracle_mut.so"))
    env = dict(os.environ, ORACLE_LIB=lib)
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_oracle.py")],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    assert r.returncode != 0, f"pins did not catch mutation {name}:\n{r.stdout[-2000:]}"


def test_unmutated_copy_passes(tmp_path):
    # Control: the same harness on an unmodified copy must pass, so the
    # failures above come from the planted slips and nothing else.
    lib = oracle.compile_to(SRC, str(tmp_path / "liboracle_copy.so"))
    env = dict(os.environ, ORACLE_LIB=lib)
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_oracle.py")],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, r.stdout[-2000:]
