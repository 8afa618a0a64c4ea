"""Planted mistakes in copies of the oracle must each fail some pin.

Each mutant is a one-line edit of ``oracle/oracle.c`` of a kind that could
plausibly slip in (an off-by-one row, '<=' for '<', a swapped residual, a
dropped temperature, an epsilon guard copied from tutorial code, ...).  The
copy is compiled with gcc into a temporary directory and the pins of
``test_oracle_pins`` are run against it; the test passes only if every
mutant is caught.  Everything runs on the CPU.
"""
import os

import pytest

import oracle
import test_oracle_bookkeeping as bpins
import test_oracle_draft as dpins
import test_oracle_flags as fpins
import test_oracle_pins as pins
import test_oracle_rows as rpins

SRC = os.path.join(os.path.dirname(oracle.__file__), "oracle.c")

MUTANTS = {
    "accept_le": ("if (!((double)u[i] < alpha))", "if (!((double)u[i] <= alpha))"),
    "draw_ge": ("if (pick < 0 && c > target) pick = v;", "if (pick < 0 && c >= target) pick = v;"),
    "residual_swapped": ("return qr ? fmax(0.0, pr[v] - qr[v]) : pr[v];",
                         "return qr ? fmax(0.0, qr[v] - pr[v]) : pr[v];"),
    "no_temperature": ("double w = exp((orc_decode(rows, dtype, base + v) - m) / T);",
                       "double w = exp((orc_decode(rows, dtype, base + v) - m));"),
    "draw_uses_first_uniform": ("orc_draw(pr, qr, V, u[k],", "orc_draw(pr, qr, V, u[0],"),
    "draw_row_off_by_one": ("const double *pr = P[n];", "const double *pr = P[n > 0 ? n - 1 : 0];"),
    "ratio_transposed": ("double ratio = px / qx;", "double ratio = qx / px;"),
    "epsilon_guard": ("double ratio = px / qx;", "double ratio = px / (qx + 1e-8);"),
    "greedy_tie_highest": ("if (z > best) { best = z; at = v; }", "if (z >= best) { best = z; at = v; }"),
    "greedy_emits_draft": ("orc_write_tokens(out, k, x, n, (int32_t)a);",
                           "orc_write_tokens(out, k, x, n, n < k ? x[n] : (int32_t)a);"),
    "uniform_slot_draft_layout": ("uniforms + trow, qg, out_alpha", "uniforms + drow, qg, out_alpha"),
    "bonus_from_draft_row": ("const double *qr = (n < k) ? Q[n] : NULL;",
                             "const double *qr = (n < k) ? Q[n] : (k > 0 ? Q[k - 1] : NULL);"),
    # drafter-side entry points
    "gathered_q_ignored": ("double px = P[i][x[i]], qx = qg ? (double)qg[i] : Q[i][x[i]];",
                           "double px = P[i][x[i]], qx = Q[i][x[i]];"),
    "gathered_not_checked": ("bad |= !(qg[i] > 0.0f && qg[i] <= 1.0f);", "bad |= 0;"),
    "draft_prob_of_neighbour": ("out_probs[r] = q[t];", "out_probs[r] = q[t > 0 ? t - 1 : t + 1];"),
    "draft_untempered": ("orc_softmax_row(logits, dtype, r, V, T, q, &m, &S);",
                         "orc_softmax_row(logits, dtype, r, V, 1.0, q, &m, &S);"),
    # post-verify bookkeeping and the n-gram drafter
    "commit_drops_emitted": ("int32_t c = out_n[b] >= 0 ? out_n[b] + 1 : 0;",
                             "int32_t c = out_n[b] >= 0 ? out_n[b] : 0;"),
    "adapt_ge": ("if (avg > 0.8)", "if (avg >= 0.8)"),
    "adapt_window_9": ("for (int32_t i = hist_count[b] - 10; i < hist_count[b]; ++i) sum += h[i];",
                       "for (int32_t i = hist_count[b] - 9; i < hist_count[b]; ++i) sum += h[i] * (10.0 / 9.0);"),
    "adapt_rate_k_plus_1": ("(double)out_n[b] / (double)k_used[b]", "(double)out_n[b] / (double)(k_used[b] + 1)"),
    "ngram_first_match": ("for (int32_t j = L - n - 1; j >= 0; --j) {", "for (int32_t j = 0; j <= L - n - 1; ++j) {"),
    "ngram_suffix_matches_itself": ("for (int32_t j = L - n - 1; j >= 0; --j) {", "for (int32_t j = L - n; j >= 0; --j) {"),
    "rows_past_rejection_read": ("for (int i = 0; i <= r.n && !row_bad; ++i)", "for (int i = 0; i <= k && !row_bad; ++i)"),
    "greedy_nonfinite_row_ignored": ("if (!isfinite(m)) { row_bad = 1; break; }", "if (0) { row_bad = 1; break; }"),
    # the degenerate-residual fallback (reading R11) and the ambiguity flags
    "fallback_from_q": ("        qr = NULL;\n        Zs.s = Zs.c = 0.0;",
                        "        pr = qr;\n        qr = NULL;\n        Zs.s = Zs.c = 0.0;"),
    "no_fallback": ("if (qr && Z < ORC_DEGENERATE_Z) {", "if (0 && qr && Z < ORC_DEGENERATE_Z) {"),
    "fallback_threshold_1e-3": ("#define ORC_DEGENERATE_Z 1e-9", "#define ORC_DEGENERATE_Z 1e-3"),
    "fallback_threshold_1e-12": ("#define ORC_DEGENERATE_Z 1e-9", "#define ORC_DEGENERATE_Z 1e-12"),
    "flag_d_never_set": ("if (degenerate) res.flags |= ORC_FLAG_D;", "if (0) res.flags |= ORC_FLAG_D;"),
    "accept_band_1e-6": ("#define ORC_ACCEPT_BAND 1e-5", "#define ORC_ACCEPT_BAND 1e-6"),
    "accept_band_1e-4": ("#define ORC_ACCEPT_BAND 1e-5", "#define ORC_ACCEPT_BAND 1e-4"),
    "cdf_band_1e-14": ("#define ORC_CDF_BAND 1e-12", "#define ORC_CDF_BAND 1e-14"),
    "cdf_band_1e-10": ("#define ORC_CDF_BAND 1e-12", "#define ORC_CDF_BAND 1e-10"),
    "offsets_order_ignored": ("        for (int32_t j = 0; !bad && j < b; ++j) bad |= offsets[j] > o;\n"
                              "        for (int32_t j = b + 2; !bad && j <= B; ++j) bad |= offsets[j] < offsets[b + 1];",
                              ""),
    "draft_greedy_highest_tie": ("orc_row_argmax(logits, dtype, r, V, &a);\n            out_tokens[r] = (int32_t)a;",
                                 "orc_row_argmax(logits, dtype, r, V, &a);\n            out_tokens[r] = (int32_t)(V - 1 - a);"),
}

PINS = [
    lambda: pins.test_inverse_cdf_hand_case(),
    lambda: pins.test_softmax_matches_scipy("f32", 0.6),
    lambda: pins.test_greedy_equals_argmax_with_ties(),
    lambda: pins.test_alpha_has_no_epsilon_guard(),
    lambda: pins.test_v2_closed_form(),
    lambda: pins.test_lossless_exact_enumeration(0),
    lambda: pins.test_lossless_exact_enumeration(1),
    lambda: pins.test_lossless_chain_k3(),
    lambda: pins.test_k_zero_emits_bonus_or_argmax(),
    lambda: pins.test_oracle_vs_numpy_composition("c3", 6),
    lambda: dpins.test_draft_sample_matches_scipy_searchsorted("f32"),
    lambda: dpins.test_draft_sample_greedy_and_errors(),
    lambda: dpins.test_gathered_reads_only_the_rejected_draft_row(),
    lambda: dpins.test_gathered_bad_values_are_data_errors(),
    lambda: bpins.test_commit_hand_case(),
    lambda: bpins.test_adapt_k_boundaries_are_strict(),
    lambda: bpins.test_adapt_k_window_is_the_last_ten(),
    lambda: bpins.test_adapt_k_rate_uses_the_rounds_own_k(),
    lambda: bpins.test_ngram_hand_cases(),
    lambda: rpins.test_nonfinite_rows_the_scan_reaches(),
    lambda: rpins.test_nonfinite_past_the_rejection_changes_nothing(),
    lambda: rpins.test_greedy_reaches_rows_up_to_the_first_mismatch(),
    lambda: pins.test_offsets_out_of_order_are_data_errors(),
    lambda: fpins.test_degenerate_residual_draws_from_the_target_row(),
    lambda: fpins.test_degenerate_residual_can_emit_the_rejected_token(),
    lambda: fpins.test_small_but_usable_residual_is_drawn_normally(),
    lambda: fpins.test_degenerate_threshold_bracket(),
    lambda: fpins.test_flag_a_inside_the_band(),
    lambda: fpins.test_flag_a_outside_the_band(),
    lambda: fpins.test_flag_a_only_on_evaluated_tests(),
    lambda: fpins.test_flag_b_on_an_exact_boundary(),
    lambda: fpins.test_flag_b_band_width(),
]


@pytest.mark.slow
@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name, tmp_path):
    old, new = MUTANTS[name]
    text = open(SRC).read()
    assert text.count(old) == 1, f"mutation anchor for {name} not unique"
    mutated = tmp_path / "oracle_mutant.c"
    mutated.write_text(text.replace(old, new))
    lib = oracle.build(str(mutated), str(tmp_path / "liboracle_mutant.so"))
    caught = None
    with oracle.using_library(lib):
        for i, pin in enumerate(PINS):
            try:
                pin()
            except AssertionError:
                caught = i
                break
    assert caught is not None, f"mutant {name} survived every pin"
