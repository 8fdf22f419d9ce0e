"""The oracle's pins must catch plausible mistakes (no GPU).

Each case copies ``oracle/ssd_oracle.c``, plants one mistake by a textual
substitution (a dropped term, a wrong sign, a wrong operand or index, a missing
transpose), builds the copy with gcc into a temporary directory and runs the pin
tests against it.  At least one pin must fail for every planted mistake.  The
committed oracle is never modified.
"""
import os
import subprocess

import pytest

import oracle
import test_oracle_moments as tm
import test_oracle_pr as tp
import test_oracle_diag as td
import test_oracle_quat as tq
import test_oracle_ssd as ts

SRC = os.path.join(os.path.dirname(oracle.__file__), "ssd_oracle.c")

MUTANTS = {
    "drop_skip_term": ("yt[p] = acc + D[h] * xt[p];", "yt[p] = acc;"),
    "decay_sign": ("const double a = exp(dtv * A[h]);", "const double a = exp(-dtv * A[h]);"),
    "y_reads_B_not_C": ("acc += H[p * R + r] * Ct[r];", "acc += H[p * R + r] * Bt[r];"),
    "dC_uses_previous_state": ("acc += dyt[p] * Ht[p * R + r];", "acc += dyt[p] * Hp[p * R + r];"),
    "ddt_drops_decay_term": ("d_dt[off_dt(d, b, h, t)] = gw + Ah * q;",
                             "d_dt[off_dt(d, b, h, t)] = gw;"),
    "adjoint_not_decayed": ("for (int64_t i = 0; i < PR; ++i) G[i] *= a;",
                            "for (int64_t i = 0; i < PR; ++i) G[i] *= 1.0;"),
    "dB_missing_dt": ("dBt[r] = dtv * acc;", "dBt[r] = acc;"),
    "dA_missing_dt": ("*d_A_acc += dtv * q;", "*d_A_acc += q;"),
    "m1_squares_rows": ("M1[r1] += row[r1];", "M1[r1] += row[r1] * row[r1];"),
    "dm2_not_symmetrised": ("S[i * R + j] = dm2[i * R + j] + dm2[j * R + i];",
                            "S[i * R + j] = 2.0 * dm2[i * R + j];"),
    "dx_transposed_contraction": ("for (int64_t r = 0; r < R; ++r) acc += G[p * R + r] * Bt[r];",
                                  "for (int64_t r = 0; r < R; ++r) acc += G[r * (P > R ? 0 : 1) + p * R] * Bt[r];"),
    "moments_count_without_headdim": ("count[b] = v * P;", "count[b] = v;"),
    "pr_centre_sign": ("S[i * R + j] = M2[i * R + j] / n - mu[i] * mu[j];",
                       "S[i * R + j] = M2[i * R + j] / n + mu[i] * mu[j];"),
    "pr_trace_of_sigma": ("if (trace) trace[o] = trm2 / n;", "if (trace) trace[o] = tr;"),
    "pr_grad_drops_numerator": ("double gh = (i == j) ? 2.0 * tr1 / tr2 : 0.0;",
                                "double gh = 0.0;"),
    "pr_dm1_not_transposed": ("acc -= (G[i * R + j] + G[j * R + i]) * mu[j];",
                              "acc -= 2.0 * G[i * R + j] * mu[j];"),
    "pr_dm2_missing_count": ("d_m2[o * R * R + k] = G[k] / n;", "d_m2[o * R * R + k] = G[k];"),
    "diag_fwd_transposed_qk": ("for (int64_t mi = 0; mi < M; ++mi) acc += qk[mo * M + mi] * V[",
                               "for (int64_t mi = 0; mi < M; ++mi) acc += qk[mi * M + mo] * V["),
    "diag_dgamma_drops_dy": ("dg += dy[dg_off(t, mo, h, M, H, P) + p] * yu;", "dg += yu;"),
    "diag_db_not_transposed": ("acc += dqk[mo * M + mi] * C[dg_off(t, mo, h, M, H, R) + r];",
                               "acc += dqk[mi * M + mo] * C[dg_off(t, mo, h, M, H, R) + r];"),
    "diag_dv_missing_gamma": ("acc += qk[mo * M + mi] * g * dy[", "acc += qk[mo * M + mi] * dy["),
    "quat_product_sign": ("const double y = a[0] * b[2] - a[1] * b[3] + a[2] * b[0] + a[3] * b[1];",
                          "const double y = a[0] * b[2] + a[1] * b[3] + a[2] * b[0] + a[3] * b[1];"),
    "quat_bwd_factor_order": ("qmul(qc, G, n);", "qmul(G, qc, n);"),
    "quat_bwd_uses_current_state": ("const double* prev = t > 0 ? cum + (t - 1) * 4 : c0;",
                                    "const double* prev = cum + t * 4;"),
}

PINS = [
    lambda: ts.test_I1_chunked_forward_matches_recurrence(4),
    ts.test_I2_scalar_case_is_a_first_order_iir_filter,
    ts.test_golden_hand_worked_example,
    lambda: ts.test_chunked_backward_matches_reverse_recurrence(4),
    ts.test_I3_finite_differences_all_seven_gradients,
    ts.test_I5_euler_identities,
    tm.test_I6_explicit_sum_brute_force,
    tm.test_I7_closed_form_matches,
    tm.test_moments_finite_differences,
    tm.test_golden_hand_worked_moments,
    lambda: tp.test_pr_equals_the_eigenvalue_form(True),
    tp.test_trace_is_the_mean_squared_sample_norm,
    lambda: tp.test_pr_gradient_matches_direct_formula(True),
    tp.test_pr_gradient_has_no_radial_part,
    td.test_siso_path_equals_general_path,
    td.test_memoryless_ssd_is_the_diagonal_term,
    td.test_finite_differences_all_four_gradients,
    lambda: td.test_linearity_in_each_input(2),
    tq.test_unit_table,
    tq.test_matches_scipy_rotation_composition,
    tq.test_finite_differences_general_quaternions,
    tq.test_page_closed_form_for_unit_quaternions,
]


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_planted_mistake_is_caught(name, tmp_path):
    before, after = MUTANTS[name]
    src = open(SRC).read()
    assert src.count(before) == 1, f"mutation anchor for {name} not unique"
    mutant = tmp_path / "mutant.c"
    mutant.write_text(src.replace(before, after))
    so = tmp_path / "libmutant.so"
    subprocess.run(["gcc", "-O2", "-std=c99", "-shared", "-fPIC", str(mutant), "-o", str(so), "-lm"],
                   check=True)
    prev = oracle.use_library(str(so))
    caught = []
    try:
        for pin in PINS:
            try:
                pin()
            except (AssertionError, RuntimeError):
                caught.append(getattr(pin, "__name__", "pin"))
    finally:
        oracle.use_library(None)
        oracle._lib = prev
    assert caught, f"no pin caught the planted mistake {name}"
