"""The oracle's pins catch plausible mistakes.

Each case plants one mistake in a copy of the oracle's C source (on the CPU,
in a temporary directory), builds it, points the oracle's numpy front end at
the mutant and runs the pins: at least one pin must fail.  This is what makes
the pins a check on the oracle rather than a restatement of it.
"""
import os
import subprocess

import pytest

import oracle.ref as R
from oracle import build as OB
import tests.test_oracle_pins as P
import tests.test_oracle_bwd_c as PB
import tests.test_oracle_trap as PT

SRC = os.path.join(os.path.dirname(OB.__file__), "ssm_ref.c")

MUTANTS = {
    "readout_reads_previous_state": (
        "    h[n] = abar * h[n] + bbar_u;               /* h_t = Abar h_{t-1} + Bbar u_t */\n"
        "    acc += Ct[n] * h[n];                       /* y_t = C_t . h_t */\n",
        "    acc += Ct[n] * h[n];\n    h[n] = abar * h[n] + bbar_u;\n"),
    "dropped_D_skip": ("(D ? D[d] : 0.0) * ut", "0.0 * ut"),
    "wrong_sign_in_fade": ("exp(delta * Arow[n])", "exp(-delta * Arow[n])"),
    "fade_uses_first_state_only": ("exp(delta * Arow[n])", "exp(delta * Arow[0])"),
    "B_and_C_swapped": ("double bbar_u = delta * Bt[n] * ut;", "double bbar_u = delta * Ct[n] * ut;"),
    "bias_dropped": ("double x = raw + (bias ? bias[d] : 0.0);", "double x = raw;"),
    "softplus_without_log1p": ("return log1p(exp(x));", "return exp(x);"),
    "gate_is_sigmoid_not_silu": ("return z / (1.0 + exp(-z));", "return 1.0 / (1.0 + exp(-z));"),
    "composition_operands_swapped": ("double b = a2[i] * b1[i] + b2[i];", "double b = a1[i] * b2[i] + b1[i];"),
    "batch_and_time_axes_swapped": ("long io = (b * j->L + t) * j->dim + d;", "long io = (t * j->batch + b) * j->dim + d;"),
    "final_state_not_per_channel": ("j->final_state[(r * j->dim + d) * j->N + n] = h[n];",
                                    "j->final_state[r * j->N + n] = h[n];"),
    "input_term_missing_u": ("double bbar_u = delta * Bt[n] * ut;", "double bbar_u = delta * Bt[n];"),
}

# Mistakes in the trapezoidal (Mamba-3) step, caught by the pins of test_oracle_trap.py.
TRAP_MUTANTS = {
    "trap_beta_without_fade": ("double beta = 0.5 * delta * alpha;", "double beta = 0.5 * delta;"),
    "trap_beta_and_gamma_swapped": ("double prev_in = Bprev ? beta * Bprev[n] * uprev : 0.0;\n"
                                    "    h[n] = alpha * h[n] + prev_in + gamma * Bt[n] * ut;",
                                    "double prev_in = Bprev ? gamma * Bprev[n] * uprev : 0.0;\n"
                                    "    h[n] = alpha * h[n] + prev_in + beta * Bt[n] * ut;"),
    "trap_full_step_weights": ("double gamma = 0.5 * delta;", "double gamma = delta;"),
    "trap_previous_input_never_kept": ("        Bprev = &j->B[bc];\n", ""),
    "trap_previous_input_is_current": ("        uprev = j->u[io];\n", "        uprev = 0.0;\n"),
    "trap_previous_B_is_current": ("double prev_in = Bprev ? beta * Bprev[n] * uprev : 0.0;",
                                   "double prev_in = Bprev ? beta * Bt[n] * uprev : 0.0;"),
    "trap_gate_dropped": ("  if (zt) v = v * ssm_ref_silu(*zt);\n  return v;\n}\n\ntypedef",
                          "  return v;\n}\n\ntypedef"),
    "trap_skip_dropped": ("  double v = acc + (D ? D[d] : 0.0) * ut;\n  if (zt) v = v * ssm_ref_silu(*zt);\n  return v;\n}\n\ntypedef",
                          "  double v = acc;\n  if (zt) v = v * ssm_ref_silu(*zt);\n  return v;\n}\n\ntypedef"),
}

# Mistakes in the backward oracle's adjoint recurrence, caught by the pins of test_oracle_bwd_c.py.
BWD_MUTANTS = {
    "bwd_adjoint_not_faded": ("        lam[n] *= a;                                   /* on to h_{t-1} */\n", ""),
    "bwd_dC_reads_previous_state": ("j->dC[bc + n] += dv * hs[t * N + n];", "j->dC[bc + n] += dv * hp[n];"),
    "bwd_step_gradient_misses_fade_term": ("ddl += lam[n] * (Ad[n] * a * hp[n] + ut * j->B[bc + n]);",
                                           "ddl += lam[n] * (ut * j->B[bc + n]);"),
    "bwd_dA_misses_step": ("j->dA[d * N + n] += lam[n] * dl * a * hp[n];", "j->dA[d * N + n] += lam[n] * a * hp[n];"),
    "bwd_softplus_derivative_dropped": ("const double dx = j->softplus_flag ? ddl * sigmoid(x) : ddl;",
                                        "const double dx = ddl;"),
    "bwd_gate_derivative_is_sigmoid": ("j->dz[io] = j->dy[io] * vs[t] * s * (1.0 + zt * (1.0 - s));",
                                       "j->dz[io] = j->dy[io] * vs[t] * s;"),
    "bwd_skip_gradient_dropped": ("double du = j->D ? j->D[d] * dv : 0.0, ddl = 0.0;", "double du = 0.0, ddl = 0.0;"),
    "bwd_dB_from_output_gradient": ("j->dB[bc + n] += lam[n] * dl * ut;", "j->dB[bc + n] += dv * dl * ut;"),
    "bwd_only_first_worker_summed": ("for (int i = 0; i < nthreads; ++i) s += jobs[i].dA[e];",
                                     "s += jobs[0].dA[e];"),
    "bwd_final_state_gradient_ignored": ("lam[n] = j->dfs ? j->dfs[(b * dim + d) * N + n] : 0.0;", "lam[n] = 0.0;"),
    "bwd_trap_previous_input_gradient_to_current_token": (
        "            du_next += lam[n] * 0.5 * dl * a * j->B[bc - N + n];",
        "            du += lam[n] * 0.5 * dl * a * j->B[bc - N + n];"),
    "bwd_trap_beta_step_derivative_without_fade": (
        "ddl += lam[n] * bu * (0.5 * a + 0.5 * dl * Ad[n] * a);", "ddl += lam[n] * bu * 0.5;"),
    "bwd_trap_current_input_full_step": ("du += lam[n] * 0.5 * dl * j->B[bc + n];", "du += lam[n] * dl * j->B[bc + n];"),
}

BWD_PINS = [
    lambda: PB.test_gradients_match_central_differences(True, True, True, True),
    lambda: PB.test_gradients_match_central_differences(False, False, True, False),
    PB.test_relay_example_gradients_by_hand,
    lambda: PB.test_agrees_with_autograd_oracle("all"),
    PB.test_thread_count_changes_only_the_order_of_sums,
    lambda: PB.test_trap_gradients_match_central_differences(True, True, True),
    lambda: PB.test_trap_agrees_with_autograd_oracle("all"),
]

TRAP_PINS = [
    PT.test_impulse_response_by_hand,
    PT.test_constant_inputs_closed_form,
    PT.test_second_order_convergence_to_the_continuous_model,
    PT.test_no_decay_is_the_cumulative_trapezoid,
    PT.test_initial_state_adds_its_own_decay,
    PT.test_skip_and_gate_alone,
]

PINS = [
    P.test_p1_relay_worked_example_composition,
    P.test_p1_relay_for_any_pad_via_decode,
    P.test_p6_relay_end_to_end_scan_n1,
    P.test_p2_associativity_identity_noncommutative,
    P.test_p4_lti_closed_form_convolution,
    lambda: P.test_p5_brute_force_unrolling(7, 16, 4, True),
    lambda: P.test_p5_brute_force_unrolling(8, 13, 3, False),
    P.test_p7_delta_limits,
    P.test_p11_zero_input,
    lambda: P.test_softplus_matches_logaddexp(-5.0),
    lambda: P.test_silu_gate_matches_expit(1.0),
    P.test_d_skip_alone,
]


@pytest.mark.parametrize("name", sorted(MUTANTS) + sorted(TRAP_MUTANTS) + sorted(BWD_MUTANTS))
def test_mutant_is_caught(name, tmp_path, monkeypatch):
    for table, table_pins in ((MUTANTS, PINS), (TRAP_MUTANTS, TRAP_PINS), (BWD_MUTANTS, BWD_PINS)):
        if name in table:
            (old, new), pins = table[name], table_pins
    src = open(SRC).read()
    assert src.count(old) >= 1, f"mutation site for {name} not found"
    mutated = src.replace(old, new, 1)
    csrc = tmp_path / "ssm_ref.c"
    csrc.write_text(mutated)
    (tmp_path / "ssm_ref.h").write_text(open(os.path.join(os.path.dirname(SRC), "ssm_ref.h")).read())
    lib = tmp_path / "libmutant.so"
    subprocess.run(["gcc", "-std=c99", "-O2", "-fPIC", "-shared", "-ffp-contract=off", "-o", str(lib), str(csrc),
                    "-lm", "-lpthread"], check=True)
    monkeypatch.setattr(R._build, "LIB", str(lib))
    monkeypatch.setattr(R, "_lib", None)
    failed = []
    for pin in pins:
        try:
            pin()
        except AssertionError:
            failed.append(getattr(pin, "__name__", "pin"))
    monkeypatch.setattr(R, "_lib", None)
    assert failed, f"no pin caught the mutant {name}"
