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


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name, tmp_path, monkeypatch):
    old, new = MUTANTS[name]
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
    for pin in PINS:
        try:
            pin()
        except AssertionError:
            failed.append(getattr(pin, "__name__", "pin"))
    monkeypatch.setattr(R, "_lib", None)
    assert failed, f"no pin caught the mutant {name}"
