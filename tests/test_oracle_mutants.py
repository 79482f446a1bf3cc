"""The oracle's pins have teeth: each planted mistake fails at least one pin.

A mistake is planted in a copy of ``oracle/gdn_oracle.c`` (on the CPU, never
on a GPU), the copy is compiled with gcc, loaded in place of the real oracle,
and the pin tests of ``test_oracle_pins.py`` are run against it.  The real
oracle is restored afterwards.
"""
import os
import subprocess
import tempfile

import pytest

import oracle
from tests import test_oracle_pins as pins

SRC = os.path.join(os.path.dirname(oracle.__file__), "gdn_oracle.c")

# (name, exact text in gdn_oracle.c, replacement)
MUTANTS = [
    ("prediction_without_decay", "double p = alpha * acc;", "double p = acc;"),
    ("delta_sign", "u[i] = beta * (v[i] - p);", "u[i] = beta * (v[i] + p);"),
    ("delta_without_beta", "u[i] = beta * (v[i] - p);", "u[i] = (v[i] - p);"),
    ("update_without_decay",
     "alpha * S[(size_t)j * dv + i] + u[i] * kh[j]",
     "S[(size_t)j * dv + i] + u[i] * kh[j]"),
    ("update_with_query",
     "alpha * S[(size_t)j * dv + i] + u[i] * kh[j]",
     "alpha * S[(size_t)j * dv + i] + u[i] * qh[j]"),
    ("output_reads_key", "acc += S[(size_t)j * dv + i] * qh[j];",
     "acc += S[(size_t)j * dv + i] * kh[j];"),
    ("output_without_scale", "o[i] = scale * acc;", "o[i] = acc;"),
    ("gate_not_exponentiated", "const double alpha = exp(g);",
     "const double alpha = 1.0 + g;"),
    ("norm_without_eps", "1.0 / sqrt(ss + ORACLE_EPS)", "1.0 / sqrt(ss)"),
    ("norm_squared", "1.0 / sqrt(ss + ORACLE_EPS)", "1.0 / (ss + ORACLE_EPS)"),
    ("key_head_interleaved", "const int kh_idx = h / group;",
     "const int kh_idx = h % h_k;"),
    ("checkpoint_off_by_one", "if (ckpt && (t + 1) % ckpt_interval == 0) {",
     "if (ckpt && t % ckpt_interval == 0 && t > 0) {"),
    ("tree_steps_from_previous_node",
     "const int p = parent[(size_t)lane * t_max + t];",
     "const int p = t - 1;"),
    ("path_commit_replays_first_nodes",
     "const size_t tok = (size_t)ll * t_max + path[(size_t)lane * t_max + j];",
     "const size_t tok = (size_t)ll * t_max + j;"),
    ("kda_gate_not_exponentiated", "const double a = exp(g[j]);",
     "const double a = 1.0 + g[j];"),
    ("kda_channels_reversed", "const double a = exp(g[j]);",
     "const double a = exp(g[dk - 1 - j]);"),
    ("kda_delta_sign", "u[i] = beta * (v[i] - acc);",
     "u[i] = beta * (v[i] + acc);"),
]

PIN_TESTS = [
    lambda: pins.test_hand_worked_two_steps(),
    lambda: pins.test_single_step_closed_form(),
    lambda: pins.test_zero_gates_leave_state_unchanged(),
    lambda: pins.test_delta_rule_writes_value_at_key("qr"),
    lambda: pins.test_delta_rule_writes_value_at_key("permuted_standard"),
    lambda: pins.test_full_forgetting(),
    lambda: pins.test_delta_rule_is_online_regression_step(),
    lambda: pins.test_exact_rational_product_form(),
    lambda: pins.test_l2norm_flag_matches_prenormalised_inputs(),
    lambda: pins.test_scale_multiplies_output_only(),
    lambda: pins.test_prefix_causality_and_commit(),
    lambda: pins.test_chained_rounds_equal_one_long_window(),
    lambda: pins.test_linear_in_state_and_values_jointly(),
    lambda: pins.test_homogeneous_part_is_non_expansive(),
    lambda: pins.test_key_head_sharing_matches_duplicated_keys(),
    lambda: pins.test_prefill_matches_window_and_checkpoints(),
    lambda: pins.test_tree_chain_is_the_linear_window(),
    lambda: pins.test_tree_node_is_its_path_as_a_window(),
    lambda: pins.test_kda_with_equal_channels_is_the_gated_delta_rule(),
    lambda: pins.test_kda_is_online_regression_step_from_the_channel_decayed_state(),
    lambda: pins.test_kda_exact_rational_product_form(),
    lambda: pins.test_kda_channel_forgetting(),
]


def _failures():
    n = 0
    for t in PIN_TESTS:
        try:
            t()
        except (AssertionError, ValueError):
            n += 1
    return n


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_pins_reject_planted_mistake(name, old, new):
    src = open(SRC).read()
    assert src.count(old) >= 1, "mutation site vanished: " + name
    with tempfile.TemporaryDirectory() as d:
        path = os.path.join(d, "mut.c")
        lib = os.path.join(d, "libmut.so")
        open(path, "w").write(src.replace(old, new))
        subprocess.run(["gcc", "-O2", "-fopenmp", "-fPIC", "-shared",
                        "-std=c11", "-ffp-contract=off", "-o", lib, path,
                        "-lm"], check=True)
        handle = oracle.use_library(lib)
        try:
            n_fail = _failures()
        finally:
            oracle.restore_library(handle)
    assert n_fail >= 1, "no pin caught mutant " + name


def test_unmutated_oracle_passes_every_pin():
    assert _failures() == 0
