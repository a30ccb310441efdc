"""The oracle's pins catch plausible mistakes (CPU only).

Each case plants one mistake in a copy of the C recurrence, builds it with the
oracle's own compiler flags, points the oracle's loader at the copy, and runs
the pins of ``test_oracle_pins``: at least one of them must fail.  The
mistakes are the ones a reading of the gated delta rule could plausibly make
(the rule named by the "SANA-WM" cookbook page, "Architecture & components",
row "Attention"): read-out before the update, the decay left off the erase
term, no sigmoid on beta, the gate's sign, no normalisation, q and k swapped
in the read-out, beta on v only, and a transposed entry state.
"""
import os
import subprocess

import pytest

import oracle.recurrence as rec
import test_oracle_pins as pins

SRC = open(rec._SRC).read()

MUTATIONS = {
    "exclusive_output": ("row[j] = alpha * row[j] + w * kh[j];\n                acc += row[j] * qh[j];",
                         "acc += row[j] * qh[j];\n                row[j] = alpha * row[j] + w * kh[j];"),
    "decay_not_on_erase": ("(vt[i] - alpha * sk)", "(vt[i] - sk)"),
    "no_beta_sigmoid": ("1.0 / (1.0 + exp(-bl))", "bl"),
    "gate_sign": ("exp(J->g[th])", "exp(-J->g[th])"),
    "no_normalisation": ("if (n < 1e-6) n = 1e-6;", "n = 1.0;"),
    "q_k_swapped": ("acc += row[j] * qh[j];", "acc += row[j] * kh[j];"),
    "beta_on_v_only": ("beta * (vt[i] - alpha * sk)", "(beta * vt[i] - alpha * sk)"),
    "state_transposed_in": (
        "memcpy(S, J->state_in + sbase, sizeof(double) * (size_t)dv * dk);",
        "for (int a = 0; a < dv; ++a) for (int c = 0; c < dk; ++c) S[a * dk + c] = J->state_in[sbase + c * dv + a];"),
}


def _pin_calls(golden_dir):
    yield "hand_worked_example", lambda: pins.test_hand_worked_example(golden_dir)
    yield "exact_rational_golden", lambda: pins.test_exact_rational_golden(golden_dir)
    yield "exact_random_rational", pins.test_exact_random_rational_cases
    yield "single_token", pins.test_single_token_closed_form
    yield "beta_zero", pins.test_beta_zero_decay_only
    yield "orthonormal_retrieval", pins.test_orthonormal_retrieval_exact
    yield "orthonormal_overwrite", pins.test_orthonormal_retrieval_random_basis_and_overwrite
    yield "small_beta_limit", pins.test_small_beta_linear_attention_limit
    yield "chunked_equals_recurrence", lambda: pins.test_chunked_equals_recurrence(16)
    yield "stream_split", pins.test_stream_split_equals_one_pass_bitwise
    yield "contraction", pins.test_state_norm_contraction_bound
    yield "linearity", pins.test_joint_linearity_in_values_and_state


def test_mutations_apply_to_the_source():
    for name, (a, _) in MUTATIONS.items():
        assert SRC.count(a) == 1, name


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_planted_mistake_fails_a_pin(name, tmp_path, monkeypatch, golden_dir):
    a, b = MUTATIONS[name]
    src = tmp_path / f"{name}.c"
    src.write_text(SRC.replace(a, b))
    lib = tmp_path / f"lib{name}.so"
    subprocess.check_call(["gcc", "-O2", "-std=c11", "-ffp-contract=off", "-fno-fast-math", "-fPIC", "-shared",
                           "-o", str(lib), str(src), "-lm", "-lpthread"])
    monkeypatch.setattr(rec, "_LIB_PATH", str(lib))
    monkeypatch.setattr(rec, "_lib", None)
    failed = []
    for pin, call in _pin_calls(golden_dir):
        try:
            call()
        except AssertionError:
            failed.append(pin)
    assert os.path.samefile(rec._load()._name, str(lib))
    assert failed, f"no pin caught the planted mistake {name}"
