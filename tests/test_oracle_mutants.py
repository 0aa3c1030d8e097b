"""The pins must be able to fail: plant plausible mistakes in copies of the C oracle (on the CPU)
and check that at least one pin rejects each mutant."""
import ctypes
import os
import subprocess

import numpy as np
import pytest

import oracle
import test_oracle_pins as pins

SRC = os.path.join(os.path.dirname(oracle.__file__), "gdn_oracle.c")

# (name, exact text in the oracle source, replacement) or (name, [(old, new), ...])
MUTANTS = [
    ("readout_before_update",
     [("            /* u = h^T k", "            {double* o0 = o + tv * dv; for (int cc = 0; cc < dv; ++cc) { o0[cc] = 0; for (int r = 0; r < dk; ++r) o0[cc] += h[(size_t)r * dv + cc] * scale * qt[r]; }}\n            /* u = h^T k"),
      ("double* ot = o + tv * dv;", "double otmp[1024]; double* ot = otmp;")]),
    ("decay_dropped_on_state", "h[(size_t)r * dv + cc] = alpha * h[(size_t)r * dv + cc] + kt[r] * u[cc];",
     "h[(size_t)r * dv + cc] = h[(size_t)r * dv + cc] + kt[r] * u[cc];"),
    ("decay_dropped_in_erase", "u[cc] = bt * (vt[cc] - alpha * u[cc]);", "u[cc] = bt * (vt[cc] - u[cc]);"),
    ("erase_sign_flipped", "u[cc] = bt * (vt[cc] - alpha * u[cc]);", "u[cc] = bt * (vt[cc] + alpha * u[cc]);"),
    ("beta_only_on_erase", "u[cc] = bt * (vt[cc] - alpha * u[cc]);", "u[cc] = vt[cc] - bt * alpha * u[cc];"),
    ("state_transposed_read", "u[cc] += h[(size_t)r * dv + cc] * kt[r];", "u[cc] += h[(size_t)cc * dv + r] * kt[r];"),
    ("gqa_modulo_mapping", "i = j / grp;", "i = j % Hqk;"),
    ("scale_dropped", "const double qr = scale * qt[r];", "const double qr = qt[r];"),
    ("decay_off_by_one", "const double alpha = exp(g[tv]);", "const double alpha = exp(t > 0 ? g[tv - Hv] : 0.0);"),
]


def _pin_tests():
    return [pins.test_hand_worked_example, pins.test_p1_beta_zero_pure_decay,
            pins.test_p2_unit_key_writes_value_exactly, pins.test_p3_single_step_invariants,
            pins.test_p4_online_objective_stationary, pins.test_p5_identical_unit_keys_closed_form,
            pins.test_p6_orthonormal_keys_decayed_linear_attention,
            lambda: pins.test_p7_brute_force_dense_transitions(7),
            lambda: pins.test_p8_chunked_equals_recurrent(16, 50),
            pins.test_p9_gqa_equals_repeated_heads, pins.test_p9_ungated_equals_delta_loop,
            pins.test_gate_limit_alpha_zero_clears_state, pins.test_scale_multiplies_q]


def _edits(m):
    return m[1] if isinstance(m[1], list) else [(m[1], m[2])]


@pytest.mark.parametrize("mut", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_pins_reject_mutant(mut, tmp_path, monkeypatch):
    name = mut[0]
    src = open(SRC).read()
    for old, new in _edits(mut):
        assert src.count(old) == 1, f"mutation site for {name} not found exactly once"
        src = src.replace(old, new)
    mpath = tmp_path / "mutant.c"
    mpath.write_text(src)
    lib = tmp_path / "libmutant.so"
    subprocess.run(["gcc", "-O1", "-fPIC", "-shared", "-fopenmp", str(mpath), "-o", str(lib), "-lm"], check=True)
    mlib = ctypes.CDLL(str(lib))
    real = oracle.load()
    mlib.gdn_oracle_recurrent.argtypes = real.gdn_oracle_recurrent.argtypes
    mlib.gdn_oracle_recurrent.restype = ctypes.c_int
    monkeypatch.setattr(oracle, "_lib", mlib)
    failed = []
    for t in _pin_tests():
        try:
            with np.errstate(all="ignore"):
                t()
        except AssertionError:
            failed.append(getattr(t, "__name__", "lambda"))
    assert failed, f"no pin rejects mutant {name}"
