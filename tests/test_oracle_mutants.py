"""Planted mistakes in a copy of the C oracle must each fail at least one pin.

Each mutant is the oracle source with one plausible slip (dropped term, wrong
sign, wrong index, transposed state, ...), compiled to a temporary library on
the CPU. The pins of test_oracle_pins.py are then run against it; a mutant
that passes every pin would mean the pins do not constrain that part.
"""
import ctypes
import os
import subprocess
import tempfile

import pytest

import oracle
from tests import test_oracle_pins as pins

SRC = os.path.join(os.path.dirname(oracle.__file__), "kda_oracle.c")

MUTANTS = {
    "erase_sign": ("e[j] = b * (orc_load(v, row * V + v0 + j, in_dtype) - s);",
                   "e[j] = b * (orc_load(v, row * V + v0 + j, in_dtype) + s);"),
    "dropped_write": ("S[c * vb + j] += kn[c] * e[j];", "(void)0;"),
    "dropped_decay": ("S[c * vb + j] *= alpha[c];", "(void)0;"),
    "softplus_form": ("log1p(exp(-fabs(x)))", "log1p(exp(-x))"),
    "no_norm": ("const double iq = 1.0 / sqrt(sq + 1e-6), ik = 1.0 / sqrt(sk + 1e-6);",
                "const double iq = 1.0, ik = 1.0;"),
    "transposed_state": ("orc_load(initial_state, ((n * H + h) * K + c) * V + v0 + j, state_dtype)",
                         "orc_load(initial_state, ((n * H + h) * K + v0 + j) * V + c, state_dtype)"),
    "clamp_direction": ("fmax(-decay_rate * orc_softplus(x), lower_bound)",
                        "fmin(-decay_rate * orc_softplus(x), lower_bound)"),
    "dropped_dt_bias": ("+ dt_bias[h * K + c]", "+ 0.0"),
    "head_index": ("const double decay_rate = exp(A_log[h]);",
                   "const double decay_rate = exp(A_log[0]);"),
    "scale_dropped": ("out[row * V + v0 + j] = scale * s;", "out[row * V + v0 + j] = s;"),
    "read_with_key": ("s += S[c * vb + j] * qn[c];", "s += S[c * vb + j] * kn[c];"),
    "varlen_off_by_one": ("eos = cu_seqlens[n + 1];", "eos = cu_seqlens[n + 1] - (n == 0);"),
    "beta_as_one": ("const double b = orc_load(beta, row, in_dtype);", "const double b = 1.0;"),
    "gate_natural_rate": ("const double decay_rate = exp(A_log[h]);",
                          "const double decay_rate = A_log[h];"),
}

PIN_TESTS = [
    (pins.test_p1_brute_force, [(128, 128, 48, 2), (8, 5, 64, 3)]),
    (pins.test_p1_brute_force_varlen, [()]),
    (pins.test_p2_exact_retrieval, [()]),
    (pins.test_p3_frozen_state, [()]),
    (pins.test_p4_linear_attention, [()]),
    (pins.test_p5_gated_closed_form, [()]),
    (pins.test_p6_varlen_equals_separate, [()]),
    (pins.test_p7_state_chaining, [(37,)]),
    (pins.test_p9_head_equivariance, [()]),
    (pins.test_p10_scale_linearity, [()]),
    (pins.test_p11_gate_closed_forms, [()]),
    (pins.test_p12_normalisation_idempotence, [()]),
]


def _build_mutant(name, tmpdir):
    old, new = MUTANTS[name]
    with open(SRC) as fh:
        src = fh.read()
    assert src.count(old) == 1, "mutation site not unique: %s" % name
    path = os.path.join(tmpdir, name + ".c")
    with open(path, "w") as fh:
        fh.write(src.replace(old, new))
    so = os.path.join(tmpdir, name + ".so")
    subprocess.check_call(["gcc", "-O1", "-std=c11", "-fopenmp", "-fPIC", "-shared", "-w",
                           "-o", so, path, "-lm"])
    return so


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name, monkeypatch):
    with tempfile.TemporaryDirectory() as td:
        so = _build_mutant(name, td)
        real = oracle._load()
        lib = ctypes.CDLL(so)
        lib.kda_oracle_fwd.restype = real.kda_oracle_fwd.restype
        lib.kda_oracle_fwd.argtypes = real.kda_oracle_fwd.argtypes
        lib.kda_oracle_max_threads.restype = ctypes.c_int
        monkeypatch.setattr(oracle, "_lib", lib)
        failed = []
        for fn, params in PIN_TESTS:
            for p in params:
                try:
                    fn(*p)
                except (AssertionError, ValueError, FloatingPointError):
                    failed.append(fn.__name__)
                    break
        assert failed, "mutant %s passed every pin" % name


# ---------------------------------------------------------------------------
# the backward oracle (oracle/backward.py): plant a slip, run the B pins on it
# ---------------------------------------------------------------------------
import importlib.util

from tests import test_oracle_backward as bpins

BWD_SRC = os.path.join(os.path.dirname(oracle.__file__), "backward.py")

BWD_MUTANTS = {
    "dbeta_sign": ("dbeta[bos + t, h] = kn[t] @ dSu", "dbeta[bos + t, h] = -(kn[t] @ dSu)"),
    "key_grad_no_erase_term": ("dkn[t] = bb[t] * dSu - X @ du", "dkn[t] = bb[t] * dSu"),
    "output_grad_no_scale": ("dS += scale * np.outer(qn[t], do[t])", "dS += np.outer(qn[t], do[t])"),
    "query_reads_previous_state": ("dqn[t] = scale * (states[t + 1] @ do[t])",
                                   "dqn[t] = scale * (states[t] @ do[t])"),
    "state_grad_no_erase": ("dX = dS - np.outer(kn[t], du)", "dX = dS"),
    "state_grad_no_decay": ("dS = a[t][:, None] * dX", "dS = dX"),
    "gate_sigmoid_sign": ("sig = 0.5 * (1.0 + np.tanh(0.5 * x))", "sig = 0.5 * (1.0 - np.tanh(0.5 * x))"),
    "clamp_passes_gradient": ("dla_free = np.where(clamped, 0.0, dla)", "dla_free = dla"),
    "A_log_grad_uses_rate": ("dA_log[h] += np.sum(dla_free * la_free)", "dA_log[h] += np.sum(dla_free * rate)"),
    "norm_grad_no_projection": ("(dxn - xn * np.sum(xn * dxn, axis=-1, keepdims=True)) / n[:, None]",
                                "dxn / n[:, None]"),
    "final_grad_ignored": ("dS = np.zeros((K, V)) if dfin is None else dfin[n, h].copy()",
                           "dS = np.zeros((K, V))"),
    "decay_grad_uses_new_state": ("dla[t] = a[t] * np.sum(dX * states[t], axis=1)",
                                  "dla[t] = a[t] * np.sum(dX * states[t + 1], axis=1)"),
    "value_grad_no_beta": ("du = bb[t] * (dS.T @ kn[t])", "du = dS.T @ kn[t]"),
}

BWD_PINS = [
    (bpins.test_b1_finite_differences, [(8, 8, 7, 2, 2)]),
    (bpins.test_b1_finite_differences_packed, [()]),
    (bpins.test_b2_one_token_closed_form, [()]),
    (bpins.test_b3_frozen_state_closed_form, [()]),
    (bpins.test_b4_clamp_blocks_gate_gradient, [()]),
]


@pytest.mark.parametrize("name", sorted(BWD_MUTANTS))
def test_backward_mutant_is_caught(name, monkeypatch):
    old, new = BWD_MUTANTS[name]
    with open(BWD_SRC) as fh:
        src = fh.read()
    assert src.count(old) == 1, "mutation site not unique: %s" % name
    spec = importlib.util.spec_from_loader("oracle._bwd_mutant", loader=None)
    mod = importlib.util.module_from_spec(spec)
    mod.__package__ = "oracle"
    exec(compile(src.replace(old, new), BWD_SRC + ":" + name, "exec"), mod.__dict__)
    monkeypatch.setattr(bpins, "obwd", mod)
    failed = []
    for fn, params in BWD_PINS:
        for p in params:
            try:
                fn(*p)
            except (AssertionError, ValueError, FloatingPointError):
                failed.append(fn.__name__)
                break
    assert failed, "backward mutant %s passed every pin" % name
