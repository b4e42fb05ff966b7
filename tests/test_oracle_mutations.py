"""The oracle's pins must catch plausible mistakes.

Each case copies oracle/kda_oracle.c to a temporary directory, plants one
mistake (a dropped term, a wrong sign or index, a missing clamp...), builds
it with gcc and reruns the pin tests against it on the CPU; at least one pin
must fail. The committed oracle is never modified.
"""
import ctypes
import os
import subprocess

import pytest

import test_oracle_pins as pins
from oracle import reference

SRC = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "oracle",
                   "kda_oracle.c")

MUTATIONS = {
    "wrong sign of the retrieval error": ("u[j] = beta * ((double)v[j] - u[j]);",
                                          "u[j] = beta * ((double)v[j] + u[j]);"),
    "gate dropped": ("for (int j = 0; j < Dv; ++j) row[j] *= a;", "(void)a; (void)row;"),
    "gate floor missing": ("if (g < g_min) g = g_min;", "(void)g_min;"),
    "gate cap missing": ("if (g > 0.0) g = 0.0;", ""),
    "readout scale dropped": ("for (int j = 0; j < Dv; ++j) o[j] *= scale;", "(void)scale;"),
    "readout with k instead of q": ("double qc = (double)q[c];", "double qc = (double)k[c];"),
    "beta dropped": ("u[j] = beta * ((double)v[j] - u[j]);", "u[j] = ((double)v[j] - u[j]);"),
    "gate channel index": ("double a = exp(clamp_gate((double)g[c], g_min));",
                           "double a = exp(clamp_gate((double)g[0], g_min));"),
    "checkpoint one token early": ("(t - t0 + 1) % ckpt_interval == 0", "(t - t0 + 2) % ckpt_interval == 0"),
    "initial state ignored": ("memcpy(S, initial_state + (size_t)unit * ssz, sizeof(double) * ssz);",
                              "memset(S, 0, sizeof(double) * ssz);"),
    "write uses value not error": ("for (int j = 0; j < Dv; ++j) u[j] = beta * ((double)v[j] - u[j]);",
                                   "for (int j = 0; j < Dv; ++j) u[j] = beta * (double)v[j];"),
    "retrieval before the gate": (
        "  /* gate: S' = Diag(alpha) S */",
        "  for (int j = 0; j < Dv; ++j) u[j] = 0.0;\n"
        "  for (int c = 0; c < Dk; ++c) for (int j = 0; j < Dv; ++j) u[j] += S[(size_t)c*Dv+j] * (double)k[c];\n"
        "  for (int c = 0; c < Dk; ++c) { double a0 = exp(clamp_gate((double)g[c], g_min)); "
        "for (int j = 0; j < Dv; ++j) S[(size_t)c*Dv+j] = S[(size_t)c*Dv+j] * a0 + 0.0; }\n"
        "  for (int j = 0; j < Dv; ++j) u[j] = beta * ((double)v[j] - u[j]);\n"
        "  for (int c = 0; c < Dk; ++c) for (int j = 0; j < Dv; ++j) S[(size_t)c*Dv+j] += (double)k[c] * u[j];\n"
        "  if (o) { for (int j = 0; j < Dv; ++j) { double s = 0; for (int c = 0; c < Dk; ++c) s += S[(size_t)c*Dv+j] * (double)q[c]; o[j] = scale * s; } }\n"
        "  return;\n"
        "  /* gate: S' = Diag(alpha) S */"),
}

PINS = [pins.test_hand_worked_example,
        lambda: pins.test_oracle_matches_exact_rational_recurrence(0, 12, 4, 3),
        pins.test_oracle_matches_dense_transition_form,
        pins.test_I1_delta_write_back_any_gate, pins.test_I2_per_step_projection,
        pins.test_I3_beta_zero_is_pure_decay, pins.test_I4_orthonormal_keys_give_ungated_linear_attention,
        pins.test_I5_standard_basis_keys_gated_closed_form, pins.test_I9_packing_and_head_independence,
        pins.test_checkpoint_positions_and_count, pins.test_gate_clamp_bounds,
        lambda: pins.test_I10_chunked_form_equals_recurrence(16, 37)]


def _build_mutant(tmp_path, old, new):
    src = open(SRC).read()
    assert src.count(old) == 1, f"mutation anchor not unique: {old!r}"
    path = tmp_path / "mut.c"
    path.write_text(src.replace(old, new))
    lib = tmp_path / "libmut.so"
    subprocess.run(["gcc", "-O1", "-fopenmp", "-fPIC", "-shared", "-std=c11", "-w", "-o", str(lib),
                    str(path), "-lm"], check=True)
    return str(lib)


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_a_pin_catches(name, tmp_path, monkeypatch):
    old, new = MUTATIONS[name]
    libpath = _build_mutant(tmp_path, old, new)
    real = reference.lib()
    mut = ctypes.CDLL(libpath)
    for fn in ("kda_oracle_prefill", "kda_oracle_decode", "kda_oracle_num_checkpoints",
               "kda_oracle_max_threads"):
        getattr(mut, fn).restype = getattr(real, fn).restype
        getattr(mut, fn).argtypes = getattr(real, fn).argtypes
    monkeypatch.setattr(reference, "_lib", mut)
    caught = []
    for pin in PINS:
        try:
            pin()
        except AssertionError:
            caught.append(getattr(pin, "__name__", "pin"))
    assert caught, f"no pin caught the planted mistake: {name}"


# ------------------------------------------------------ front-end oracle
import importlib.util  # noqa: E402

import test_oracle_frontend as fe_pins  # noqa: E402

FE_SRC = os.path.join(os.path.dirname(SRC), "frontend.py")

FE_MUTATIONS = {
    "softplus sign": ("return -np.logaddexp(0.0,", "return np.logaddexp(0.0,"),
    "softplus replaced by the logit": ("return -np.logaddexp(0.0, np.asarray(a, dtype=np.float64))",
                                       "return -np.asarray(a, dtype=np.float64)"),
    "norm without the square root": ("x / np.sqrt(np.sum(x * x, axis=-1, keepdims=True) + float(eps))",
                                     "x / (np.sum(x * x, axis=-1, keepdims=True) + float(eps))"),
    "norm over the wrong axis": ("np.sum(x * x, axis=-1, keepdims=True)", "np.sum(x * x, axis=-2, keepdims=True)"),
    "norm eps dropped": ("keepdims=True) + float(eps))", "keepdims=True))"),
    "sigmoid sign": ("1.0 / (1.0 + np.exp(-b))", "1.0 / (1.0 + np.exp(b))"),
    "k left unnormalised": ("q, k = l2_normalize(q, eps), l2_normalize(k, eps)", "q = l2_normalize(q, eps)"),
    "beta flag applies the gate": ("beta = beta_from_logits(beta)", "beta = gate_from_logits(beta)"),
}


@pytest.mark.parametrize("name", sorted(FE_MUTATIONS))
def test_a_front_end_pin_catches(name, tmp_path):
    old, new = FE_MUTATIONS[name]
    src = open(FE_SRC).read()
    assert src.count(old) == 1, f"mutation anchor not unique: {old!r}"
    path = tmp_path / "frontend_mut.py"
    path.write_text(src.replace(old, new))
    spec = importlib.util.spec_from_file_location("frontend_mut", str(path))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    caught = []
    for check in fe_pins.CHECKS:
        try:
            check(mod)
        except AssertionError:
            caught.append(check.__name__)
    assert caught, f"no front-end pin caught the planted mistake: {name}"


# ------------------------------------------------------ gate variants
import test_oracle_variants as var_pins  # noqa: E402

VAR_SRC = os.path.join(os.path.dirname(SRC), "variants.py")

VAR_MUTATIONS = {
    "head gate ignored": ("return np.broadcast_to(np.asarray(g, dtype=np.float64)[..., None], shape).copy()",
                          "return np.zeros(shape)"),
    "head gate taken from the first head": (
        "return np.broadcast_to(np.asarray(g, dtype=np.float64)[..., None], shape).copy()",
        "return np.broadcast_to(np.asarray(g, dtype=np.float64)[..., :1, None], shape).copy()"),
    "no gate decays at the floor": ("        return np.zeros(shape)\n    raise",
                                    "        return np.full(shape, -0.6931471805599453)\n    raise"),
    "head gate negated": ("return np.broadcast_to(np.asarray(g, dtype=np.float64)[..., None], shape).copy()",
                          "return np.broadcast_to(-np.asarray(g, dtype=np.float64)[..., None], shape).copy()"),
}


@pytest.mark.parametrize("name", sorted(VAR_MUTATIONS))
def test_a_variant_pin_catches(name, tmp_path):
    old, new = VAR_MUTATIONS[name]
    src = open(VAR_SRC).read()
    assert src.count(old) == 1, f"mutation anchor not unique: {old!r}"
    path = tmp_path / "variants_mut.py"
    path.write_text(src.replace(old, new))
    spec = importlib.util.spec_from_file_location("variants_mut", str(path))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    caught = []
    for check in var_pins.CHECKS:
        try:
            check(mod)
        except AssertionError:
            caught.append(check.__name__)
    assert caught, f"no variant pin caught the planted mistake: {name}"
