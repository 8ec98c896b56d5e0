"""Plant plausible mistakes in a copy of the C oracle and check that the pins
in test_oracle.py catch every one of them (on the CPU, in a temp dir)."""
import os
import subprocess
import tempfile

import pytest

import oracle
from tests import test_oracle as pins

SRC = os.path.join(os.path.dirname(oracle.__file__), "gdn_oracle.c")

# (name, text in gdn_oracle.c, replacement)
MUTANTS = [
    ("no decay before the erase", "S[i * dv + j] *= a;", "S[i * dv + j] *= 1.0;"),
    ("error sign flipped", "u[j] = vt[j] - acc;", "u[j] = vt[j] + acc;"),
    ("beta dropped from the write", "S[i * dv + j] += b * kt[i] * u[j];",
     "S[i * dv + j] += kt[i] * u[j];"),
    ("read with k instead of q", "for (int i = 0; i < dk; ++i) acc += S[i * dv + j] * qt[i];",
     "for (int i = 0; i < dk; ++i) acc += S[i * dv + j] * kt[i];"),
    ("closed form decays the write",
     "a * (S[i * dv + j] - b * kt[i] * u[j]) + b * kt[i] * vt[j];",
     "a * (S[i * dv + j] - b * kt[i] * u[j] + b * kt[i] * vt[j]);"),
    ("closed form erase without beta", "a * (S[i * dv + j] - b * kt[i] * u[j])",
     "a * (S[i * dv + j] - kt[i] * u[j])"),
    ("half decay", "const double a = exp(log_alpha[t * H + h]);",
     "const double a = exp(0.5 * log_alpha[t * H + h]);"),
    ("transposed state read", "for (int i = 0; i < dk; ++i) acc += S[i * dv + j] * qt[i];",
     "for (int i = 0; i < dk; ++i) acc += S[(j % dk) * dv + (i % dv)] * qt[i];"),
    ("conv taps reversed", "acc += w[c * K + j] * x[((t0 + src) * H + h) * d + i];",
     "acc += w[c * K + (K - 1 - j)] * x[((t0 + src) * H + h) * d + i];"),
    ("conv not causal-aligned", "const int64_t src = t - (K - 1) + j;",
     "const int64_t src = t - (K - 2) + j;"),
    ("silu as sigmoid", "a[i] = acc / (1.0 + exp(-acc));", "a[i] = 1.0 / (1.0 + exp(-acc));"),
    ("rms without mean", "const double inv = 1.0 / sqrt(ss / d + eps);",
     "const double inv = 1.0 / sqrt(ss + eps);"),
    ("gain without the zero centre", "const double gain = 1.0 + (w ? w[i] : 0.0);",
     "const double gain = (w ? w[i] : 1.0);"),
    ("gate sign", "const double gate = 1.0 / (1.0 + exp(-zr[i]));",
     "const double gate = 1.0 / (1.0 + exp(zr[i]));"),
    ("softplus without its linear part",
     "const double sp = (x > 0.0 ? x : 0.0) + log1p(exp(-fabs(x)));",
     "const double sp = log1p(exp(-fabs(x)));"),
    ("decay bias dropped", "const double x = a[i] + (b_alpha ? b_alpha[h] : 0.0);",
     "const double x = a[i];"),
    ("decay scale A without exp", "log_alpha[i] = -exp(A[h]) * sp;",
     "log_alpha[i] = -A[h] * sp;"),
    ("beta sigmoid sign", "beta[i] = 1.0 / (1.0 + exp(-b[i]));",
     "beta[i] = 1.0 / (1.0 + exp(b[i]));"),
    ("bwd: dk without the read-back term", "dk_out[row * dk + i] -= acc;",
     "dk_out[row * dk + i] -= 0.0 * acc;"),
    ("bwd: state gradient not decayed", "dS[i * dv + j] = a * dSt;", "dS[i * dv + j] = dSt;"),
    ("bwd: dq from the previous state", "for (int j = 0; j < dv; ++j) acc += Sn[i * dv + j] * dyt[j];",
     "for (int j = 0; j < dv; ++j) acc += Sp[i * dv + j] * dyt[j];"),
    ("bwd: erase term missing", "const double dSt = dS[i * dv + j] - kt[i] * de[j];",
     "const double dSt = dS[i * dv + j];"),
    ("bwd: dbeta sign", "dbeta[row] = db;", "dbeta[row] = -db;"),
    ("bwd: dlog_alpha without alpha", "dlog_alpha[row] = a * dalpha;", "dlog_alpha[row] = dalpha;"),
    ("bwd: dv without beta", "de[j] = b * acc;", "de[j] = acc;"),
    ("gate bwd: softplus slope as beta", "da[i] = dlog_alpha[i] * (-exp(A[h]) * sig);",
     "da[i] = dlog_alpha[i] * (-exp(A[h]) * (1.0 - sig));"),
    ("gate bwd: dA without log_alpha", "dA[h] += dlog_alpha[i] * la;", "dA[h] += dlog_alpha[i];"),
]

PIN_FUNCS = [
    lambda: [pins.test_forms_agree(dk, dv, T) for dk, dv, T in [(2, 3, 40), (8, 8, 60)]],
    lambda: pins.test_identity_gates_leave_state(oracle.FORM_ERASE_WRITE),
    lambda: pins.test_identity_gates_leave_state(oracle.FORM_CLOSED),
    lambda: [pins.test_orthonormal_keys_retrieve_values(d) for d in (2, 4)],
    pins.test_orthonormal_keys_with_decay,
    pins.test_full_write_then_read_same_key,
    pins.test_pure_decay,
    pins.test_scalar_closed_form,
    pins.test_rotation_equivariance,
    pins.test_conv_matches_torch_conv1d_and_silu,
    pins.test_conv_impulse_response_tap_order,
    pins.test_l2norm_gives_unit_rows_and_matches_twin,
    pins.test_output_gate_against_torch_rms_norm,
    pins.test_gates_from_raw_against_torch_and_identities,
    pins.test_bwd_matches_finite_differences,
    pins.test_gates_from_raw_bwd_matches_finite_differences,
]


# The C-versus-NumPy comparison is left out on purpose: both were written from
# the same reading of the pages, so each mutant must be caught by a property
# that does not depend on that reading.


@pytest.fixture(scope="module")
def workdir():
    with tempfile.TemporaryDirectory() as d:
        yield d


def test_unmutated_source_passes_all_pins():
    for f in PIN_FUNCS:
        f()


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_mutant_is_caught(name, old, new, workdir):
    src = open(SRC).read()
    assert src.count(old) >= 1, "mutation site not found: %s" % name
    mutated = src.replace(old, new)
    cpath = os.path.join(workdir, "m.c")
    so = os.path.join(workdir, "m_%d.so" % (abs(hash(name)) % 10 ** 8))
    open(cpath, "w").write(mutated)
    subprocess.check_call(["gcc", "-O1", "-fopenmp", "-fPIC", "-shared", "-o", so, cpath, "-lm"])
    caught = 0
    with oracle.use_library(so):
        for f in PIN_FUNCS:
            try:
                f()
            except AssertionError:
                caught += 1
    assert caught >= 1, "no pin caught mutant: %s" % name
