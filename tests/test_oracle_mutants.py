"""Plausible mistakes planted in copies of the oracle (on the CPU) must each be
caught by at least one pin; this is what makes the pins a check on the oracle
rather than a restatement of it."""
import os
import shutil
import subprocess

import pytest

import oracle
from oracle_pins import ALL_PINS

SRC = os.path.join(os.path.dirname(oracle.__file__), "kda_oracle.c")

# (name, exact text in kda_oracle.c, replacement)
MUTANTS = [
    ("write_sign", "(vv[j] - r[j])", "(vv[j] + r[j])"),
    ("write_drops_beta", "S[i * dv + j] += b * kh[i] *", "S[i * dv + j] += kh[i] *"),
    ("predict_with_query", "predict(dk, dv, S, kh, r);", "predict(dk, dv, S, qh, r);"),
    ("read_transposed", "acc += S[i * dv + j] * qh[i];",
     "acc += S[(j % dk) * dv + (i % dv)] * qh[i];"),
    ("read_unscaled", "ot[j] = scale * acc;", "ot[j] = acc;"),
    ("decay_on_columns", "S[i * dv + j] *= alpha[i];", "S[i * dv + j] *= alpha[j % dk];"),
    ("gate_not_exponentiated", "alpha[i] = exp(jb->log_alpha[row_k + i]);",
     "alpha[i] = 1.0 + jb->log_alpha[row_k + i];"),
    ("predict_before_decay", "decay_rows(dk, dv, S, alpha);\n        predict(dk, dv, S, kh, r);",
     "predict(dk, dv, S, kh, r);\n        decay_rows(dk, dv, S, alpha);"),
    ("read_before_write", "write_error(dk, dv, S, kh, vv, r, b);\n        read_state(dk, dv, S, qh, jb->scale, ot);",
     "read_state(dk, dv, S, qh, jb->scale, ot);\n        write_error(dk, dv, S, kh, vv, r, b);"),
    ("conv_taps_reversed", "wc[1] * hist[2 * d + c] +\n                   wc[2] * hist[1 * d + c] + wc[3] * hist[0 * d + c]",
     "wc[3] * hist[2 * d + c] +\n                   wc[2] * hist[1 * d + c] + wc[1] * hist[0 * d + c]"),
    ("silu_is_sigmoid", "out[c] = y * sigmoid(y);", "out[c] = sigmoid(y);"),
    ("no_l2_norm", "double inv = 1.0 / sqrt(ss + eps);", "double inv = 1.0 + 0.0 * ss * eps;"),
    ("v_normalised", "l2_normalise(dk, kh, jb->l2_eps);",
     "l2_normalise(dk, kh, jb->l2_eps);\n            l2_normalise(dv, vv, jb->l2_eps);"),
    ("rms_uses_sum", "ms /= dv;", "ms /= 1.0;"),
    ("gate_not_sigmoid", "sigmoid(jb->g[row_v + j])", "(jb->g[row_v + j])"),
    ("conv_hist_shift", "hist[1 * d + c] = hist[2 * d + c];", "hist[1 * d + c] = x_t[c];"),
    ("state_in_ignored", "memcpy(S, jb->s_in + ((size_t)n * H + h) * sdim, sdim * sizeof(double));",
     "memset(S, 0, sdim * sizeof(double));"),
    ("gate_w_transposed", "zc += z[t * r + j] * w[c * r + j];", "zc += z[t * r + j] * w[(j * H * d + c) % (H * d * r)];"),
    ("gate_bias_sign", "const double u = zc + b[c];", "const double u = zc - b[c];"),
    ("gate_a_not_exponentiated", "const double ea = exp(a[h]);", "const double ea = a[h];"),
    ("gate_a_wrong_head", "const double ea = exp(a[h]);", "const double ea = exp(a[0]);"),
    ("gate_floor_not_five", "-5.0 * sigmoid(ea * u)", "-1.0 * sigmoid(ea * u)"),
    ("softplus_a_inside", "-ea * softplus(u)", "-softplus(ea * u)"),
    ("softplus_sign", "u + log1p(exp(-u))", "u - log1p(exp(-u))"),
    ("softplus_naive_overflows", "u > 0.0 ? u + log1p(exp(-u)) : log1p(exp(u))", "log1p(exp(u))"),
    ("softplus_is_sigmoid_branch", "log1p(exp(u)); }", "exp(u); }"),
    ("beta_logit_sign", "beta[i] = 1.0 / (1.0 + exp(-w[i]));", "beta[i] = 1.0 / (1.0 + exp(w[i]));"),
    ("beta_logit_identity", "beta[i] = 1.0 / (1.0 + exp(-w[i]));", "beta[i] = w[i];"),
    ("beta_logit_tanh", "beta[i] = 1.0 / (1.0 + exp(-w[i]));", "beta[i] = 0.5 * (1.0 + tanh(w[i]));"),
]


@pytest.fixture(scope="module")
def workdir(tmp_path_factory):
    return tmp_path_factory.mktemp("mutants")


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not available")
@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_mutant_is_caught(workdir, name, old, new):
    src = open(SRC).read()
    assert src.count(old) == 1, f"mutation site for {name} not found exactly once"
    path = os.path.join(workdir, f"{name}.c")
    with open(path, "w") as f:
        f.write(src.replace(old, new))
    lib = os.path.join(workdir, f"{name}.so")
    oracle.build(path, lib)
    orc = oracle.Oracle(lib)
    caught = []
    for pin in ALL_PINS:
        try:
            pin(orc)
        except AssertionError:
            caught.append(pin.__name__)
    assert caught, f"no pin catches the planted mistake {name}"
