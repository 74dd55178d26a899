"""Plant a mistake in a copy of the oracle's source (on the CPU) and check
that at least one pin rejects it.  This is the evidence that the pins can
tell a right oracle from a plausible wrong one."""
import os

import pytest

import oracle
from tests import oracle_pins

# (name, original text, replacement) -- each a plausible slip in the arithmetic.
MUTANTS = [
    ("decay dropped", "for (int i = 0; i < dk * dv; i++) S[i] *= alpha;", ""),
    ("delta sign", "u[j] = b * (vt[j] - acc);", "u[j] = b * (vt[j] + acc);"),
    ("beta misplaced", "u[j] = b * (vt[j] - acc);", "u[j] = b * vt[j] - acc;"),
    ("beta twice", "u[j] = b * (vt[j] - acc);", "u[j] = b * b * (vt[j] - acc);"),
    ("write dropped", "S[i * dv + j] += kh[i] * u[j];", "S[i * dv + j] += 0.0 * kh[i] * u[j];"),
    ("read with key", "acc += S[i * dv + j] * qh[i];", "acc += S[i * dv + j] * kh[i];"),
    ("read before write", "        /* write: S <- S + k u^T */\n        for (int i = 0; i < dk; i++)\n            for (int j = 0; j < dv; j++) S[i * dv + j] += kh[i] * u[j];\n",
     ""),
    ("head map", "(h / (Hv / Hk))", "(h % Hk)"),
    ("norm without sqrt", "f = mul / sqrt(ss + GDN_ORACLE_L2_EPS);", "f = mul / (ss + GDN_ORACLE_L2_EPS);"),
    ("eps outside sqrt", "f = mul / sqrt(ss + GDN_ORACLE_L2_EPS);", "f = mul / (sqrt(ss) + GDN_ORACLE_L2_EPS);"),
    ("half gate", "exp(J->g[t * Hv + h])", "exp(0.5 * J->g[t * Hv + h])"),
    ("state_in ignored", "if (J->state_in)\n", "if (0)\n"),
    ("conv taps reversed", "acc += w[c * W + j] * xv;", "acc += w[c * W + (W - 1 - j)] * xv;"),
    ("conv window order", "xv = win_in ? win_in[((long)s * Wm1 + (Wm1 + src)) * C + c] : 0.0;\n                    acc",
     "xv = win_in ? win_in[((long)s * Wm1 + (-1 - src)) * C + c] : 0.0;\n                    acc"),
    ("silu sign", "return a / (1.0 + exp(-a));", "return a / (1.0 + exp(a));"),
    ("f32 conv taps reversed", "acc = fmaf(w[c * W + j], xv, acc);", "acc = fmaf(w[c * W + (W - 1 - j)], xv, acc);"),
    ("exp coefficient", "p = fmaf(p, r, (float)(1.0 / 6.0));", "p = fmaf(p, r, (float)(1.0 / 7.0));"),
    ("exp reduction", "r = fmaf(-n, c2, r);", "r = r;"),
    ("norm sum for mean", "sqrt(ss / d + eps)", "sqrt(ss + eps)"),
    ("norm eps outside", "sqrt(ss / d + eps)", "(sqrt(ss / d) + eps)"),
    ("norm weight dropped", "y[r * d + j] = w[j] * orow[j]", "y[r * d + j] = orow[j]"),
    ("norm gate as sigmoid", "inv_rms * silu_f64(zrow[j])", "inv_rms * silu_f64(zrow[j]) / zrow[j]"),
    ("norm over all rows", "ss += orow[j] * orow[j];", "ss += o[j] * o[j];"),
    ("gating softplus as exp", "-exp(A_log[h]) * softplus_f64(a[i] + dt_bias[h])", "-exp(A_log[h]) * exp(a[i] + dt_bias[h])"),
    ("gating A_log not exponentiated", "-exp(A_log[h]) * softplus_f64", "-A_log[h] * softplus_f64"),
    ("gating sign", "g[i] = -exp(A_log[h])", "g[i] = exp(A_log[h])"),
    ("gating bias dropped", "softplus_f64(a[i] + dt_bias[h])", "softplus_f64(a[i])"),
    ("gating bias of head 0", "softplus_f64(a[i] + dt_bias[h])", "softplus_f64(a[i] + dt_bias[0])"),
    ("beta sign", "beta[i] = 1.0 / (1.0 + exp(-b[i]));", "beta[i] = 1.0 / (1.0 + exp(b[i]));"),
    ("softplus large-x branch", "(x > 0.0 ? x : 0.0) + log1p(exp(-fabs(x)))", "log1p(exp(-fabs(x)))"),
]


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_mutant_is_caught(tmp_path, name, old, new):
    src = oracle.source_text()
    assert src.count(old) >= 1, f"mutation site for '{name}' not found"
    mutant = oracle.build_variant(src.replace(old, new, 1), os.path.join(str(tmp_path), "mutant.so"))
    caught = []
    for pin in oracle_pins.ALL_PINS:
        try:
            pin(mutant)
        except AssertionError:
            caught.append(pin.__name__)
    assert caught, f"no pin rejects the mutant '{name}'"
