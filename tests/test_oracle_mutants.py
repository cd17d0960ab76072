"""Plant plausible mistakes in copies of the oracle and require a pin to catch each.

Each mutant is the oracle's own source with one textual change (a dropped term, a
wrong sign or index, a transposed operand), loaded as a separate module on the CPU.
The real oracle is never modified.
"""
import importlib.util
import os
import types

import pytest

import oracle_checks as oc

SRC = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "oracle", "bam_oracle.py")

MUTANTS = {
    "offset sign": ("x = d - float(mu)", "x = d + float(mu)"),
    "dropped 1/sqrt(Dh)": ("S = (q @ k.T) / math.sqrt(Dh)", "S = (q @ k.T)"),
    "causal mask direction": ("visible = (j <= i) if causal", "visible = (j >= i) if causal"),
    "SSMax not applied to bias": ("L[visible] = (c * (S + bias))[visible]", "L[visible] = (c * S + bias)[visible]"),
    "SSMax n off by one": ("return float(s) * np.log(n)", "return float(s) * np.log(n + 1)"),
    "bias sign": ("out[nz] = -np.power(u[nz], beta)\n    return out", "out[nz] = np.power(u[nz], beta)\n    return out"),
    "transposed P in PV": ("O[r0:r0 + chunk] = P @ v", "O[r0:r0 + chunk] = P.T @ v"),
    "lse without max": ("return E / Z, (m + np.log(Z))[:, 0]", "return E / Z, (np.log(Z))[:, 0]"),
    "bwd: c dropped from dq/dk": ("G = c * dZ / math.sqrt(Dh)", "G = dZ / math.sqrt(Dh)"),
    "bwd: dV uses P not P^T": ("dv[b, h] = P.T @ dd", "dv[b, h] = P @ dd"),
    "bwd: beta factor dropped in db/dalpha": ("out[nz] = beta * np.power(u[nz], beta) / float(alpha)",
                                              "out[nz] = np.power(u[nz], beta) / float(alpha)"),
    "bwd: D from V instead of O": ("D = (dd * O).sum(axis=1, keepdims=True)", "D = (dd * vv).sum(axis=1, keepdims=True)"),
    "bwd: ds without bias term": ("tsum = dZ[visible] * lnn * (S[visible] + bias[visible])",
                                  "tsum = dZ[visible] * lnn * S[visible]"),
    "bwd: dbeta sign": ("out[nz] = -np.power(u[nz], beta) * np.log(u[nz])", "out[nz] = np.power(u[nz], beta) * np.log(u[nz])"),
    "decode query position": ("np.array([n - 1]), alpha[h]", "np.array([n - 2]), alpha[h]"),
    "alpha as multiplier": ("return np.abs(x) / float(alpha)", "return np.abs(x) * float(alpha)"),
    "ref: offset sign": ("return -np.asarray(d, np.float64) - ref_mu(theta_mu)",
                         "return -np.asarray(d, np.float64) + ref_mu(theta_mu)"),
    "ref: distance sign with offset": ("return -np.asarray(d, np.float64) - ref_mu(theta_mu)",
                                       "return np.asarray(d, np.float64) - ref_mu(theta_mu)"),
    "ref: eps dropped": ("g = np.abs(_ref_x(d, theta_mu)) + float(eps)\n    return -math.exp",
                         "g = np.abs(_ref_x(d, theta_mu))\n    return -math.exp"),
    "ref: mu = 2 cosh": ("return math.exp(t) - math.exp(-t)", "return math.exp(t) + math.exp(-t)"),
    "ref: chain factor of theta_mu dropped": (" / g * (math.exp(t) + math.exp(-t))", " / g"),
    "ref: dtheta_beta log without eps": ("return prior_bias_ref(d, theta_alpha, theta_beta, theta_mu, eps) * np.log(g)",
                                         "return prior_bias_ref(d, theta_alpha, theta_beta, theta_mu, eps) * np.log(g - float(eps) + 1e-300)"),
    "sandwich: frequency exponent i/d_bar": ("np.cos(d / 10000.0 ** (2.0 * i / float(d_bar)))",
                                             "np.cos(d / 10000.0 ** (1.0 * i / float(d_bar)))"),
    "sandwich: ratio multiplies": ("return out / float(ratio)", "return out * float(ratio)"),
    "sandwich: one frequency too many": ("nf = int(float(d_bar)) // 2", "nf = int(float(d_bar)) // 2 + 1"),
    "A_alpha without |.|": ("A[0, h] += np.abs(ta).sum()", "A[0, h] += ta.sum()"),
    "A_beta from the alpha terms": ("A[1, h] += np.abs(tb).sum()", "A[1, h] += np.abs(ta).sum()"),
    "A_s without ln n": ("A[2, h] += np.abs(tsum).sum()", "A[2, h] += np.abs(tsum / lnn).sum()"),
    "A_mu over every entry": ("A[3, h] += np.abs(tm).sum()", "A[3, h] += np.abs(tm).sum() + np.abs(c * dZ).sum()"),
    "dmu sign": ("out[nz] = beta * np.power(u[nz], beta) / x[nz]", "out[nz] = -beta * np.power(u[nz], beta) / x[nz]"),
}


def _load_mutant(old, new):
    src = open(SRC).read()
    assert src.count(old) == 1, f"mutation site not unique or missing: {old!r}"
    mod = types.ModuleType("bam_oracle_mutant")
    mod.__file__ = SRC
    exec(compile(src.replace(old, new), SRC + " (mutant)", "exec"), mod.__dict__)
    return mod


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name):
    mod = _load_mutant(*MUTANTS[name])
    failed = []
    for check in oc.ALL_CHECKS:
        try:
            check(mod)
        except Exception as e:  # AssertionError, or an exception the mistake provokes
            failed.append((check.__name__, type(e).__name__))
    assert failed, f"mutant '{name}' passes every pin"
