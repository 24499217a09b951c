"""Plant plausible mistakes in the oracle (on the CPU) and require the pins to
catch every one of them.

Each mutant is the oracle's C source with one edit: a dropped term, a wrong
sign or index, a transposed operand, a reordered step, or an alternative
reading of the pages that the design rejects.  The mutant is compiled to a
temporary library and every pin of ``oracle_pins`` is run against it; at
least one must fail.  This checks the pins, not the oracle.
"""
import os
import tempfile

import pytest

import oracle
import oracle_pins

SRC = os.path.join(os.path.dirname(oracle.__file__), "kdn_oracle.c")


def _block(src, start, end):
    a = src.index(start)
    b = src.index(end, a)
    return a, b


def _swap(src, m1, m2, m3):
    """Swap the text [m1, m2) with [m2, m3)."""
    a, b = _block(src, m1, m2)
    _, c = _block(src, m2, m3)
    return src[:a] + src[b:c] + src[a:b] + src[c:]


def _sub(old, new):
    def f(src):
        assert old in src, old
        return src.replace(old, new, 1)
    return f


MUTANTS = {
    "error_sign": _sub("e[j] = vt[j] - e[j];", "e[j] = vt[j] + e[j];"),
    "predict_alpha_not_squared": _sub(
        "pm[i] = a[i] * a[i] * p[i] + xi[tok * dk + i];",
        "pm[i] = a[i] * p[i] + xi[tok * dk + i];"),
    "predict_drops_process_noise": _sub(
        "pm[i] = a[i] * a[i] * p[i] + xi[tok * dk + i];",
        "pm[i] = a[i] * a[i] * p[i];"),
    "innovation_k_not_squared": _sub("s += pm[i] * kt[i] * kt[i];",
                                     "s += pm[i] * kt[i];"),
    "innovation_drops_obs_noise": _sub("double s = rt;", "double s = 0.0 * rt;"),
    "mu_in_current_gain": _sub("s += pm[i] * kt[i] * kt[i];",
                               "s += mu * pm[i] * kt[i] * kt[i];"),
    "mu_dropped": _sub("const double den = rt + mu * pm[i] * kt[i] * kt[i];",
                       "const double den = rt + pm[i] * kt[i] * kt[i];"),
    "moment_matching_projection": _sub(
        "p[i] = (den != 0.0) ? pm[i] * rt / den : pm[i];",
        "p[i] = pm[i] - pm[i] * pm[i] * kt[i] * kt[i] / s;"),
    "gain_uses_prior_not_predicted": _sub(
        "w[i] = (s != 0.0) ? pm[i] * kt[i] / s : 0.0;",
        "w[i] = (s != 0.0) ? p[i] * kt[i] / s : 0.0;"),
    "gain_without_variance": _sub(
        "w[i] = (s != 0.0) ? pm[i] * kt[i] / s : 0.0;",
        "w[i] = (s != 0.0) ? kt[i] / s : 0.0;"),
    "decay_after_read": lambda s: _swap(s, "        /* 3. Decay", "        /* 4. Read",
                                        "        /* 5. Correct"),
    "output_before_write": lambda s: _swap(s, "        /* 5. Correct",
                                           "        /* 6. Read the output",
                                           "    }\n}\n"),
    "output_reads_key": _sub("ot[j] += S[i * dv + j] * qt[i];",
                             "ot[j] += S[i * dv + j] * kt[i];"),
    "write_wrong_value_index": _sub("S[i * dv + j] += w[i] * e[j];",
                                    "S[i * dv + j] += w[i] * e[dv - 1 - j];"),
    "read_transposed": _sub("e[j] += S[i * dv + j] * kt[i];",
                            "e[j] += S[i * dv + j] * kt[dk - 1 - i];"),
    "channel_decay_reversed": _sub("a[i] = alpha[tok * dk + i];",
                                   "a[i] = alpha[tok * dk + (dk - 1 - i)];"),
    "beta_from_head_zero": _sub("const double bt = beta[tok];",
                                "const double bt = beta[(b * T + t) * H];"),
    "decay_on_value_axis": _sub("S[i * dv + j] *= a[i];",
                                "S[i * dv + j] *= a[j % dk];"),
    "initial_state_ignored": _sub("        if (S0) {", "        if (0) {"),
    "no_decay_scalar_gate": _sub("a[i] = alpha[tok];", "a[i] = 1.0;"),
    "variance_not_carried": _sub("p[i] = (den != 0.0) ? pm[i] * rt / den : pm[i];",
                                 "p[i] = (den != 0.0) ? p[i] : pm[i];"),
    # backward
    "bwd_dq_from_previous_memory": _sub("r += St[i * dv + j] * dot[j];",
                                        "r += Sp[i * dv + j] * dot[j];"),
    "bwd_output_term_dropped": _sub("dS[i * dv + j] += qt[i] * dot[j];",
                                    "dS[i * dv + j] += 0.0 * qt[i] * dot[j];"),
    "bwd_de_without_beta": _sub("r += dS[i * dv + j] * bt * kt[i];",
                                "r += dS[i * dv + j] * kt[i];"),
    "bwd_read_term_dropped": _sub("dSm[i * dv + j] = dS[i * dv + j] - kt[i] * de[j];",
                                  "dSm[i * dv + j] = dS[i * dv + j];"),
    "bwd_dk_sign": _sub("dk_out[tok * dk + i] = -r + bt * dw[i];",
                        "dk_out[tok * dk + i] = r + bt * dw[i];"),
    "bwd_dk_without_write_term": _sub("dk_out[tok * dk + i] = -r + bt * dw[i];",
                                      "dk_out[tok * dk + i] = -r;"),
    "bwd_decay_grad_from_new_memory": _sub("r += dSm[i * dv + j] * Sp[i * dv + j];",
                                           "r += dSm[i * dv + j] * St[i * dv + j];"),
    "bwd_memory_grad_not_decayed": _sub("dS[i * dv + j] = a[i] * dSm[i * dv + j];",
                                        "dS[i * dv + j] = dSm[i * dv + j];"),
    "bwd_dbeta_wrong_vector": _sub("db += kt[i] * dw[i];", "db += qt[i] * dw[i];"),
    # isotropic-KDN backward (the variance chain)
    "iso_bwd_gain_term_sign": _sub("dpm += db * rt / (s * s);", "dpm -= db * rt / (s * s);"),
    "iso_bwd_update_not_squared": _sub("dpm += dp * rt * rt / (den * den);",
                                       "dpm += dp * rt / den;"),
    "iso_bwd_variance_not_decayed": _sub("dp = dpm * a2;", "dp = dpm;"),
    "iso_bwd_noise_not_averaged": _sub("dxi[tok * dk + i] = dpm / (double)dk;",
                                       "dxi[tok * dk + i] = dpm;"),
    "iso_bwd_key_norm_factor": _sub("dk_out[tok * dk + i] += dkk * 2.0 * k[tok * dk + i];",
                                    "dk_out[tok * dk + i] += dkk * k[tok * dk + i];"),
    "iso_bwd_obs_noise_update_term": _sub("drt += dp * m * pm * pm * kk / (den * den);",
                                          "drt += 0.0 * dp;"),
    "iso_bwd_decay_from_new_variance": _sub("const double da2 = dpm * pp;",
                                            "const double da2 = dpm * pm;"),
    # diagonal-KDN backward
    "diag_bwd_error_grad_uses_key": _sub("rd += dS[i * dv + j] * wt[i];",
                                         "rd += dS[i * dv + j] * kt[i];"),
    "diag_bwd_innovation_sign": _sub("ds -= dwt[i] * pm * kt[i] / (s * s);",
                                     "ds += dwt[i] * pm * kt[i] / (s * s);"),
    "diag_bwd_gain_key_term_dropped": _sub("double dki = du * pm + 2.0 * ds * pm * kt[i];",
                                           "double dki = du * pm;"),
    "diag_bwd_update_term_not_squared": _sub("dpm += dp[i] * rt * rt / (den * den);",
                                             "dpm += dp[i] * rt / den;"),
    "diag_bwd_obs_noise_gain_term": _sub("double drt = ds;", "double drt = 0.0;"),
    "diag_bwd_variance_not_decayed": _sub("dp[i] = a[i] * a[i] * dpm;", "dp[i] = dpm;"),
    "diag_bwd_decay_grad_missing_factor": _sub(
        "dalpha[tok * dk + i] += 2.0 * a[i] * pp[i] * dpm;",
        "dalpha[tok * dk + i] += a[i] * pp[i] * dpm;"),
    # isotropic KDN
    "iso_alpha_not_squared": _sub("a2 += a[i] * a[i];", "a2 += a[i];"),
    "iso_drops_process_noise": _sub("xm += xi[tok * dk + i];", "xm += 0.0;"),
    "iso_sum_not_mean": _sub(
        "const double pmi = (a2 / (double)dk) * p[0] + xm / (double)dk;",
        "const double pmi = a2 * p[0] + xm;"),
    "iso_noise_sum_not_mean": _sub(
        "const double pmi = (a2 / (double)dk) * p[0] + xm / (double)dk;",
        "const double pmi = (a2 / (double)dk) * p[0] + xm;"),
    "iso_k_not_squared": _sub("kk += kt[i] * kt[i];", "kk += kt[i];"),
    "iso_mu_not_over_dk": _sub("(mu / (double)dk) * pmi * kk", "mu * pmi * kk"),
    "iso_mu_in_gain": _sub("const double s = rt + pmi * kk;",
                           "const double s = rt + mu * pmi * kk;"),
    "iso_drops_obs_noise": _sub("const double s = rt + pmi * kk;",
                                "const double s = pmi * kk;"),
    "iso_gain_uses_prior": _sub("w[i] = (s != 0.0) ? pmi * kt[i] / s : 0.0;",
                                "w[i] = (s != 0.0) ? p[0] * kt[i] / s : 0.0;"),
    "iso_moment_matching": _sub("p[0] = (den != 0.0) ? pmi * rt / den : pmi;",
                                "p[0] = pmi - pmi * pmi * kk / (s * (double)dk);"),
    "iso_variance_not_carried": _sub("p[0] = (den != 0.0) ? pmi * rt / den : pmi;",
                                     "p[0] = (den != 0.0) ? p[0] : pmi;"),
}


@pytest.fixture(scope="module")
def tmpdir_mut():
    with tempfile.TemporaryDirectory() as d:
        yield d


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_mutant(name, tmpdir_mut):
    with open(SRC) as f:
        src = f.read()
    mutated = MUTANTS[name](src)
    assert mutated != src
    c = os.path.join(tmpdir_mut, f"{name}.c")
    so = os.path.join(tmpdir_mut, f"lib{name}.so")
    with open(c, "w") as f:
        f.write(mutated)
    oracle.build(src=c, out=so)
    lib = oracle.OracleLib(so)
    caught = []
    pins = [(p, (lib.recurrence,)) for p in oracle_pins.ALL_PINS]
    pins += [(p, (lib,)) for p in oracle_pins.BWD_PINS]
    for pin, args in pins:
        try:
            pin(*args)
        except (AssertionError, FloatingPointError, ValueError,
                ZeroDivisionError, RuntimeError):
            caught.append(pin.__name__)
    assert caught, f"no pin caught the planted mistake {name!r}"


def test_unmutated_source_passes_every_pin(tmpdir_mut):
    so = os.path.join(tmpdir_mut, "libclean.so")
    oracle.build(src=SRC, out=so)
    lib = oracle.OracleLib(so)
    for pin in oracle_pins.ALL_PINS:
        pin(lib.recurrence)
    for pin in oracle_pins.BWD_PINS:
        pin(lib)
