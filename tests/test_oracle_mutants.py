"""Each pin earns its place: a build of the oracle with one plausible mistake
planted in it (CPU only, in a temporary directory) must fail at least one pin.
The mistakes are the kinds the oracle could plausibly contain: a dropped
term, a wrong comparison, an inverted ratio, a wrong index or exponent."""
import os
import subprocess
import tempfile

import pytest

import oracle
from oracle import build as obuild
from tests import oracle_pins as pins

MUTANTS = {
    "tie_uses_ge": ("(norm > max_norm) ? 1 : 0", "(norm >= max_norm) ? 1 : 0"),
    "norm_without_sqrt": ("const double norm = sqrt(sumsq);", "const double norm = sumsq;"),
    "ratio_inverted": ("clip ? max_norm / norm : 1.0", "clip ? norm / max_norm : 1.0"),
    "l1_instead_of_squares": ("total += u * u;", "total += fabs(u);"),
    "last_tensor_dropped": ("if (n < 0 || !dtype_ok(dt) || !sumsq || !nonfinite) return -1;\n  double total = 0.0;\n  int32_t nf = 0;\n  for (int32_t t = 0; t < n; ++t) {",
                            "if (n < 0 || !dtype_ok(dt) || !sumsq || !nonfinite) return -1;\n  double total = 0.0;\n  int32_t nf = 0;\n  for (int32_t t = 0; t + 1 < n; ++t) {"),
    "truncating_round": ("double r = nearbyint(q);", "double r = floor(q);"),
    "avg_not_in_norm": ("const double u = avg * g;", "const double u = g;"),
    "avg_not_in_factor": ("*scale = avg * coef;", "*scale = coef;"),
    "inf_not_nonfinite": ("if (!isfinite(g)) nf = 1;", "if (isnan(g)) nf = 1;"),
    "subnormal_exponent_off_by_one": ("v = ldexp((double)m, 1 - bias - mb);", "v = ldexp((double)m, -bias - mb);"),
    "no_subnormal_clamp": ("if (E < emin) E = emin;", "if (E < emin - 100) E = emin;"),
    "stop_switch_ignored": ("*skip = (nonfinite && error_if_nonfinite) ? 1 : 0;", "*skip = 0;"),
    "sign_dropped": ("return sign ? -v : v;", "return v;"),
    "exponent_transposed": ("const double q = ldexp(a, mb - E);", "const double q = ldexp(a, E - mb);"),
    "avg_squared_twice": ("const double u = avg * g;", "const double u = avg * avg * g;"),
    "scale_skips_last_element": ("for (int64_t i = 0; i < numels[t]; ++i) {\n      const double g = oracle_decode(ptrs[t], i, dt);\n      store_bits",
                                 "for (int64_t i = 0; i + 1 < numels[t]; ++i) {\n      const double g = oracle_decode(ptrs[t], i, dt);\n      store_bits"),
    "adamw_no_bias_correction": ("const double mhat = mi / bc1;", "const double mhat = mi;"),
    "adamw_eps_inside_sqrt": ("p_out[i] = pi - lr * (mhat / (sqrt(vhat) + eps) + wd * pi);",
                              "p_out[i] = pi - lr * (mhat / sqrt(vhat + eps) + wd * pi);"),
    "adamw_decay_coupled": ("const double g = s * oracle_decode(grad, i, dt);",
                            "const double g = s * oracle_decode(grad, i, dt) + wd * (double)p[i];"),
    "adamw_betas_swapped": ("const double mi = b1 * (double)m[i] + (1.0 - b1) * g;",
                            "const double mi = b2 * (double)m[i] + (1.0 - b2) * g;"),
    "adamw_clip_factor_dropped": ("const double g = s * oracle_decode(grad, i, dt);",
                                  "const double g = oracle_decode(grad, i, dt);"),
    "adamw_step_off_by_one": ("const double bc1 = 1.0 - pow(b1, (double)step);",
                              "const double bc1 = 1.0 - pow(b1, (double)(step + 1));"),
    "amp_scale_not_inverted": ("return 1.0 / (n_microbatches * (double)scale);",
                               "return n_microbatches * (double)scale;"),
    "amp_microbatches_ignored": ("return 1.0 / (n_microbatches * (double)scale);", "return 1.0 / (double)scale;"),
    "amp_backoff_keeps_count": ("    *scale = (float)((double)*scale * backoff);\n    *tracker = 0;",
                                "    *scale = (float)((double)*scale * backoff);"),
    "amp_grows_on_inf": ("    *scale = (float)((double)*scale * backoff);", "    *scale = (float)((double)*scale * growth);"),
    "amp_no_overflow_guard": ("if (isfinite(grown)) *scale = grown;", "*scale = grown;"),
    "amp_interval_off_by_one": ("if (clean == interval) {", "if (clean > interval) {"),
    "per_tensor_uses_list_norm": ("oracle_decide(tout[3 * t + 1], nf_t,", "oracle_decide(sqrt(list_sumsq), nf_t,"),
    "per_tensor_takes_next_tensor": ("oracle_sumsq((const void* const*)&ptrs[t], &numels[t], 1, dt, avg, &tout[3 * t], &nf_t);",
                                     "oracle_sumsq((const void* const*)&ptrs[t], &numels[t], t + 1 < n ? 2 : 1, dt, avg, &tout[3 * t], &nf_t);"),
    "per_tensor_stop_only_bad_tensor": ("    tout[3 * t + 2] = skip ? 1.0 : s_t;", "    tout[3 * t + 2] = unused ? 1.0 : s_t;"),
    "per_tensor_stop_ignored": ("    if (!skip) oracle_scale(&ptrs[t], &numels[t], 1, dt, s_t);",
                                "    oracle_scale(&ptrs[t], &numels[t], 1, dt, s_t);"),
    "per_tensor_scales_first_only": ("    if (!skip) oracle_scale(&ptrs[t], &numels[t], 1, dt, s_t);",
                                     "    if (!skip && t == 0) oracle_scale(&ptrs[t], &numels[t], 1, dt, s_t);"),
    "accumulate_drops_contribution": ("const double s = oracle_decode(acc[t], i, dt) + oracle_decode(g[t], i, dt);",
                                      "const double s = oracle_decode(acc[t], i, dt);"),
    "accumulate_subtracts": ("const double s = oracle_decode(acc[t], i, dt) + oracle_decode(g[t], i, dt);",
                             "const double s = oracle_decode(acc[t], i, dt) - oracle_decode(g[t], i, dt);"),
    "accumulate_next_element": ("const double s = oracle_decode(acc[t], i, dt) + oracle_decode(g[t], i, dt);",
                                "const double s = oracle_decode(acc[t], i, dt) + oracle_decode(g[t], i + 1 < numels[t] ? i + 1 : i, dt);"),
    "overflow_not_to_inf": ("if (E > emax) return sign | exp_all;  /* already", "if (E > emax + 1) return sign | exp_all;  /* already"),
}


def _build_mutant(tmp, name, find, repl):
    src = open(obuild.SRC).read()
    assert src.count(find) >= 1, f"mutant {name}: pattern not found"
    msrc = src.replace(find, repl, 1)
    cpath = os.path.join(tmp, f"{name}.c")
    lpath = os.path.join(tmp, f"lib{name}.so")
    with open(cpath, "w") as f:
        f.write(msrc)
    subprocess.run(["gcc", "-O2", "-ffp-contract=off", "-fPIC", "-shared", "-o", lpath, cpath, "-lm"], check=True)
    return lpath


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name, tmp_path):
    find, repl = MUTANTS[name]
    lib = _build_mutant(str(tmp_path), name, find, repl)
    o = oracle.Oracle(lib)
    failed = []
    for pin in pins.ALL_PINS:
        try:
            pin(o)
        except (AssertionError, ValueError, ZeroDivisionError, OverflowError):
            failed.append(pin.__name__)
            break
    assert failed, f"no pin catches the planted mistake {name!r}"


def test_unmutated_source_passes_all_pins(tmp_path):
    lib = _build_mutant(str(tmp_path), "identity", "#include <math.h>", "#include <math.h>")
    o = oracle.Oracle(lib)
    for pin in pins.ALL_PINS:
        pin(o)
