"""The oracle's pins must catch plausible mistakes (CPU only).

Each mutant plants one mistake in a copy of oracle/iabn_oracle.c -- a dropped
term, a wrong sign, a wrong index, a misplaced constant -- builds it into a
temporary library, and runs the pin tests of test_oracle.py against it.  At
least one pin must fail for every mutant; the unmodified source must pass them.
"""
import os

import numpy as np
import pytest

import oracle
from oracle import build as oracle_build
import workloads

import test_oracle as pins

MUTANTS = {
    "unbiased_normalising_variance": ("const double v = ss / (double)m;",
                                      "const double v = ss / (double)(m - 1);"),
    "eps_outside_root": ("const double is = 1.0 / sqrt(v + eps);",
                         "const double is = 1.0 / (sqrt(v) + eps);"),
    "mean_term_sign": ("dx[AT(n, c, i)] = k * (dz - sdz / (double)m - xhat * sdzx / (double)m);\n"
                       "                if (xhat_out)",
                       "dx[AT(n, c, i)] = k * (dz + sdz / (double)m - xhat * sdzx / (double)m);\n"
                       "                if (xhat_out)"),
    "dropped_xhat_term": ("dx[AT(n, c, i)] = k * (dz - sdz / (double)m - xhat * sdzx / (double)m);\n"
                          "                if (xhat_out)",
                          "dx[AT(n, c, i)] = k * (dz - sdz / (double)m);\n"
                          "                if (xhat_out)"),
    "leaky_inverse_multiplies": ("return y > 0.0 ? y : y / p;", "return y > 0.0 ? y : y * p;"),
    "elu_derivative_drops_alpha": ("return y > 0.0 ? 1.0 : y + p;   /* p*exp(z) = y + p */",
                                   "return y > 0.0 ? 1.0 : y + 1.0;"),
    "elu_forward_exp": ("return z > 0.0 ? z : p * expm1(z);", "return z > 0.0 ? z : p * exp(z);"),
    "running_var_biased": ("+ momentum * v * (double)m / (double)(m - 1);", "+ momentum * v;"),
    "momentum_swapped": ("running_mean[c] = (1.0 - momentum) * running_mean[c] + momentum * mu;",
                         "running_mean[c] = momentum * running_mean[c] + (1.0 - momentum) * mu;"),
    "transposed_index": ("#define AT(n, c, i) ((((int64_t)(n)) * C + (c)) * HW + (i))",
                         "#define AT(n, c, i) ((((int64_t)(c)) * N + (n)) * HW + (i))"),
    "beta_not_removed": ("const double xhat = (z - beta[c]) / gamma[c];\n                sdz += dz;",
                         "const double xhat = z / gamma[c];\n                sdz += dz;"),
    "bf16_truncates": ("r = ldexp(nearbyint(ldexp(f, 8)), e - 8);",
                       "r = ldexp(trunc(ldexp(f, 8)), e - 8);"),
    "eval_backward_drops_slope": ("const double dz = act_derivative_from_y(act, p, yy) * dy[AT(n, c, i)];\n"
                                  "                sdz += dz;\n                sdzx += dz * (z - beta[c]) / gamma[c];",
                                  "const double dz = dy[AT(n, c, i)];\n"
                                  "                sdz += dz;\n                sdzx += dz * (z - beta[c]) / gamma[c];"),
    "eval_backward_eps_outside_root": ("const double k = gamma[c] / sqrt(running_var[c] + eps);",
                                       "const double k = gamma[c] / (sqrt(running_var[c]) + eps);"),
    "eval_backward_keeps_beta": ("sdzx += dz * (z - beta[c]) / gamma[c];",
                                 "sdzx += dz * z / gamma[c];"),
    "f16_flushes_subnormals": ("r = ldexp(nearbyint(ldexp(v, 24)), -24);", "r = 0.0 * v;"),
    "f16_wrong_precision": ("r = ldexp(nearbyint(ldexp(f, 11)), e - 11);",
                            "r = ldexp(nearbyint(ldexp(f, 10)), e - 10);"),
    "gamma_not_applied": ("const double z = gamma[c] * xhat + beta[c];\n"
                          "                y[AT(n, c, i)] = act_forward(act, p, z);",
                          "const double z = xhat + beta[c];\n"
                          "                y[AT(n, c, i)] = act_forward(act, p, z);"),
    # optimized checkpointing
    "ckpt_xhat_not_scaled": ("const double xh = (x[AT(n, c, i)] - mu) * is;",
                             "const double xh = (x[AT(n, c, i)] - mu);"),
    "ckpt_dgamma_uses_z": ("sdzx += dz * xh;", "sdzx += dz * z;"),
    "ckpt_dx_drops_mean_term": ("dx[AT(n, c, i)] = k * (dz - sdz / (double)m - xh * sdzx / (double)m);",
                                "dx[AT(n, c, i)] = k * (dz - xh * sdzx / (double)m);"),
    "ckpt_z_rounded_twice": ("return fma(gamma, xhat, beta);", "return gamma * xhat + beta;"),
    "ckpt_recompute_drops_beta": ("y[AT(n, c, i)] = act_forward(act, p, gamma[c] * xhat[AT(n, c, i)] + beta[c]);",
                                  "y[AT(n, c, i)] = act_forward(act, p, gamma[c] * xhat[AT(n, c, i)]);"),
}


def _pin_suite():
    """Run the pin tests of test_oracle.py; return the names of those that fail."""
    cases = []
    for wl in pins.SMALL:
        cases.append(("torch:" + wl.name, lambda wl=wl: pins.test_forward_and_backward_match_torch_fp64(wl)))
        cases.append(("invariants:" + wl.name, lambda wl=wl: pins.test_invariants(wl)))
    cases += [
        ("finite_differences", pins.test_backward_matches_finite_differences),
        ("textbook_bn", lambda: pins.test_identity_activation_is_textbook_bn(False)),
        ("rational_example", pins.test_exact_rational_example),
        ("brute_force", pins.test_statistics_brute_force),
        ("running_closed_form", pins.test_running_statistics_closed_form),
        ("bf16_rounding", pins.test_round_storage_bf16_matches_torch_on_f32_values),
        ("eval", lambda: pins.test_eval_forward_matches_torch("elu", 1.0)),
        ("eval_backward", lambda: pins.test_eval_backward_matches_torch("leaky_relu", 0.2)),
        ("eval_backward_fd", pins.test_eval_backward_matches_finite_differences),
        ("f16_rounding", pins.test_round_storage_f16_matches_numpy_on_f32_values),
        ("ckpt_backward_fd", pins.test_ckpt_backward_matches_finite_differences),
        ("ckpt_exact_sign", pins.test_ckpt_backward_branches_on_the_exact_sign_of_z),
    ]
    for wl in pins.SMALL[:3]:
        cases.append(("ckpt_forward:" + wl.name,
                      lambda wl=wl: pins.test_ckpt_forward_matches_torch_fp64(wl)))
        cases.append(("ckpt_backward:" + wl.name,
                      lambda wl=wl: pins.test_ckpt_backward_matches_torch_fp64(wl)))
    failed = []
    for name, fn in cases:
        try:
            fn()
        except (AssertionError, ValueError):
            failed.append(name)
    return failed


@pytest.fixture(scope="module")
def source():
    with open(oracle_build.SRC) as f:
        return f.read()


def test_unmodified_source_passes(source, tmp_path):
    lib = oracle_build.compile_source(oracle_build.SRC, str(tmp_path / "orig.so"))
    oracle.use_library(lib)
    try:
        assert _pin_suite() == []
    finally:
        oracle.use_library(None)


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name, source, tmp_path):
    old, new = MUTANTS[name]
    assert source.count(old) == 1, "mutation site not found exactly once: " + name
    src = tmp_path / ("mutant_%s.c" % name)
    src.write_text(source.replace(old, new))
    lib = oracle_build.compile_source(str(src), str(tmp_path / ("mutant_%s.so" % name)))
    oracle.use_library(lib)
    try:
        failed = _pin_suite()
    finally:
        oracle.use_library(None)
    assert failed, "no pin caught mutant " + name
