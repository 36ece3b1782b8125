"""Plant plausible mistakes in a temporary copy of the oracle source and check
that at least one pin fails for each (CPU only).  The oracle itself is untouched."""
import os

import pytest

import oracle
from tests import oracle_pins

# (name, original text, mutated text)
MUTANTS = [
    ("drop_D_skip", "double y = acc + (Dv ? Dv[d] : 0.0) * ur[t];", "double y = acc;"),
    ("y_from_old_state",
     "h[n] = abar * h[n] + bbar * ur[t];\n        acc += Cb[n * L + t] * h[n];",
     "acc += Cb[n * L + t] * h[n];\n        h[n] = abar * h[n] + bbar * ur[t];"),
    ("sign_of_A", "const double abar = exp(dt * a_dn);\n        double bbar;\n        if ((flags & ORACLE_ZOH) && a_dn != 0.0)\n          bbar = expm1(dt * a_dn) / a_dn * Ab",
     "const double abar = exp(-dt * a_dn);\n        double bbar;\n        if ((flags & ORACLE_ZOH) && a_dn != 0.0)\n          bbar = expm1(dt * a_dn) / a_dn * Ab"),
    ("bias_outside_softplus", "softplus_f64(dr[t] + (bias ? bias[d] : 0.0))",
     "(softplus_f64(dr[t]) + (bias ? bias[d] : 0.0))"),
    ("B_transposed", "bbar = dt * Ab[n * L + t];", "bbar = dt * Ab[t * N + n];"),
    ("softplus_missing_abs", "log1p(exp(-fabs(x)))", "log1p(exp(-x))"),
    ("silu_sign", "return z / (1.0 + exp(-z));", "return z / (1.0 + exp(z));"),
    ("D_outside_gate",
     "double y = acc + (Dv ? Dv[d] : 0.0) * ur[t];\n      if (zr) y *= silu_f64(zr[t]);",
     "double y = acc;\n      if (zr) y *= silu_f64(zr[t]);\n      y += (Dv ? Dv[d] : 0.0) * ur[t];"),
    ("input_u_dropped", "h[n] = abar * h[n] + bbar * ur[t];", "h[n] = abar * h[n] + bbar;"),
    ("C_off_by_one", "acc += Cb[n * L + t] * h[n];", "acc += Cb[n * L + (t > 0 ? t - 1 : 0)] * h[n];"),
    ("initial_state_ignored", "h[n] = h0 ? h0[r * N + n] : 0.0;", "h[n] = 0.0;"),
    ("reverse_ignored", "(flags & ORACLE_REVERSE) ? (L - 1 - s) : s;\n      const double dt = softplus_f64(dr[t] + (bias ? bias[d] : 0.0));",
     "s;\n      const double dt = softplus_f64(dr[t] + (bias ? bias[d] : 0.0));"),
    ("bwd_reverse_ignored", "(flags & ORACLE_REVERSE) ? (L - 1 - s) : s;\n          const double x = dr[t] + bd;",
     "s;\n          const double x = dr[t] + bd;"),
    ("zoh_sign", "bbar = expm1(dt * a_dn) / a_dn * Ab[n * L + t];", "bbar = -expm1(dt * a_dn) / a_dn * Ab[n * L + t];"),
    ("step_drops_u", "*h = abar * *h + bbar * u[r];", "*h = abar * *h + bbar;"),
    ("A_transposed", "const double a_dn = A[d * N + n];\n        const double abar = exp(dt * a_dn);\n        double bbar;\n        if ((flags & ORACLE_ZOH) && a_dn != 0.0)\n          bbar = expm1(dt * a_dn) / a_dn * Ab",
     "const double a_dn = A[n * Dm + d];\n        const double abar = exp(dt * a_dn);\n        double bbar;\n        if ((flags & ORACLE_ZOH) && a_dn != 0.0)\n          bbar = expm1(dt * a_dn) / a_dn * Ab"),
    ("state_written_before_last_step", "for (int64_t n = 0; n < N; ++n) final_state[r * N + n] = h[n];",
     "for (int64_t n = 0; n < N; ++n) final_state[r * N + n] = h[n] * 0.5;"),
    ("step_zoh_sign", "bbar = expm1(dt * a_dn) / a_dn * Bm[b * N + n];",
     "bbar = -expm1(dt * a_dn) / a_dn * Bm[b * N + n];"),
    ("step_zoh_without_expm1", "bbar = expm1(dt * a_dn) / a_dn * Bm[b * N + n];",
     "bbar = (exp(dt * a_dn) - 1.0) / a_dn * Bm[b * N + n];"),
    ("step_zoh_ignored", "if ((flags & ORACLE_ZOH) && a_dn != 0.0)\n        bbar = expm1(dt * a_dn) / a_dn * Bm",
     "if (0)\n        bbar = expm1(dt * a_dn) / a_dn * Bm"),
    ("step_bias_dropped", "const double dt = softplus_f64(delta[r] + (bias ? bias[d] : 0.0));",
     "const double dt = softplus_f64(delta[r]);"),
    ("conv_taps_flipped", "v += w[d * K + k] * xe[t + k];", "v += w[d * K + (K - 1 - k)] * xe[t + k];"),
    ("conv_lookahead", "v += w[d * K + k] * xe[t + k];",
     "v += w[d * K + k] * xe[t + k + 1 < H + L ? t + k + 1 : t + k];"),
    ("conv_bias_dropped", "double v = bias ? bias[d] : 0.0;", "double v = 0.0;"),
    ("conv_no_silu", "u[r * L + t] = silu_f64(v);", "u[r * L + t] = v;"),
    ("conv_state_ignored", "xe[j] = state_in ? state_in[r * H + j] : 0.0;", "xe[j] = 0.0;"),
    ("conv_state_reversed", "xe[j] = state_in ? state_in[r * H + j] : 0.0;",
     "xe[j] = state_in ? state_in[r * H + (H - 1 - j)] : 0.0;"),
    ("conv_state_out_shifted", "state_out[r * H + j] = xe[L + j];",
     "state_out[r * H + j] = xe[L + j > 0 ? L + j - 1 : 0];"),
    ("conv_weight_row_stride", "v += w[d * K + k] * xe[t + k];", "v += w[k * Dm + d] * xe[t + k];"),
    ("bwd_adjoint_not_decayed", "          G[n] *= a;\n", "\n"),
    ("bwd_dC_uses_old_state", "sC[n * L + t] += dy * hs[(s + 1) * N + n];", "sC[n * L + t] += dy * hs[s * N + n];"),
    ("bwd_dB_drops_u", "sB[n * L + t] += G[n] * e * ur[t];", "sB[n * L + t] += G[n] * e;"),
    ("bwd_dA_drops_dt", "rA[r * N + n] += G[n] * (hp * a * dt +", "rA[r * N + n] += G[n] * (hp * a +"),
    ("bwd_softplus_derivative", "const double dx = ddt / (1.0 + exp(-x));", "const double dx = ddt;"),
    ("bwd_ddt_drops_decay_term", "ddt += G[n] * (hp * a * an + e_dt * ur[t] * Ab[n * L + t]);",
     "ddt += G[n] * (e_dt * ur[t] * Ab[n * L + t]);"),
    ("bwd_zoh_e_dt_is_one", "const double e_dt = zoh ? a : 1.0;", "const double e_dt = 1.0;"),
    ("bwd_zoh_dA_term_dropped", "const double e_dA = !zoh ? 0.0 :", "const double e_dA = 1 ? 0.0 :"),
    ("bwd_zoh_dA_sign", "(dt * a - e) / an", "(e - dt * a) / an"),
    ("bwd_zoh_dA_limit", "double s = 0.0, f = 2.0, p = 1.0;", "double s = 0.0, f = 1.0, p = 1.0;"),
    ("zoh_dA_closed_form_near_zero", "if (fabs(x) < 1e-2) {", "if (0) {"),
    ("zoh_e_without_expm1", "bbar = expm1(dt * a_dn) / a_dn * Ab[n * L + t];",
     "bbar = (exp(dt * a_dn) - 1.0) / a_dn * Ab[n * L + t];"),
    ("bwd_zoh_forward_euler", "const double h = a * hs[s * N + n] + e * Ab[n * L + t] * ur[t];",
     "const double h = a * hs[s * N + n] + dt * Ab[n * L + t] * ur[t];"),
    ("bwd_dz_silu_derivative", "sg * (1.0 + zr[t] * (1.0 - sg));", "sg;"),
    ("bwd_du_drops_skip", "double dut = dy * Dd;", "double dut = 0.0;"),
    ("bwd_adjoint_seed_ignored", "G[n] = dfs ? dfs[r * N + n] : 0.0;", "G[n] = 0.0;"),
    ("bwd_dy_ungated", "dy = dout[r * L + t] * silu_f64(zr[t]);", "dy = dout[r * L + t];"),
    ("bwd_adjoint_before_C", "G[n] += dy * Cb[n * L + t];\n            sC", "G[n] += 0.0 * Cb[n * L + t];\n            sC"),
]


@pytest.mark.parametrize("name,orig,mut", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_pins_catch_mutant(tmp_path, name, orig, mut):
    src = oracle.source()
    assert src.count(orig) == 1, "mutation anchor must occur exactly once: " + name
    path = oracle.compile_variant(src.replace(orig, mut), os.path.join(str(tmp_path), "mut_%s.so" % name))
    bad = oracle.Oracle(path)
    caught = []
    for check in oracle_pins.ALL_CHECKS:
        try:
            check(bad)
        except (AssertionError, FloatingPointError, ValueError, RuntimeError):
            caught.append(check.__name__)
    assert caught, "no pin caught mutant " + name
