"""Plant plausible mistakes in copies of the oracle (on the CPU) and check that
the pins catch every one of them. The oracle source is never modified: each
mutant is a patched copy compiled into a temporary directory."""
import os

import pytest

import oracle
import pins

_UPDATE = """        for (int64_t n = 0; n < N; ++n) {
            const double a = A[d * N + n];
            const double abar = exp(dt * a);
            double bcoef = dt;                                   /* Euler: Delta */
            if (zoh && a != 0.0) bcoef = expm1(dt * a) / a;      /* (1 - exp(Delta a)) / (-a) */
            h[n] = abar * h[n] + bcoef * Bm[bc + n] * u;
        }
"""
_READOUT = """        double yt = 0.0;
        for (int64_t n = 0; n < N; ++n) yt += Cm[bc + n] * h[n];"""

MUTANTS = {
    "conv_taps_reversed": [
        ("c += conv_w[d * K + k] * win[k];", "c += conv_w[d * K + (K - 1 - k)] * win[k];"),
        ("c += conv_w[d * K + (K - 1)] * xt;", "c += conv_w[d * K + 0] * xt;"),
    ],
    "conv_history_not_shifted": [("if (K > 1) win[K - 2] = xt;", "if (K > 1) win[0] = xt;")],
    "no_silu_after_conv": [("u = silu(c);", "u = c;")],
    "softplus_drops_bias": [("softplus(delta[row] + (delta_bias ? delta_bias[d] : 0.0))",
                             "softplus(delta[row])")],
    "softplus_log1p_dropped": [("return m + log1p(exp(-fabs(v)));", "return m + exp(-fabs(v));")],
    "decay_sign_flipped": [("abar = exp(dt * a);", "abar = exp(-dt * a);")],
    "zoh_instead_of_euler": [("if (zoh && a != 0.0)", "if (a != 0.0)")],
    "euler_instead_of_zoh": [("if (zoh && a != 0.0)", "if (0 && a != 0.0)")],
    "zoh_sign_flipped": [("bcoef = expm1(dt * a) / a;", "bcoef = expm1(dt * a) / (-a);")],
    "zoh_without_minus_one": [("bcoef = expm1(dt * a) / a;", "bcoef = exp(dt * a) / a;")],
    "zoh_extra_delta": [("bcoef = expm1(dt * a) / a;", "bcoef = dt * expm1(dt * a) / a;")],
    "zoh_zero_a_drops_input": [("if (zoh && a != 0.0) bcoef = expm1(dt * a) / a;",
                                "if (zoh) bcoef = (a != 0.0) ? expm1(dt * a) / a : 0.0;")],
    "write_term_without_delta": [("double bcoef = dt;", "double bcoef = 1.0;")],
    "state_not_carried": [("h[n] = abar * h[n] + bcoef", "h[n] = abar * 0.0 + bcoef")],
    "B_and_C_swapped": [("bcoef * Bm[bc + n] * u", "bcoef * Cm[bc + n] * u"),
                        ("yt += Cm[bc + n] * h[n];", "yt += Bm[bc + n] * h[n];")],
    "readout_before_update": [(_UPDATE + "\n" + _READOUT, _READOUT + "\n" + _UPDATE)],
    "skip_dropped": [("yt += (Dskip ? Dskip[d] : 0.0) * u;", "yt += 0.0 * u;")],
    "skip_uses_x": [("yt += (Dskip ? Dskip[d] : 0.0) * u;", "yt += (Dskip ? Dskip[d] : 0.0) * xt;")],
    "gate_sigmoid_not_silu": [("if (z) yt *= silu(z[row]);", "if (z) yt *= 1.0 / (1.0 + exp(-z[row]));")],
    "gate_before_skip": [("""        yt += (Dskip ? Dskip[d] : 0.0) * u;

        if (z) yt *= silu(z[row]);""", """        if (z) yt *= silu(z[row]);
        yt += (Dskip ? Dskip[d] : 0.0) * u;""")],
    "initial_state_ignored": [("h[n] = ssm_state ? ssm_state[(b * D + d) * N + n] : 0.0;", "h[n] = 0.0;")],
    "conv_history_ignored": [("win[k] = conv_state ? conv_state[(b * D + d) * (K - 1) + k] : 0.0;",
                              "win[k] = 0.0;")],
    # backward
    "bwd_adjoint_not_decayed": [("g_next[n] = ab * g;", "g_next[n] = g;")],
    "bwd_dA_missing_delta": [("dA_loc[n] += g * (dt[t] * ab * hp", "dA_loc[n] += g * (ab * hp")],
    "bwd_ddelta_missing_write_term": [("dDelta += g * (an * ab * hp + dw_ddt * Bn * u[t]);",
                                       "dDelta += g * (an * ab * hp);")],
    "bwd_dC_uses_previous_state": [("dCacc[bc + n] += dyg * h[(t + 1) * N + n];",
                                    "dCacc[bc + n] += dyg * h[t * N + n];")],
    "bwd_dB_missing_u": [("dBacc[bc + n] += g * w * u[t];", "dBacc[bc + n] += g * w;")],
    "bwd_dz_with_gated_output": [("a->dz[row] = a->dy[row] * yt * dsilu(zt);",
                                  "a->dz[row] = a->dy[row] * yt * silu(zt) * dsilu(zt);")],
    "bwd_softplus_derivative_flipped": [("const double ddel = dDelta * sigmoid(v[t]);",
                                         "const double ddel = dDelta * sigmoid(-v[t]);")],
    "bwd_conv_taps_reversed": [("dxa[t + k] += a->conv_w[d * K + k] * dc;",
                                "dxa[t + k] += a->conv_w[d * K + (K - 1 - k)] * dc;")],
    "bwd_dsilu_is_dsigmoid": [("return s * (1.0 + v * (1.0 - s));", "return s * (1.0 - s);")],
    "bwd_skip_gradient_dropped": [("double du = dsk * dyg, dDelta = 0.0;", "double du = 0.0 * dyg, dDelta = 0.0;")],
    "bwd_zoh_dwdA_sign": [("dw_dA = (dt[t] * ab - w) / an;", "dw_dA = (w - dt[t] * ab) / an;")],
    "bwd_zoh_dwddelta_euler": [("dw_ddt = ab;", "dw_ddt = 1.0;")],
    "bwd_final_state_grad_ignored": [("g_next[n] = a->dstate_final ? a->dstate_final[(b * D + d) * N + n] : 0.0;",
                                      "g_next[n] = 0.0;")],
    "bwd_final_history_grad_misplaced": [("dxa[L + k] += a->dconv_final[(b * D + d) * H + k];",
                                          "dxa[L + H - 1 - k] += a->dconv_final[(b * D + d) * H + k];")],
    # bidirectional
    "bidir_backward_runs_forward": [("const int64_t t = reverse ? L - 1 - i : i;", "const int64_t t = i;")],
    "bidir_backward_output_not_reversed": [("        acc[t] += out;", "        acc[i] += out;")],
    "bidir_backward_uses_forward_params": [("direction_channel(L, D, N, K, x, &bw, 1,", "direction_channel(L, D, N, K, x, &fw, 1,")],
    "bidir_merge_averaged": [("y[at] = z ? acc[t] * silu(z[at]) : acc[t];",
                              "y[at] = z ? 0.5 * acc[t] * silu(z[at]) : 0.5 * acc[t];")],
    "bidir_gate_dropped": [("y[at] = z ? acc[t] * silu(z[at]) : acc[t];", "y[at] = acc[t];")],
    "bidir_skip_dropped": [("double out = skip * uv;", "double out = 0.0 * uv;")],
    "bidir_decay_from_next_step": [("st[n] = exp(step * an) * st[n] + wn * p->Bm[bn + n] * uv;",
                                    "st[n] = exp(prevstep * an) * st[n] + wn * p->Bm[bn + n] * uv;"),
                                   ("        const double step = softplus(p->delta[at] + bias);",
                                    "        const double step = softplus(p->delta[at] + bias);\n"
                                    "        const double prevstep = i > 0 ? softplus(p->delta[(b * L + (reverse ? t + 1 : t - 1)) * D + d] + bias) : step;")],
    "bidir_zoh_ignored": [("const double wn = (zoh && an != 0.0) ?", "const double wn = (0 && an != 0.0) ?")],
    "bidir_conv_taps_reversed": [("cv += p->conv_w[d * K + k] * prev[k];", "cv += p->conv_w[d * K + (K - 2 - k)] * prev[k];")],
}


@pytest.fixture(scope="module")
def src():
    with open(oracle.SRC) as f:
        return f.read()


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name, src, tmp_path):
    s = src
    for old, new in MUTANTS[name]:
        assert s.count(old) == 1, f"mutation anchor not found once: {old!r}"
        s = s.replace(old, new)
    path = tmp_path / "mutant.c"
    path.write_text(s)
    lib = oracle.build(str(path), str(tmp_path / "libmutant.so"))
    orc = oracle.Oracle(lib)
    caught = []
    for pin in pins.ALL_PINS:
        try:
            pin(orc)
        except AssertionError:
            caught.append(pin.__name__)
    assert caught, f"mutant {name} passed every pin"
