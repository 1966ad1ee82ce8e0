"""Plant plausible mistakes in copies of the oracle (on the CPU) and check that
the pins catch every one of them. The oracle source is never modified: each
mutant is a patched copy compiled into a temporary directory."""
import os

import pytest

import oracle
import pins

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
    "decay_sign_flipped": [("exp(dt * A[d * N + n])", "exp(-dt * A[d * N + n])")],
    "zoh_instead_of_euler": [("h[n] = abar * h[n] + dt * Bm[bc + n] * u;",
                              "h[n] = abar * h[n] + (1.0 - abar) / (-A[d * N + n]) * Bm[bc + n] * u;")],
    "write_term_without_delta": [("h[n] = abar * h[n] + dt * Bm[bc + n] * u;",
                                  "h[n] = abar * h[n] + Bm[bc + n] * u;")],
    "state_not_carried": [("h[n] = abar * h[n] + dt", "h[n] = abar * 0.0 + dt")],
    "B_and_C_swapped": [("dt * Bm[bc + n] * u", "dt * Cm[bc + n] * u"),
                        ("yt += Cm[bc + n] * h[n];", "yt += Bm[bc + n] * h[n];")],
    "readout_before_update": [
        ("""        for (int64_t n = 0; n < N; ++n) {
            const double abar = exp(dt * A[d * N + n]);
            h[n] = abar * h[n] + dt * Bm[bc + n] * u;
        }

        double yt = 0.0;
        for (int64_t n = 0; n < N; ++n) yt += Cm[bc + n] * h[n];""",
         """        double yt = 0.0;
        for (int64_t n = 0; n < N; ++n) yt += Cm[bc + n] * h[n];
        for (int64_t n = 0; n < N; ++n) {
            const double abar = exp(dt * A[d * N + n]);
            h[n] = abar * h[n] + dt * Bm[bc + n] * u;
        }""")],
    "skip_dropped": [("yt += (Dskip ? Dskip[d] : 0.0) * u;", "yt += 0.0 * u;")],
    "skip_uses_x": [("yt += (Dskip ? Dskip[d] : 0.0) * u;", "yt += (Dskip ? Dskip[d] : 0.0) * xt;")],
    "gate_sigmoid_not_silu": [("if (z) yt *= silu(z[row]);", "if (z) yt *= 1.0 / (1.0 + exp(-z[row]));")],
    "gate_before_skip": [("""        yt += (Dskip ? Dskip[d] : 0.0) * u;

        if (z) yt *= silu(z[row]);""", """        if (z) yt *= silu(z[row]);
        yt += (Dskip ? Dskip[d] : 0.0) * u;""")],
    "initial_state_ignored": [("h[n] = ssm_state ? ssm_state[(b * D + d) * N + n] : 0.0;", "h[n] = 0.0;")],
    "conv_history_ignored": [("win[k] = conv_state ? conv_state[(b * D + d) * (K - 1) + k] : 0.0;",
                              "win[k] = 0.0;")],
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
