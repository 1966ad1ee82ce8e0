"""Independent pins of the fp64 oracle.

Each pin checks the oracle against something other than itself: the unrolled
closed form of the recurrence, the LTI convolution-kernel view (by FFT), the
worked example on the ozercemkelahmet.com page, the pages' small/large step
size limits, a library convolution (torch conv1d) and library sigmoid /
softplus (scipy.special.expit, numpy.logaddexp). The zero-order-hold variant is
pinned to Van Loan's matrix-exponential form of the exact discretisation
(scipy.linalg.expm), to the continuous system's equilibrium and to the
composition property of the exact flow. Every pin takes an oracle
handle so that the same checks can be run on deliberately broken copies of
the oracle (tests/test_oracle_mutants.py) to show that they catch mistakes.

The pins never call the HIP library.
"""
from __future__ import annotations

import json
import math
import os

import numpy as np
import torch
from scipy.linalg import expm
from scipy.special import expit

HERE = os.path.dirname(os.path.abspath(__file__))


# ---------------------------------------------------------------------------
# small independent helpers (library routines, not the oracle's code)

def lib_softplus(v):
    return np.logaddexp(0.0, v)


def lib_silu(v):
    return v * expit(v)


def lib_conv_silu(x, conv_w, conv_b, conv_state):
    """u = SiLU(causal depthwise conv) through torch.nn.functional.conv1d.
    x [B,L,D], conv_w [D,K], conv_state [B,D,K-1] history (oldest first)."""
    Bsz, L, D = x.shape
    K = conv_w.shape[1]
    xt = torch.from_numpy(np.ascontiguousarray(np.transpose(x, (0, 2, 1)))).double()  # [B,D,L]
    hist = torch.zeros(Bsz, D, K - 1, dtype=torch.float64) if conv_state is None \
        else torch.from_numpy(np.asarray(conv_state, dtype=np.float64))
    full = torch.cat([hist, xt], dim=2)
    w = torch.from_numpy(np.asarray(conv_w, dtype=np.float64)).unsqueeze(1)  # [D,1,K]
    b = None if conv_b is None else torch.from_numpy(np.asarray(conv_b, dtype=np.float64))
    c = torch.nn.functional.conv1d(full, w, b, groups=D)  # [B,D,L]
    u = torch.nn.functional.silu(c)
    return np.transpose(u.numpy(), (0, 2, 1)), np.transpose(c.numpy(), (0, 2, 1))


def closed_form(x, delta, A, B, C, conv_w=None, conv_b=None, delta_bias=None, D=None, z=None,
                ssm_state=None, conv_state=None):
    """Unrolled solution of the recurrence, evaluated by brute force O(L^2 D N):
    y_t = sum_n C_t[n] (prod_{k<=t} Abar_k[n] h0[n] + sum_{s<=t} prod_{s<k<=t} Abar_k[n] Delta_s B_s[n] u_s)
          + D u_t, then times SiLU(z_t), with prod Abar = exp(A * sum of Delta)."""
    x = np.asarray(x, np.float64)
    Bsz, L, Dn = x.shape
    N = A.shape[1]
    if conv_w is not None:
        u, _ = lib_conv_silu(x, conv_w, conv_b, conv_state)
    else:
        u = x
    v = np.asarray(delta, np.float64) + (0.0 if delta_bias is None else np.asarray(delta_bias, np.float64))
    dt = lib_softplus(v)                                   # [B,L,D]
    cum = np.cumsum(dt, axis=1)                            # sum_{k<=t}
    y = np.zeros((Bsz, L, Dn))
    h_final = np.zeros((Bsz, Dn, N))
    h0 = np.zeros((Bsz, Dn, N)) if ssm_state is None else np.asarray(ssm_state, np.float64)
    for b in range(Bsz):
        for t in range(L):
            # contribution of the initial state: exp(A * cum_t)
            hv = np.exp(A * cum[b, t][:, None]) * h0[b]                       # [D,N]
            for s in range(t + 1):
                decay = np.exp(A * (cum[b, t] - cum[b, s])[:, None])            # [D,N]
                hv = hv + decay * (dt[b, s] * u[b, s])[:, None] * B[b, s][None, :]
            y[b, t] = (hv * C[b, t][None, :]).sum(axis=1)
            if t == L - 1:
                h_final[b] = hv
    if D is not None:
        y = y + np.asarray(D, np.float64)[None, None, :] * u
    if z is not None:
        y = y * lib_silu(np.asarray(z, np.float64))
    return y, h_final


def relerr(a, b):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    scale = max(np.max(np.abs(b)), math.sqrt(np.mean(b * b)) if b.size else 0.0, 1e-300)
    return float(np.max(np.abs(a - b)) / scale) if b.size else 0.0


def rand_case(rng, Bsz, L, D, N, K=4, conv=True, gate=True, skip=True, bias=True, states=False):
    c = dict(
        x=rng.standard_normal((Bsz, L, D)),
        delta=rng.standard_normal((Bsz, L, D)),
        A=-rng.uniform(0.2, 3.0, (D, N)),
        B=rng.standard_normal((Bsz, L, N)),
        C=rng.standard_normal((Bsz, L, N)),
    )
    if conv:
        c["conv_w"] = rng.uniform(-0.5, 0.5, (D, K))
        c["conv_b"] = rng.uniform(-0.2, 0.2, D)
    if bias:
        c["delta_bias"] = rng.uniform(-2.0, 0.5, D)
    if skip:
        c["D"] = rng.standard_normal(D)
    if gate:
        c["z"] = rng.standard_normal((Bsz, L, D))
    if states:
        c["ssm_state"] = rng.standard_normal((Bsz, D, N))
        if conv:
            c["conv_state"] = rng.standard_normal((Bsz, D, K - 1))
    return c


# ---------------------------------------------------------------------------
# pins

def pin_closed_form(orc, seed=1, shape=(2, 9, 3, 4), states=True):
    """The recurrence against its unrolled closed form (brute force)."""
    rng = np.random.default_rng(seed)
    c = rand_case(rng, *shape, states=states)
    y, h, _ = orc.conv_scan_fwd(**c)
    y_ref, h_ref = closed_form(**c)
    assert relerr(y, y_ref) < 1e-12, relerr(y, y_ref)
    if states:
        assert relerr(h, h_ref) < 1e-12, relerr(h, h_ref)


def pin_lti_fft(orc, seed=2, Bsz=1, L=64, D=3, N=5):
    """With Delta, B, C fixed over time the scan is a causal convolution of u with
    K_j[d] = sum_n C[n] Abar[d,n]^j Delta[d] B[n]; evaluated with numpy.fft."""
    rng = np.random.default_rng(seed)
    A = -rng.uniform(0.05, 1.0, (D, N))
    Bv = rng.standard_normal(N)
    Cv = rng.standard_normal(N)
    dpre = rng.uniform(-3.0, 0.0, D)
    x = rng.standard_normal((Bsz, L, D))
    delta = np.broadcast_to(dpre, (Bsz, L, D)).copy()
    Bm = np.broadcast_to(Bv, (Bsz, L, N)).copy()
    Cm = np.broadcast_to(Cv, (Bsz, L, N)).copy()
    Dsk = rng.standard_normal(D)
    y, _, _ = orc.conv_scan_fwd(x, delta, A, Bm, Cm, D=Dsk)
    dt = lib_softplus(dpre)
    j = np.arange(L)
    Ab = np.exp(dt[:, None] * A)                                           # [D,N]
    Kj = ((Cv * Bv)[None, None, :] * Ab[None, :, :] ** j[:, None, None]).sum(-1) * dt[None, :]  # [L,D]
    nfft = 2 * L
    Kf = np.fft.rfft(Kj, n=nfft, axis=0)
    for b in range(Bsz):
        yf = np.fft.irfft(np.fft.rfft(x[b], n=nfft, axis=0) * Kf, n=nfft, axis=0)[:L]
        ref = yf + Dsk[None, :] * x[b]
        assert relerr(y[b], ref) < 1e-12, relerr(y[b], ref)


def load_worked_example():
    with open(os.path.join(HERE, "golden", "worked_example.json")) as f:
        return json.load(f)


def pin_worked_example(orc):
    """The scalar walk-through of the ozercemkelahmet.com page, with delta = ln 2."""
    g = load_worked_example()
    inp = g["inputs"]
    u = np.array(inp["u"], np.float64)[None, :, None]
    L = u.shape[1]
    delta = np.array(inp["delta_pre_softplus"], np.float64)[None, :, None]
    A = np.array([[inp["A"]]])
    Bm = np.full((1, L, 1), inp["B"])
    Cm = np.full((1, L, 1), inp["C"])
    y, h, _ = orc.conv_scan_fwd(u, delta, A, Bm, Cm, D=np.array([inp["D"]]),
                                ssm_state=np.zeros((1, 1, 1)))
    want = np.array(g["expected"]["y_over_ln2"]) * math.log(2.0)
    assert np.max(np.abs(y[0, :, 0] - want)) <= 4e-16 * np.max(np.abs(want)), (y[0, :, 0], want)
    assert abs(h[0, 0, 0] - g["expected"]["final_state_over_ln2"] * math.log(2.0)) < 1e-15


def pin_selective_walkthrough(orc):
    """Same walk-through with a selective step size: large on the salient inputs
    (steps 1 and 4), tiny elsewhere. The state is rewritten on the salient steps
    and kept across the quiet ones, as the page describes."""
    u = np.array([1.0, 0.0, 0.0, 5.0, 0.0])[None, :, None]
    pre = np.array([20.0, -20.0, -20.0, 20.0, -20.0])[None, :, None]
    dt = lib_softplus(pre[0, :, 0])
    y, _, _ = orc.conv_scan_fwd(u, pre, np.array([[-1.0]]), np.ones((1, 5, 1)), np.ones((1, 5, 1)))
    y = y[0, :, 0]
    assert abs(y[0] - dt[0]) < 1e-12 * dt[0]
    assert abs(y[1] - y[0]) < 1e-7 * y[0] and abs(y[2] - y[0]) < 1e-7 * y[0]
    assert abs(y[3] - (math.exp(-dt[3]) * y[2] + dt[3] * 5.0)) < 1e-12 * y[3]
    assert abs(y[3] - dt[3] * 5.0) < 1e-6 * y[3]


def pin_small_step_keeps_state(orc, seed=3, shape=(2, 16, 4, 6)):
    """Delta -> 0 (pre-softplus -30): Abar -> 1 and the write term vanishes, so the
    state is kept: h_L = h_0 and y_t = C_t . h_0 + D u_t (times the gate)."""
    rng = np.random.default_rng(seed)
    c = rand_case(rng, *shape, bias=False, states=True)
    c["delta"] = np.full_like(c["delta"], -30.0)
    y, h, _ = orc.conv_scan_fwd(**c)
    assert relerr(h, c["ssm_state"]) < 1e-11
    u, _ = lib_conv_silu(c["x"], c["conv_w"], c["conv_b"], c["conv_state"])
    ref = np.einsum("bln,bdn->bld", c["C"], c["ssm_state"]) + c["D"] * u
    ref = ref * lib_silu(c["z"])
    assert relerr(y, ref) < 1e-11, relerr(y, ref)


def pin_large_step_forgets(orc, seed=4, shape=(2, 12, 3, 4)):
    """Large Delta (pre-softplus +50, A <= -1): Abar ~ e^-50, the old state is
    forgotten and h_t = Delta_t B_t u_t."""
    rng = np.random.default_rng(seed)
    c = rand_case(rng, *shape, bias=False, states=True)
    c["A"] = -np.broadcast_to(np.arange(1, shape[3] + 1, dtype=np.float64), (shape[2], shape[3])).copy()
    c["delta"] = np.full_like(c["delta"], 50.0)
    y, h, _ = orc.conv_scan_fwd(**c)
    u, _ = lib_conv_silu(c["x"], c["conv_w"], c["conv_b"], c["conv_state"])
    dt = lib_softplus(50.0)
    h_ref = dt * u[:, -1, :, None] * c["B"][:, -1, None, :]
    assert relerr(h, h_ref) < 1e-12
    ref = dt * u * np.einsum("bln,bln->bl", c["C"], c["B"])[:, :, None] + c["D"] * u
    ref = ref * lib_silu(c["z"])
    assert relerr(y, ref) < 1e-12


def _readout_u(orc, x, conv_w, conv_b=None, conv_state=None):
    """Observe u through the skip path: C = 0, D = 1, no gate -> y = u."""
    Bsz, L, D = x.shape
    N = 2
    y, _, cs = orc.conv_scan_fwd(x, np.zeros((Bsz, L, D)), -np.ones((D, N)), np.zeros((Bsz, L, N)),
                                 np.zeros((Bsz, L, N)), conv_w=conv_w, conv_b=conv_b, D=np.ones(D),
                                 conv_state=conv_state)
    return y, cs


def pin_conv_impulse(orc, seed=5, L=10, D=3, t0=3):
    """A unit impulse at t0 through the causal conv: pre-SiLU value at t0+j is
    conv_w[d, K-1-j] + bias (only current and past positions contribute)."""
    rng = np.random.default_rng(seed)
    w = rng.uniform(-0.5, 0.5, (D, 4))
    bias = rng.uniform(-0.2, 0.2, D)
    x = np.zeros((1, L, D))
    x[0, t0, :] = 1.0
    y, _ = _readout_u(orc, x, w, bias)
    c = np.tile(bias, (L, 1))
    for j in range(4):
        c[t0 + j] += w[:, 3 - j]
    assert relerr(y[0], lib_silu(c)) < 1e-14
    # identity filter: u = SiLU(x)
    x2 = rng.standard_normal((1, L, D))
    w2 = np.zeros((D, 4))
    w2[:, 3] = 1.0
    y2, _ = _readout_u(orc, x2, w2)
    assert relerr(y2, lib_silu(x2)) < 1e-14


def pin_conv_library(orc, seed=6, shape=(2, 11, 5)):
    """Conv front end with history against torch.nn.functional.conv1d, and the
    returned conv history equals the last K-1 inputs."""
    rng = np.random.default_rng(seed)
    x = rng.standard_normal(shape)
    w = rng.uniform(-0.5, 0.5, (shape[2], 4))
    bias = rng.uniform(-0.2, 0.2, shape[2])
    hist = rng.standard_normal((shape[0], shape[2], 3))
    y, cs = _readout_u(orc, x, w, bias, hist)
    u, _ = lib_conv_silu(x, w, bias, hist)
    assert relerr(y, u) < 1e-14
    assert np.array_equal(cs, np.transpose(x[:, -3:, :], (0, 2, 1)))


def pin_gate_and_skip(orc, seed=7, shape=(1, 8, 4, 3)):
    """z = 0 gives 0; the gate multiplies by SiLU(z); C = 0 leaves D*u*SiLU(z)."""
    rng = np.random.default_rng(seed)
    c = rand_case(rng, *shape)
    y_g, _, _ = orc.conv_scan_fwd(**c)
    c0 = dict(c)
    c0["z"] = np.zeros_like(c["z"])
    y0, _, _ = orc.conv_scan_fwd(**c0)
    assert np.all(y0 == 0.0)
    cu = dict(c)
    cu.pop("z")
    y_u, _, _ = orc.conv_scan_fwd(**cu)
    assert relerr(y_g, y_u * lib_silu(c["z"])) < 1e-14
    cc = dict(c)
    cc["C"] = np.zeros_like(c["C"])
    y_c, _, _ = orc.conv_scan_fwd(**cc)
    u, _ = lib_conv_silu(c["x"], c["conv_w"], c["conv_b"], None)
    assert relerr(y_c, c["D"] * u * lib_silu(c["z"])) < 1e-14


def pin_softplus_sum(orc, seed=8, L=40, D=3):
    """With A = 0 the decay is 1 and, for N = 1, B = C = 1, u = 1, the output is the
    running sum of the step sizes: checks softplus (with bias) over a wide range."""
    rng = np.random.default_rng(seed)
    pre = rng.uniform(-40.0, 40.0, (1, L, D))
    bias = rng.uniform(-1.0, 1.0, D)
    y, _, _ = orc.conv_scan_fwd(np.ones((1, L, D)), pre, np.zeros((D, 1)), np.ones((1, L, 1)),
                                np.ones((1, L, 1)), delta_bias=bias)
    ref = np.cumsum(lib_softplus(pre + bias), axis=1)
    assert relerr(y, ref) < 1e-13


def pin_state_handoff(orc, seed=9, shape=(2, 23, 3, 4), splits=(1, 7, 16, 22)):
    """Processing a sequence in two chunks, passing (ssm_state, conv_state) from
    the first to the second, gives the same outputs as one pass."""
    rng = np.random.default_rng(seed)
    c = rand_case(rng, *shape, states=True)
    y, h, cs = orc.conv_scan_fwd(**c)
    for L1 in splits:
        def part(sl, st_h, st_c):
            d = dict(c)
            for k in ("x", "delta", "z", "B", "C"):
                d[k] = c[k][:, sl]
            d["ssm_state"], d["conv_state"] = st_h, st_c
            return orc.conv_scan_fwd(**d)
        y1, h1, c1 = part(slice(0, L1), c["ssm_state"], c["conv_state"])
        y2, h2, c2 = part(slice(L1, None), h1, c1)
        assert relerr(np.concatenate([y1, y2], axis=1), y) < 1e-13
        assert relerr(h2, h) < 1e-13 and np.array_equal(c2, cs)


def pin_step_matches_scan(orc, seed=10, shape=(3, 6, 4, 5)):
    """L decode steps from a carried state reproduce the full-sequence pass."""
    rng = np.random.default_rng(seed)
    c = rand_case(rng, *shape, states=True)
    y, h, cs = orc.conv_scan_fwd(**c)
    hs, css = c["ssm_state"], c["conv_state"]
    ys = []
    for t in range(shape[1]):
        yt, hs, css = orc.step(c["x"][:, t], c["delta"][:, t], c["A"], c["B"][:, t], c["C"][:, t], hs,
                               conv_w=c["conv_w"], conv_b=c["conv_b"], delta_bias=c["delta_bias"],
                               D=c["D"], z=c["z"][:, t], conv_state=css)
        ys.append(yt)
    assert relerr(np.stack(ys, axis=1), y) < 1e-13
    assert relerr(hs, h) < 1e-13 and np.array_equal(css, cs)


# ---------------------------------------------------------------------------
# zero-order hold (inferensys.com "Mamba", the discretization bullet; the
# ai360xpert.com "Mamba" code section writes the same "simplified ZOH" term)

def inv_softplus(dt):
    """Pre-activation whose softplus is dt (dt > 0)."""
    return np.log(np.expm1(np.asarray(dt, np.float64)))


def pin_zoh_van_loan(orc, seed=11, shape=(2, 7, 3, 5)):
    """ZOH is the exact solution of h' = a h + b u over one step of length Delta
    with u, b held. Van Loan: expm(Delta [[a, b u], [0, 0]]) has the transition
    exp(a Delta) top-left and the held-input response top-right. Chaining those
    2x2 transitions from h0 (library expm, no recurrence formula) and reading out
    C . h must give the oracle's ZOH scan, including a = 0 and a -> 0 states."""
    rng = np.random.default_rng(seed)
    Bsz, L, D, N = shape
    c = rand_case(rng, *shape, states=True)
    c["A"][:, 0] = 0.0
    c["A"][:, 1] = -1e-9
    y, h, _ = orc.conv_scan_fwd(**c, zoh=True)
    u, _ = lib_conv_silu(c["x"], c["conv_w"], c["conv_b"], c["conv_state"])
    dt = lib_softplus(c["delta"] + c["delta_bias"])
    y_ref = np.zeros((Bsz, L, D))
    h_ref = np.zeros((Bsz, D, N))
    for b in range(Bsz):
        for d in range(D):
            for n in range(N):
                v = np.array([c["ssm_state"][b, d, n], 1.0])
                for t in range(L):
                    gen = np.array([[c["A"][d, n], c["B"][b, t, n] * u[b, t, d]], [0.0, 0.0]])
                    v = expm(dt[b, t, d] * gen) @ v
                    y_ref[b, t, d] += c["C"][b, t, n] * v[0]
                h_ref[b, d, n] = v[0]
    y_ref = (y_ref + c["D"] * u) * lib_silu(c["z"])
    assert relerr(y, y_ref) < 1e-12, relerr(y, y_ref)
    assert relerr(h, h_ref) < 1e-12, relerr(h, h_ref)


def pin_zoh_equilibrium(orc, seed=12, L=30, D=3, N=4):
    """With u and B held, h* = -B u / a is the equilibrium of the continuous
    system and so a fixed point of its exact discretisation for every step size:
    a state started there stays there while Delta varies wildly from step to step,
    and y_t = C_t . h* + D u."""
    rng = np.random.default_rng(seed)
    A = -rng.uniform(0.2, 3.0, (D, N))
    Bv = rng.standard_normal(N)
    uv = rng.standard_normal(D)
    hstar = -(uv[:, None] * Bv[None, :]) / A
    x = np.broadcast_to(uv, (1, L, D)).copy()
    Bm = np.broadcast_to(Bv, (1, L, N)).copy()
    Cm = rng.standard_normal((1, L, N))
    Dsk = rng.standard_normal(D)
    y, h, _ = orc.conv_scan_fwd(x, rng.uniform(-6.0, 6.0, (1, L, D)), A, Bm, Cm, D=Dsk,
                                ssm_state=hstar[None], zoh=True)
    assert relerr(h[0], hstar) < 1e-13, relerr(h[0], hstar)
    ref = np.einsum("ln,dn->ld", Cm[0], hstar) + Dsk * uv
    assert relerr(y[0], ref) < 1e-13, relerr(y[0], ref)


def pin_zoh_composition(orc, seed=13, D=3, N=4):
    """The exact flow composes: with u, B held, two ZOH steps of sizes Delta1 and
    Delta2 reach the same state as one step of Delta1 + Delta2."""
    rng = np.random.default_rng(seed)
    A = -rng.uniform(0.2, 3.0, (D, N))
    Bv = rng.standard_normal(N)
    uv = rng.standard_normal(D)
    h0 = rng.standard_normal((1, D, N))
    d1 = rng.uniform(0.05, 2.0, D)
    d2 = rng.uniform(0.05, 2.0, D)

    def run(steps):
        L = len(steps)
        pre = inv_softplus(np.stack(steps))[None]
        _, h, _ = orc.conv_scan_fwd(np.broadcast_to(uv, (1, L, D)).copy(), pre, A,
                                    np.broadcast_to(Bv, (1, L, N)).copy(), np.zeros((1, L, N)),
                                    ssm_state=h0, zoh=True)
        return h

    h_two = run([d1, d2])
    h_one = run([d1 + d2])
    assert relerr(h_two, h_one) < 1e-12, relerr(h_two, h_one)


ALL_PINS = [
    pin_closed_form, pin_lti_fft, pin_worked_example, pin_selective_walkthrough,
    pin_small_step_keeps_state, pin_large_step_forgets, pin_conv_impulse, pin_conv_library,
    pin_gate_and_skip, pin_softplus_sum, pin_state_handoff, pin_step_matches_scan,
    pin_zoh_van_loan, pin_zoh_equilibrium, pin_zoh_composition,
]


# ---------------------------------------------------------------------------
# backward (gradients through the forward): the hand-derived adjoint sweep of the
# oracle against (1) central finite differences of the forward oracle and (2)
# torch float64 autograd through an independently written forward.

GRAD_INPUTS = ("x", "delta", "z", "B", "C", "A", "D", "conv_w", "conv_b", "delta_bias", "ssm_state", "conv_state")
GRAD_NAME = {"x": "dx", "delta": "ddelta", "z": "dz", "B": "dB", "C": "dC", "A": "dA", "D": "dD",
             "conv_w": "dconv_w", "conv_b": "dconv_b", "delta_bias": "ddelta_bias",
             "ssm_state": "dstate_init", "conv_state": "dconv_init"}


def bwd_case(seed, shape=(2, 7, 3, 4), zoh=False):
    rng = np.random.default_rng(seed)
    c = rand_case(rng, *shape, states=True)
    Bsz, L, D, N = shape
    cot = dict(dy=rng.standard_normal((Bsz, L, D)), dstate_final=rng.standard_normal((Bsz, D, N)),
               dconv_final=rng.standard_normal((Bsz, D, 3)))
    return c, cot


def loss_of(orc, c, cot, zoh):
    y, h, cs = orc.conv_scan_fwd(**c, zoh=zoh)
    return float(np.sum(cot["dy"] * y) + np.sum(cot["dstate_final"] * h) + np.sum(cot["dconv_final"] * cs))


def _pin_bwd_fd(orc, zoh, seed, eps=1e-6):
    c, cot = bwd_case(seed, zoh=zoh)
    g = orc.conv_scan_bwd(**c, **cot, zoh=zoh)
    rng = np.random.default_rng(seed + 1000)
    for name in GRAD_INPUTS:
        v = rng.standard_normal(np.shape(c[name]))
        cp, cm = dict(c), dict(c)
        cp[name] = c[name] + eps * v
        cm[name] = c[name] - eps * v
        fd = (loss_of(orc, cp, cot, zoh) - loss_of(orc, cm, cot, zoh)) / (2 * eps)
        an = float(np.sum(g[GRAD_NAME[name]] * v))
        assert abs(fd - an) <= 1e-6 * max(1.0, abs(an)), (name, fd, an)


def pin_bwd_finite_differences(orc, seed=21):
    """Directional derivative of the loss along a random direction, for every input
    tensor: central difference of the forward oracle vs the backward's gradient."""
    _pin_bwd_fd(orc, False, seed)


def pin_bwd_finite_differences_zoh(orc, seed=22):
    _pin_bwd_fd(orc, True, seed)


def torch_forward(c, zoh):
    """The forward written with torch ops (float64), for autograd: conv over the
    history-padded input, SiLU, softplus as logaddexp(v, 0), the recurrence over t
    with the Euler or zero-order-hold write term, readout, skip and SiLU gate."""
    x, delta, A, B, C = c["x"], c["delta"], c["A"], c["B"], c["C"]
    Bsz, L, D = x.shape
    xp = torch.cat([c["conv_state"].transpose(1, 2), x], dim=1)               # [B, L+3, D]
    pre = c["conv_b"] + sum(c["conv_w"][:, k] * xp[:, k:k + L, :] for k in range(4))
    u = pre * torch.sigmoid(pre)
    dt = torch.logaddexp(delta + c["delta_bias"], torch.zeros((), dtype=torch.float64))
    h = c["ssm_state"]
    ys = []
    for t in range(L):
        at = dt[:, t, :, None] * A                                             # [B, D, N]
        w = torch.expm1(at) / A if zoh else dt[:, t, :, None]
        h = torch.exp(at) * h + w * B[:, t, None, :] * u[:, t, :, None]
        ys.append((h * C[:, t, None, :]).sum(-1) + c["D"] * u[:, t])
    y = torch.stack(ys, 1) * (c["z"] * torch.sigmoid(c["z"]))
    return y, h, xp[:, L:L + 3, :].transpose(1, 2)


def _pin_bwd_autograd(orc, zoh, seed):
    c, cot = bwd_case(seed, shape=(2, 6, 3, 5), zoh=zoh)
    g = orc.conv_scan_bwd(**c, **cot, zoh=zoh)
    tc = {k: torch.tensor(v, dtype=torch.float64, requires_grad=True) for k, v in c.items()}
    y, h, cs = torch_forward(tc, zoh)
    loss = ((y * torch.from_numpy(cot["dy"])).sum() + (h * torch.from_numpy(cot["dstate_final"])).sum()
            + (cs * torch.from_numpy(cot["dconv_final"])).sum())
    names = list(GRAD_INPUTS)
    grads = torch.autograd.grad(loss, [tc[n] for n in names])
    for n, tg in zip(names, grads):
        ref = tg.numpy()
        assert relerr(g[GRAD_NAME[n]], ref) < 1e-10, (n, relerr(g[GRAD_NAME[n]], ref))


def pin_bwd_autograd(orc, seed=23):
    """Every gradient element against torch autograd through torch_forward."""
    _pin_bwd_autograd(orc, False, seed)


def pin_bwd_autograd_zoh(orc, seed=24):
    _pin_bwd_autograd(orc, True, seed)


def pin_bwd_without_optional_pieces(orc, seed=25):
    """No conv, gate, skip, bias or initial states: the gradients that remain still
    match autograd (u = x, ungated output, zero initial state)."""
    rng = np.random.default_rng(seed)
    c = rand_case(rng, 1, 5, 2, 3, conv=False, gate=False, skip=False, bias=False)
    dy = rng.standard_normal((1, 5, 2))
    g = orc.conv_scan_bwd(**c, dy=dy)
    assert set(g) == {"dx", "ddelta", "dB", "dC", "dA", "dstate_init"}
    tc = {k: torch.tensor(v, dtype=torch.float64, requires_grad=True) for k, v in c.items()}
    dt = torch.logaddexp(tc["delta"], torch.zeros((), dtype=torch.float64))
    h = torch.zeros(1, 2, 3, dtype=torch.float64)
    ys = []
    for t in range(5):
        h = torch.exp(dt[:, t, :, None] * tc["A"]) * h + dt[:, t, :, None] * tc["B"][:, t, None, :] * tc["x"][:, t, :, None]
        ys.append((h * tc["C"][:, t, None, :]).sum(-1))
    loss = (torch.stack(ys, 1) * torch.from_numpy(dy)).sum()
    for n, tg in zip(("x", "delta", "B", "C", "A"), torch.autograd.grad(loss, [tc[k] for k in ("x", "delta", "B", "C", "A")])):
        assert relerr(g[GRAD_NAME[n]], tg.numpy()) < 1e-10, n
    assert np.all(g["dstate_init"] != 0.0)


BWD_PINS = [pin_bwd_finite_differences, pin_bwd_finite_differences_zoh, pin_bwd_autograd, pin_bwd_autograd_zoh,
            pin_bwd_without_optional_pieces]
ALL_PINS = ALL_PINS + BWD_PINS


# ---------------------------------------------------------------------------
# bidirectional scan (ozercemkelahmet.com "Mamba", "Variants and extensions")

def lib_anticausal_conv_silu(x, conv_w, conv_b):
    """u' = SiLU(conv_b + sum_k conv_w[k] x_{t+(K-1)-k}), zeros past the end, through
    torch.nn.functional.conv1d (a cross-correlation) on the right-padded input with the
    taps in reverse order."""
    Bsz, L, D = x.shape
    K = conv_w.shape[1]
    xt = torch.from_numpy(np.ascontiguousarray(np.transpose(x, (0, 2, 1)))).double()
    full = torch.cat([xt, torch.zeros(Bsz, D, K - 1, dtype=torch.float64)], dim=2)
    w = torch.from_numpy(np.ascontiguousarray(np.asarray(conv_w, np.float64)[:, ::-1])).unsqueeze(1)
    b = None if conv_b is None else torch.from_numpy(np.asarray(conv_b, np.float64))
    c = torch.nn.functional.conv1d(full, w, b, groups=D)
    return np.transpose(torch.nn.functional.silu(c).numpy(), (0, 2, 1))


def brute_bidir(x, fwd, rev, z=None, zoh=False):
    """Both directions unrolled by brute force, O(L^2 D N):
    forward  h_t = sum_{s<=t} exp(A sum_{s<k<=t} Delta_k) W_s B_s u_s,
    backward g_t = sum_{s>=t} exp(A' sum_{t<=k<s} Delta'_k) W'_s B'_s u'_s,
    y_t = (C_t.h_t + D u_t + C'_t.g_t + D' u'_t) SiLU(z_t); W = Delta (Euler) or
    expm1(Delta A)/A (zero-order hold)."""
    x = np.asarray(x, np.float64)
    Bsz, L, Dn = x.shape
    out = np.zeros((Bsz, L, Dn))
    for q, backward in ((fwd, False), (rev, True)):
        A = np.asarray(q["A"], np.float64)
        if q.get("conv_w") is None:
            u = x
        elif backward:
            u = lib_anticausal_conv_silu(x, q["conv_w"], q.get("conv_b"))
        else:
            u, _ = lib_conv_silu(x, q["conv_w"], q.get("conv_b"), None)
        v = np.asarray(q["delta"], np.float64) + (0.0 if q.get("delta_bias") is None else q["delta_bias"])
        dt = lib_softplus(v)
        for b in range(Bsz):
            for t in range(L):
                hv = np.zeros(A.shape)
                srange = range(t, L) if backward else range(t + 1)
                for s in srange:
                    span = dt[b, t:s].sum(0) if backward else dt[b, s + 1:t + 1].sum(0)   # [D]
                    decay = np.exp(A * span[:, None])
                    w = (np.expm1(dt[b, s][:, None] * A) / A) if zoh else dt[b, s][:, None]
                    hv = hv + decay * w * u[b, s][:, None] * np.asarray(q["B"], np.float64)[b, s][None, :]
                out[b, t] += (hv * np.asarray(q["C"], np.float64)[b, t][None, :]).sum(1)
        if q.get("D") is not None:
            out += np.asarray(q["D"], np.float64)[None, None, :] * u
    if z is not None:
        out *= lib_silu(np.asarray(z, np.float64))
    return out


def bidir_case(seed, shape=(2, 9, 3, 4), separate=True, conv=True):
    rng = np.random.default_rng(seed)
    c = rand_case(rng, *shape, conv=conv, states=False)
    keys = ("conv_w", "conv_b", "delta", "delta_bias", "A", "B", "C", "D")
    fwd = {k: c[k] for k in keys if k in c}
    if separate:
        r = rand_case(rng, *shape, conv=conv, states=False)
        rev = {k: r[k] for k in keys if k in r}
    else:
        rev = dict(fwd)
    return c["x"], c.get("z"), fwd, rev


def _bidir_call(orc, x, z, fwd, rev, zoh=False, shared=False):
    return orc.conv_scan_bidir(x, fwd["delta"], fwd["A"], fwd["B"], fwd["C"], conv_w=fwd.get("conv_w"),
                               conv_b=fwd.get("conv_b"), delta_bias=fwd.get("delta_bias"), D=fwd.get("D"), z=z,
                               rev=None if shared else rev, zoh=zoh)


def pin_bidir_closed_form(orc, seed=31):
    """Both directions against their unrolled closed forms, separate and shared
    parameters (the anti-causal conv through torch conv1d)."""
    for i, separate in enumerate((True, False)):
        x, z, fwd, rev = bidir_case(seed + i, separate=separate)
        y = _bidir_call(orc, x, z, fwd, rev, shared=not separate)
        ref = brute_bidir(x, fwd, rev, z)
        assert relerr(y, ref) < 1e-12, relerr(y, ref)


def pin_bidir_closed_form_zoh(orc, seed=33):
    x, z, fwd, rev = bidir_case(seed, shape=(1, 8, 3, 4))
    y = _bidir_call(orc, x, z, fwd, rev, zoh=True)
    ref = brute_bidir(x, fwd, rev, z, zoh=True)
    assert relerr(y, ref) < 1e-12, relerr(y, ref)


def pin_bidir_lti_fft(orc, seed=34, Bsz=2, L=48, D=3, N=5):
    """Delta, B, C fixed over time, shared parameters, no conv: the output is a
    two-sided convolution y_t = sum_{s<=t} K_{t-s} u_s + sum_{s>=t} K_{s-t} u_s + 2 D u_t
    with the LTI kernel K_j = sum_n C[n] exp(Delta A[n])^j Delta B[n], by numpy.fft."""
    rng = np.random.default_rng(seed)
    A = -rng.uniform(0.05, 1.0, (D, N))
    Bv, Cv = rng.standard_normal(N), rng.standard_normal(N)
    dpre = rng.uniform(-3.0, 0.0, D)
    x = rng.standard_normal((Bsz, L, D))
    Dsk = rng.standard_normal(D)
    delta = np.broadcast_to(dpre, (Bsz, L, D)).copy()
    Bm = np.broadcast_to(Bv, (Bsz, L, N)).copy()
    Cm = np.broadcast_to(Cv, (Bsz, L, N)).copy()
    y = orc.conv_scan_bidir(x, delta, A, Bm, Cm, D=Dsk)
    dt = lib_softplus(dpre)
    j = np.arange(L)
    Kj = ((Cv * Bv)[None, None, :] * np.exp(dt[:, None] * A)[None] ** j[:, None, None]).sum(-1) * dt[None, :]
    nfft = 2 * L
    Kf = np.fft.rfft(Kj, n=nfft, axis=0)
    for b in range(Bsz):
        causal = np.fft.irfft(np.fft.rfft(x[b], n=nfft, axis=0) * Kf, n=nfft, axis=0)[:L]
        anti = np.fft.irfft(np.fft.rfft(x[b][::-1], n=nfft, axis=0) * Kf, n=nfft, axis=0)[:L][::-1]
        ref = causal + anti + 2.0 * Dsk[None, :] * x[b]
        assert relerr(y[b], ref) < 1e-12, relerr(y[b], ref)


def pin_bidir_mirror(orc, seed=35):
    """Reversing the sequence and exchanging the two directions' parameters reverses
    the output."""
    x, z, fwd, rev = bidir_case(seed, shape=(2, 11, 3, 4))
    y = _bidir_call(orc, x, z, fwd, rev)
    flip = lambda q: {k: (v[:, ::-1].copy() if k in ("delta", "B", "C") else v) for k, v in q.items()}  # noqa: E731
    ym = _bidir_call(orc, x[:, ::-1].copy(), z[:, ::-1].copy(), flip(rev), flip(fwd))
    assert relerr(ym[:, ::-1], y) < 1e-13, relerr(ym[:, ::-1], y)


BIDIR_PINS = [pin_bidir_closed_form, pin_bidir_closed_form_zoh, pin_bidir_lti_fft, pin_bidir_mirror]
ALL_PINS = ALL_PINS + BIDIR_PINS
