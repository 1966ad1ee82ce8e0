"""GPU parity at the step size's two limits (ai360xpert.com "Mamba", "The selection
mechanism"; ozercemkelahmet.com "Mamba", "Step 3"): a tiny step keeps the state,
a large one forgets it.

- delta = -30: Delta = softplus(-30 + b) < 1e-13, so exp(Delta A) rounds to 1 in fp32
  and the write term vanishes: h_L = h_0 and y_t = (C_t . h_0 + D u_t) SiLU(z_t).
- delta = +50 with A <= -1: exp(Delta A) < 1e-20, so h_t = W_t B_t u_t with W_t =
  Delta_t (Euler) or -1/A (zero-order hold), independent of h_{t-1}.
- a sequence that switches between the two (and ordinary steps) every few hundred
  tokens, so that some chunks' aggregate sweeps drop no state index and others drop
  every index after their first group (and the carry correction runs to a chunk's
  end or drops every carry at once).

Every case runs on each forward path (one-lane chunked kernels with the aggregate
pass, one-lane kernels with the carry correction, lane-quad kernels, the decode
step, the zero-order hold, the bidirectional reversed pass), compared element by
element with the fp64 oracle at the fp32 bar,
and the two limits are also checked against their closed forms directly."""
import numpy as np
import pytest
import torch

import oracle
import workloads as W
from gpu_util import TOL, check_inputs, host, maxrel, to_dev
from test_gpu_bidir import check_bidir

pytestmark = pytest.mark.gpu

SMALL, LARGE = np.float32(-30.0), np.float32(50.0)

# (batch, seqlen, d_inner): one-lane chunked shapes with 256-token chunks (aggregate
# pass first) and 1024-token chunks (carry correction after), and a lane-quad shape
ONE_LANE = (2, 16384, 1024)
CARRY = (2, 65536, 1024)
QUAD = (1, 4096, 64)
SHAPES = {"one_lane": ONE_LANE, "carry": CARRY, "quad": QUAD}


@pytest.fixture(scope="module")
def ss():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import selective_state_space_73_amd as mod
    return mod


def _inputs(shape, seed, io="f32"):
    Bsz, L, Dn = shape
    spec = W.ScanSpec("lim", Bsz, L, Dn, 16, io_dtype=io, delta_mode="bias", seed=seed)
    return W.gen_scan_inputs(spec)


def _plan(ss, shape, io="f32", zoh=False, pass_=0):
    Bsz, L, Dn = shape
    dims = ss.make_dims(Bsz, L, Dn, 16, 0 if io == "f32" else 1,
                        discretization=ss.SS_ZOH if zoh else ss.SS_EULER)
    return ss.ss_scan_plan(dims, pass_)


def _assert_path(ss, shape, quad, pass_=0, carry=False):
    p = _plan(ss, shape, pass_=pass_)
    assert p["nchunks"] > 1, p
    assert p["lane_quad"] == quad, p
    assert p["carry_correction"] == carry, p


def _mixed_delta(L):
    """Segments of 700 tokens at delta = -30, 300 at +50 and 500 ordinary (N(0,1)),
    repeating: chunks inside the first kind keep every state, the second forget."""
    pattern = np.concatenate([np.full(700, SMALL), np.full(300, LARGE), np.full(500, np.nan, np.float32)])
    return np.resize(pattern, L)


DSEL = np.array([0, 1, 63, 64, 255, 256, 700, 1023])


@pytest.mark.parametrize("zoh", [False, True], ids=["euler", "zoh"])
@pytest.mark.parametrize("path", ["one_lane", "carry", "quad"])
def test_small_step_keeps_the_state(ss, path, zoh):
    shape = SHAPES[path]
    _assert_path(ss, shape, path == "quad", carry=path == "carry")
    inp = _inputs(shape, 301)
    inp["delta"][:] = SMALL
    Bsz, L, Dn = shape
    dsel = DSEL[DSEL < Dn]
    st = W.gen_states(Bsz, Dn, 16, seed=302)
    check_inputs(ss, inp, "f32", states=True, dsel=dsel, zoh=zoh, label=f"small step {path}",
                 state_tol=TOL["f32"])
    # closed form on the GPU side alone: the returned state is the initial one
    g = to_dev(inp, "f32")
    h = torch.from_numpy(st["ssm_state"]).cuda()
    c = torch.from_numpy(st["conv_state"]).cuda()
    y = ss.ss_conv_scan_fwd(g["x"], g["delta"], g["A"], g["B"], g["C"], conv_w=g["conv_w"], conv_b=g["conv_b"],
                            delta_bias=g["delta_bias"], D=g["D"], z=g["z"], ssm_state=h, conv_state=c, zoh=zoh)
    torch.cuda.synchronize()
    assert maxrel(host(h), st["ssm_state"]) <= 1e-6
    # y_t = (C_t . h_0 + D u_t) SiLU(z_t), with u from the conv of the oracle's own
    # window (the conv history is exact, checked above): compare on the sample
    x = inp["x"].astype(np.float64)
    cw, cb = inp["conv_w"].astype(np.float64), inp["conv_b"].astype(np.float64)
    hist = st["conv_state"].astype(np.float64)
    xp = np.concatenate([hist.transpose(0, 2, 1), x], axis=1)               # [B, L+3, D]
    cpre = cb + sum(cw[:, k] * xp[:, k:k + L] for k in range(4))
    u = cpre / (1.0 + np.exp(-cpre))
    zz = inp["z"].astype(np.float64)
    gate = zz / (1.0 + np.exp(-zz))
    ch0 = np.einsum("bln,bdn->bld", inp["C"].astype(np.float64), st["ssm_state"].astype(np.float64))
    want = (ch0 + inp["D"].astype(np.float64) * u) * gate
    e = maxrel(host(y)[:, :, dsel], want[:, :, dsel])
    print(f"small step {path} closed form y maxrel {e:.3e}", flush=True)
    assert e <= TOL["f32"]


@pytest.mark.parametrize("zoh", [False, True], ids=["euler", "zoh"])
@pytest.mark.parametrize("path", ["one_lane", "carry", "quad"])
def test_large_step_forgets_the_state(ss, path, zoh):
    shape = SHAPES[path]
    _assert_path(ss, shape, path == "quad", carry=path == "carry")
    inp = _inputs(shape, 311)
    inp["delta"][:] = LARGE
    Bsz, L, Dn = shape
    dsel = DSEL[DSEL < Dn]
    check_inputs(ss, inp, "f32", states=True, dsel=dsel, zoh=zoh, label=f"large step {path}",
                 state_tol=TOL["f32"])
    # closed form: h_L = W B_{L-1} u_{L-1} whatever the initial state
    g = to_dev(inp, "f32")
    h = torch.from_numpy(W.gen_states(Bsz, Dn, 16, seed=312)["ssm_state"]).cuda()
    ss.ss_conv_scan_fwd(g["x"], g["delta"], g["A"], g["B"], g["C"], conv_w=g["conv_w"], conv_b=g["conv_b"],
                        delta_bias=g["delta_bias"], D=g["D"], z=g["z"], ssm_state=h, zoh=zoh)
    torch.cuda.synchronize()
    x = inp["x"][:, -4:].astype(np.float64)                                   # [B, 4, D]
    cpre = inp["conv_b"].astype(np.float64) + np.einsum("bkd,dk->bd", x, inp["conv_w"].astype(np.float64))
    u = cpre / (1.0 + np.exp(-cpre))                                          # [B, D]
    v = LARGE + inp["delta_bias"].astype(np.float64)
    dt = v + np.log1p(np.exp(-v))                                             # [D]
    A = inp["A"].astype(np.float64)
    W_ = (-1.0 / A) * np.ones_like(dt)[:, None] if zoh else dt[:, None] * np.ones_like(A)
    want = W_[None] * inp["B"][:, -1, None, :].astype(np.float64) * u[:, :, None]
    e = maxrel(host(h)[:, dsel], want[:, dsel])
    print(f"large step {path} closed form state maxrel {e:.3e}", flush=True)
    assert e <= TOL["f32"]


@pytest.mark.parametrize("zoh", [False, True], ids=["euler", "zoh"])
@pytest.mark.parametrize("path", ["one_lane", "carry", "quad"])
def test_switching_steps(ss, path, zoh):
    shape = SHAPES[path]
    _assert_path(ss, shape, path == "quad", carry=path == "carry")
    inp = _inputs(shape, 321)
    mix = _mixed_delta(shape[1])
    keep = ~np.isnan(mix)
    inp["delta"][:, keep, :] = mix[keep][None, :, None]
    dsel = DSEL[DSEL < shape[2]]
    check_inputs(ss, inp, "f32", states=True, dsel=dsel, zoh=zoh, label=f"switching {path}", state_tol=TOL["f32"])


@pytest.mark.parametrize("kind", ["small", "large", "switching"])
def test_limits_bf16_one_lane(ss, kind):
    """The same limits with bf16 inputs (-30 and 50 are exact in bf16) at the bf16 bar."""
    inp = _inputs(ONE_LANE, 331, io="bf16")
    if kind == "switching":
        mix = _mixed_delta(ONE_LANE[1])
        keep = ~np.isnan(mix)
        inp["delta"][:, keep, :] = mix[keep][None, :, None]
    else:
        inp["delta"][:] = SMALL if kind == "small" else LARGE
    check_inputs(ss, inp, "bf16", states=True, dsel=DSEL, label=f"bf16 {kind}")


@pytest.mark.parametrize("zoh", [False, True], ids=["euler", "zoh"])
@pytest.mark.parametrize("kind", ["small", "large", "switching"])
def test_limits_decode_step(ss, kind, zoh):
    """ss_step over 12 tokens from N(0,1) states: the state is kept (small), rewritten
    each token (large), or both in turn (switching every 3 tokens)."""
    S, Dn, steps = 64, 256, 12
    spec = W.ScanSpec("limstep", S, steps, Dn, 16, io_dtype="f32", delta_mode="bias", seed=341)
    inp = W.gen_scan_inputs(spec)
    if kind == "small":
        inp["delta"][:] = SMALL
    elif kind == "large":
        inp["delta"][:] = LARGE
    else:
        inp["delta"][:, 0::6] = SMALL
        inp["delta"][:, 1::6] = SMALL
        inp["delta"][:, 2::6] = SMALL
        inp["delta"][:, 3::6] = LARGE
    st = W.gen_states(S, Dn, 16, seed=342)
    g = to_dev(inp, "f32")
    h = torch.from_numpy(st["ssm_state"]).cuda()
    c = torch.from_numpy(st["conv_state"]).cuda()
    hr, cr = st["ssm_state"].astype(np.float64), st["conv_state"].astype(np.float64)
    for t in range(steps):
        y = ss.ss_step(g["x"][:, t].contiguous(), g["delta"][:, t].contiguous(), g["A"], g["B"][:, t].contiguous(),
                       g["C"][:, t].contiguous(), h, conv_state=c, conv_w=g["conv_w"], conv_b=g["conv_b"],
                       delta_bias=g["delta_bias"], D=g["D"], z=g["z"][:, t].contiguous(), zoh=zoh)
        yr, hr, cr = oracle.step(inp["x"][:, t], inp["delta"][:, t], inp["A"], inp["B"][:, t], inp["C"][:, t], hr,
                                 conv_w=inp["conv_w"], conv_b=inp["conv_b"], delta_bias=inp["delta_bias"],
                                 D=inp["D"], z=inp["z"][:, t], conv_state=cr, zoh=zoh)
        e = maxrel(host(y), yr)
        assert e <= TOL["f32"], (kind, t, e)
    torch.cuda.synchronize()
    assert maxrel(host(h), hr) <= TOL["f32"]
    if kind == "small":
        assert maxrel(host(h), st["ssm_state"]) <= 1e-6
    assert np.array_equal(host(c).astype(np.float64), cr)


@pytest.mark.parametrize("zoh", [False, True], ids=["euler", "zoh"])
@pytest.mark.parametrize("kind", ["small", "large", "switching"])
def test_limits_bidirectional(ss, kind, zoh):
    """The reversed pass (its own chunk aggregates in reversed token order) at the limits."""
    shape = ONE_LANE
    p = _plan(ss, shape, pass_=ss.SS_PASS_BIDIR)
    assert p["nchunks"] > 1 and not p["lane_quad"], p
    inp = _inputs(shape, 351)
    if kind == "switching":
        mix = _mixed_delta(shape[1])
        keep = ~np.isnan(mix)
        inp["delta"][:, keep, :] = mix[keep][None, :, None]
    else:
        inp["delta"][:] = SMALL if kind == "small" else LARGE
    check_bidir(ss, inp, "f32", dsel=DSEL, zoh=zoh, label=f"bidir {kind}")
