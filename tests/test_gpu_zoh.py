"""GPU parity of the zero-order-hold write term (dims.discretization = SS_ZOH):
W = (exp(Delta A) - 1) / A instead of Delta (inferensys.com "Mamba", the
discretization bullet; ai360xpert.com "Mamba", code section). The HIP library
through its C ABI against the fp64 oracle run with zoh=True, on the same seeded
inputs and tolerances as the Euler tests: the bench workloads, ragged and edge
shapes, the chunked path (aggregate pass in its telescoped ZOH form), A = 0
states (the limit Delta), small |A| (the coefficient's series branch) and A > 0,
the aggregate bound's exact fallback, and the decode step."""
import numpy as np
import pytest
import torch

import oracle
import workloads as W
from gpu_util import TOL, check_fwd, check_inputs, gpu_fwd, host, maxrel, oracle_fwd, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def ss():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import selective_state_space_73_amd as mod
    return mod


# ----------------------------------------------------------------------------- workloads

@pytest.mark.parametrize("states", [False, True])
@pytest.mark.parametrize("name", ["tiny", "block"])
def test_zoh_small_workloads(ss, name, states):
    check_fwd(ss, W.WORKLOADS[name], states=states, zoh=True, label=f"zoh {name}")


def test_zoh_is_not_euler(ss):
    """The two rules differ by far more than the tolerance on these inputs, so the
    parity tests tell them apart; and each GPU result matches its own oracle."""
    spec = W.WORKLOADS["block"]
    inp = W.gen_scan_inputs(spec)
    g = to_dev(inp, spec.io_dtype)
    y_e = host(gpu_fwd(ss, g))
    y_z = host(gpu_fwd(ss, g, zoh=True))
    dsel = np.arange(0, 1024, 97)
    r_e, _, _ = oracle_fwd(inp, dsel=dsel)
    r_z, _, _ = oracle_fwd(inp, dsel=dsel, zoh=True)
    assert maxrel(r_z, r_e) > 100 * TOL["f32"]
    assert maxrel(y_z[:, :, dsel], r_z) <= TOL["f32"] and maxrel(y_e[:, :, dsel], r_e) <= TOL["f32"]


def test_zoh_train_full_size_sampled_channels(ss):
    dsel = np.unique(np.concatenate([np.arange(0, 5120, 127), [0, 1, 63, 64, 255, 256, 5119]]))
    check_fwd(ss, W.WORKLOADS["train"], states=True, dsel=dsel, zoh=True, label="zoh train")


def test_zoh_long_full_size_sampled_channels(ss):
    dsel = np.array([0, 1, 63, 64, 255, 256, 1023, 1024, 2047])
    check_fwd(ss, W.WORKLOADS["long"], states=True, dsel=dsel, zoh=True, label="zoh long")


# ----------------------------------------------------------------------------- shapes and pieces

EDGE_SHAPES = [
    dict(batch=1, seqlen=1, d_inner=8, d_state=4),
    dict(batch=2, seqlen=2, d_inner=5, d_state=4),
    dict(batch=3, seqlen=67, d_inner=70, d_state=8),
    dict(batch=1, seqlen=131, d_inner=257, d_state=16),
    dict(batch=2, seqlen=200, d_inner=64, d_state=32),
    dict(batch=1, seqlen=150, d_inner=33, d_state=64),
]


@pytest.mark.parametrize("io", ["f32", "bf16"])
@pytest.mark.parametrize("shape", EDGE_SHAPES, ids=lambda s: "B{batch}L{seqlen}D{d_inner}N{d_state}".format(**s))
def test_zoh_edge_shapes(ss, io, shape):
    spec = W.ScanSpec("zedge", 1, 1, 1, 4, io_dtype=io, delta_mode="bias", seed=4343)
    check_fwd(ss, spec, shape=shape, states=True, zoh=True, label=f"zoh edge {shape} {io}")


@pytest.mark.parametrize("flags", [dict(conv=False), dict(gate=False),
                                   dict(conv=False, gate=False, skip=False, bias=False)],
                         ids=lambda f: "-".join(f"no_{k}" for k in f))
def test_zoh_optional_pieces(ss, flags):
    spec = W.ScanSpec("zflags", 2, 90, 72, 16, io_dtype="f32", delta_mode="bias", seed=98)
    check_fwd(ss, spec, states=True, flags=flags, zoh=True, label=f"zoh flags {flags}")


@pytest.mark.parametrize("io", ["f32", "bf16"])
@pytest.mark.parametrize("shape", [dict(batch=1, seqlen=4096, d_inner=64, d_state=16),
                                   dict(batch=2, seqlen=3001, d_inner=100, d_state=8)],
                         ids=["chunked_even", "chunked_ragged"])
def test_zoh_chunked_path(ss, io, shape):
    dims = ss.make_dims(shape["batch"], shape["seqlen"], shape["d_inner"], shape["d_state"], 0,
                        discretization=ss.SS_ZOH)
    assert ss.ss_workspace_bytes(dims) > 0, "shape does not select the chunked path"
    spec = W.ScanSpec("zchunk", 1, 1, 1, 4, io_dtype=io, delta_mode="bias", seed=8)
    check_fwd(ss, spec, shape=shape, states=True, zoh=True, label=f"zoh chunked {shape} {io}")


@pytest.mark.parametrize("seqlen", [100, 4096], ids=["one_chunk", "chunked"])
def test_zoh_zero_and_growing_A(ss, seqlen):
    """A = 0 in some states (the write coefficient's limit Delta), A > 0 (a growing
    state) in some channels and small negative A in others: there Delta*A is tiny
    and the coefficient must come from its series, not from exp(Delta A) - 1."""
    spec = W.ScanSpec("zzero", 1, 1, 1, 16, io_dtype="f32", delta_mode="bias", seed=126)
    inp = W.gen_scan_inputs(spec, batch=1, seqlen=seqlen, d_inner=200)
    inp["A"][0:60:3, 5] = np.float32(0.0)
    inp["A"][1, :] = np.float32(0.0)
    inp["A"][130, 2:6] = np.float32(0.0)
    inp["A"][7::11] = np.float32(0.002)
    inp["A"][3::13] = np.float32(-1e-3)
    inp["A"][5::17, ::2] = np.float32(-3e-5)
    check_inputs(ss, inp, "f32", states=True, zoh=True, label=f"zoh zero/growing A L={seqlen}")


def test_zoh_long_chunks_fp32_truncated_aggregates(ss):
    spec = W.ScanSpec("zlc", 1, 65536, 1024, 16, io_dtype="f32", delta_mode="direct", seed=127)
    inp = W.gen_scan_inputs(spec)
    check_inputs(ss, inp, "f32", states=True, dsel=np.array([0, 5, 511, 700, 1023]), zoh=True,
                 label="zoh long chunks fp32")


def test_zoh_aggregate_bound_fallback(ss):
    """Constant step 0.1 drops every state 278 tokens before a chunk's end, inputs 1e10
    times larger sit just before that point (287-326 tokens before the chunk end; their
    carry is 8e-3 of the chunk's end state, which the truncated sweep would miss), so
    the aggregate pass's exact recurrence must take over; the gate is shut (z = -30)
    over the rows the large inputs would otherwise dominate. The rows are placed from
    the chunk length the library reports (512 tokens on this shape, which takes the
    aggregate pass rather than the carry correction)."""
    from test_gpu_parity import one_lane_chunk_len
    spec = W.ScanSpec("zfb", 1, 65536, 1024, 16, io_dtype="f32", delta_mode="direct", seed=128)
    inp = W.gen_scan_inputs(spec)
    inp["delta"][:] = np.float32(np.log(np.expm1(0.1)))
    cl = one_lane_chunk_len(ss, inp, "f32", zoh=True, carry=False)
    assert cl >= 512, cl
    r = np.arange(65536) % cl
    inp["x"][:, (r >= cl - 327) & (r < cl - 287), :] *= np.float32(1e10)
    inp["z"][:, (r >= cl - 327) & (r < cl - 22), :] = np.float32(-30.0)
    check_inputs(ss, inp, "f32", states=True, dsel=np.array([0, 3, 512, 1023]), zoh=True,
                 label="zoh bound fallback")


# ----------------------------------------------------------------------------- decode step

def _step_oracle(inp, t, hr, cr, zoh=True):
    return oracle.step(inp["x"][:, t], inp["delta"][:, t], inp["A"], inp["B"][:, t], inp["C"][:, t], hr,
                       conv_w=inp["conv_w"], conv_b=inp["conv_b"], delta_bias=inp["delta_bias"], D=inp["D"],
                       z=inp["z"][:, t], conv_state=cr, zoh=zoh)


def _step_gpu(ss, g, t, h, c):
    return ss.ss_step(g["x"][:, t].contiguous(), g["delta"][:, t].contiguous(), g["A"], g["B"][:, t].contiguous(),
                      g["C"][:, t].contiguous(), h, conv_state=c, conv_w=g["conv_w"], conv_b=g["conv_b"],
                      delta_bias=g["delta_bias"], D=g["D"], z=g["z"][:, t].contiguous(), zoh=True)


@pytest.mark.parametrize("io", ["f32", "bf16"])
@pytest.mark.parametrize("S,Dn,N", [(1, 8, 4), (3, 70, 8), (5, 64, 16), (6, 33, 32), (7, 130, 64), (64, 257, 16)],
                         ids=lambda v: str(v))
def test_zoh_step_edge_shapes(ss, io, S, Dn, N):
    """ss_step with zoh against the oracle, with one A = 0 state per fifth channel."""
    spec = W.ScanSpec("zstep", 1, 1, 1, 4, io_dtype=io, delta_mode="bias", seed=81)
    inp = W.gen_scan_inputs(spec, batch=S, seqlen=5, d_inner=Dn, d_state=N)
    inp["A"][::5, N - 1] = np.float32(0.0)
    st = W.gen_states(S, Dn, N, seed=82)
    g = to_dev(inp, io)
    h = torch.from_numpy(st["ssm_state"]).cuda()
    c = torch.from_numpy(st["conv_state"]).cuda()
    hr, cr = st["ssm_state"].astype(np.float64), st["conv_state"].astype(np.float64)
    for t in range(5):
        y = _step_gpu(ss, g, t, h, c)
        yr, hr, cr = _step_oracle(inp, t, hr, cr)
        e = maxrel(host(y), yr)
        assert e <= TOL[io], (t, e)
    torch.cuda.synchronize()
    assert maxrel(host(h), hr) <= TOL["f32"]
    assert np.array_equal(host(c).astype(np.float64), cr)


@pytest.mark.parametrize("io", ["f32", "bf16"])
def test_zoh_steps_match_scan(ss, io):
    spec = W.ScanSpec("zsteps", 3, 1, 1, 16, io_dtype=io, delta_mode="bias", seed=12)
    inp = W.gen_scan_inputs(spec, batch=3, seqlen=24, d_inner=130)
    st = W.gen_states(3, 130, 16)
    g = to_dev(inp, io)
    h_s, c_s = torch.from_numpy(st["ssm_state"]).cuda(), torch.from_numpy(st["conv_state"]).cuda()
    y_scan = gpu_fwd(ss, g, h_s, c_s, zoh=True)
    h, c = torch.from_numpy(st["ssm_state"]).cuda(), torch.from_numpy(st["conv_state"]).cuda()
    y_step = torch.stack([_step_gpu(ss, g, t, h, c) for t in range(24)], dim=1)
    e_y, e_h = maxrel(host(y_step), host(y_scan)), maxrel(host(h), host(h_s))
    assert e_y <= TOL[io] and e_h <= TOL["f32"], (e_y, e_h)
    assert torch.equal(c, c_s)


def test_zoh_decode_full_shape_sampled(ss):
    """Decode shapes (64 streams x 8192 channels, N=16, bf16 token inputs) for 10
    steps of one layer; the oracle follows 6 streams x 40 channels."""
    spec = W.DECODE
    S, Dn, N = spec.streams, spec.d_inner, spec.d_state
    s_sel = np.array([0, 1, 17, 31, 62, 63])
    d_sel = np.unique(np.concatenate([np.arange(0, Dn, 211), [0, 1, 255, 256, 8191]]))
    par = W.gen_decode_layer_params(spec, 3)
    st = W.gen_states(S, Dn, N, seed=1003)
    gp = {k: torch.from_numpy(v).cuda() for k, v in par.items()}
    hs = torch.from_numpy(st["ssm_state"]).cuda()
    cs = torch.from_numpy(st["conv_state"]).cuda()
    hr = st["ssm_state"][s_sel][:, d_sel].astype(np.float64)
    cr = st["conv_state"][s_sel][:, d_sel].astype(np.float64)
    worst = 0.0
    for step in range(10):
        si = W.gen_decode_step_inputs(spec, 3, step % spec.pool)
        gs = {k: torch.from_numpy(v).cuda().to(torch.bfloat16) for k, v in si.items()}
        y = ss.ss_step(gs["x"], gs["delta"], gp["A"], gs["B"], gs["C"], hs, conv_state=cs, conv_w=gp["conv_w"],
                       conv_b=gp["conv_b"], delta_bias=gp["delta_bias"], D=gp["D"], z=gs["z"], zoh=True)
        yr, hr, cr = oracle.step(si["x"][s_sel][:, d_sel], si["delta"][s_sel][:, d_sel], par["A"][d_sel],
                                 si["B"][s_sel], si["C"][s_sel], hr, conv_w=par["conv_w"][d_sel],
                                 conv_b=par["conv_b"][d_sel], delta_bias=par["delta_bias"][d_sel],
                                 D=par["D"][d_sel], z=si["z"][s_sel][:, d_sel], conv_state=cr, zoh=True)
        worst = max(worst, maxrel(host(y)[s_sel][:, d_sel], yr))
    torch.cuda.synchronize()
    eh = maxrel(host(hs)[s_sel][:, d_sel], hr)
    print(f"zoh decode: y maxrel {worst:.3e} state maxrel {eh:.3e}", flush=True)
    assert worst <= TOL["bf16"] and eh <= TOL["bf16"]
