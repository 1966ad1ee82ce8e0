"""GPU parity of the power fast path of the one-lane scan kernels: when every channel of
a workgroup has A[d, n] = (n + 1) A[d, 0] (the A = -(1..N) initialisation of
ozercemkelahmet.com "Mamba", "A minimal selective scan in PyTorch"), the decays are
exp(Delta A[d, 0])^(n+1), one exponential and a chain of multiplies; otherwise the
general decays exp(Delta A[d, n]) run. Both against the fp64 oracle, for d_state 8,
16 and 64 (4 never takes the fast path), fp32 and bf16 I/O, unchunked and chunked
shapes, workgroups of either kind side by side, and the forward recompute of the
backward and the reversed pass of the bidirectional scan. Under the zero-order hold the
power path also forms every write coefficient (exp(Delta A_n) - 1) / A_n from the first
one and the geometric sum 1 + a_0 + ... + a_0^n. The path is taken only where A[d, 0] is
0 or at most -1/2; channels with A[d, 0] = -1e-3, 0 and +1e-4 check that gate. The error of the final
state is reported per state index n, where the chain's rounding would grow with n."""
import numpy as np
import pytest
import torch

import workloads as W
from gpu_util import TOL, check_inputs, gpu_fwd, host, maxrel, oracle_fwd, to_dev
from test_gpu_bidir import check_bidir
from test_gpu_bwd import check_bwd

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def ss():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import selective_state_space_73_amd as mod
    return mod


def _break_identity(A, rows):
    """Make A[d, n] = (n + 1) A[d, 0] fail on the given channels (one ulp-scale change of
    every n >= 1, so the result moves by rounding only)."""
    A = A.copy()
    A[rows, 1:] *= np.float32(1.0 + 2.0 ** -20)
    return A


def _per_state_errors(ss, inp, io, label, dsel=None, zoh=False):
    """One forward with initial states; y and the final state against the oracle, the
    state's error per state index n."""
    Bsz, L, Dn = inp["x"].shape
    N = inp["A"].shape[1]
    st = W.gen_states(Bsz, Dn, N, seed=4242)
    g = to_dev(inp, io)
    hs = torch.from_numpy(st["ssm_state"]).cuda()
    cs = torch.from_numpy(st["conv_state"]).cuda()
    y = gpu_fwd(ss, g, hs, cs, zoh=zoh)
    torch.cuda.synchronize()
    yr, hr, cr = oracle_fwd(inp, st["ssm_state"], st["conv_state"], dsel=dsel, zoh=zoh)
    yg = host(y) if dsel is None else host(y)[:, :, dsel]
    hg = host(hs) if dsel is None else host(hs)[:, dsel]
    ey = maxrel(yg, yr)
    per_n = [maxrel(hg[..., n], hr[..., n]) for n in range(N)]
    print(f"{label}: y {ey:.2e} state per n " + " ".join(f"{e:.1e}" for e in per_n), flush=True)
    assert ey <= TOL[io], (label, ey)
    assert max(per_n) <= TOL["f32"], (label, per_n)
    return per_n


SHAPES = {  # (batch, seqlen, d_inner): one chunk (enough channels), and the chunked one-lane path
    "unchunked": (32, 200, 4096),
    "chunked": (1, 16384, 1024),
}


@pytest.mark.parametrize("io", ["f32", "bf16"])
@pytest.mark.parametrize("N", [8, 16, 64])
@pytest.mark.parametrize("shape", list(SHAPES), ids=str)
@pytest.mark.parametrize("kind", ["power", "general", "mixed"])
def test_power_and_general_decays(ss, kind, shape, N, io):
    Bsz, L, Dn = SHAPES[shape]
    dims = ss.make_dims(Bsz, L, Dn, N, 0 if io == "f32" else 1)
    plan = ss.ss_scan_plan(dims)
    assert not plan["lane_quad"] and (plan["nchunks"] > 1) == (shape == "chunked"), plan
    spec = W.ScanSpec("pow", Bsz, L, Dn, N, io_dtype=io, delta_mode="direct", seed=500 + N)
    inp = W.gen_scan_inputs(spec)
    assert np.array_equal(inp["A"], -np.arange(1, N + 1, dtype=np.float32)[None, :].repeat(Dn, 0))
    if kind == "general":
        inp["A"] = _break_identity(inp["A"], slice(None))
    elif kind == "mixed":
        # workgroups of 256 channels: 256..511 general throughout, one channel of 768..1023
        # breaks the whole workgroup's vote, the rest take the power chain
        inp["A"] = _break_identity(inp["A"], np.r_[256:512, 800])
    dsel = np.array([0, 1, 255, 256, 300, 511, 512, 767, 768, 800, 1000, Dn - 1])
    _per_state_errors(ss, inp, io, f"{kind} {shape} N{N} {io}", dsel=dsel)


def test_power_path_long_workload_per_state(ss):
    """The long workload (B1 L131072 D2048 N16 bf16, 64 chunks) on the power path:
    per-state error of the final state on sampled channels, fp32 state bar."""
    spec = W.WORKLOADS["long"]
    inp = W.gen_scan_inputs(spec)
    dsel = np.array([0, 1, 63, 64, 255, 256, 1000, 1023, 1024, 2047])
    per_n = _per_state_errors(ss, inp, "bf16", "long power", dsel=dsel)
    inp["A"] = _break_identity(inp["A"], slice(None))
    per_g = _per_state_errors(ss, inp, "bf16", "long general", dsel=dsel)
    # the chain may not make the high states' error grow beyond the general path's scale
    assert max(per_n) <= 10 * max(max(per_g), 1e-6), (per_n, per_g)


@pytest.mark.parametrize("zoh", [False, True], ids=["euler", "zoh"])
@pytest.mark.parametrize("kind", ["power", "general", "special"])
def test_backward_both_paths(ss, kind, zoh):
    """The backward on either path: the checkpoint pass, the sweep (whose power launch takes
    its recompute's decays, and under the zero-order hold its coefficients, from the chain
    and the geometric sum) and the adjoint aggregates. "special": the channels of
    _special_power_A (A[d, 0] = 0 keeps the power path; -1e-3 and +1e-4 take the general one)."""
    spec = W.ScanSpec("powbwd", 2, 8192, 1024, 16, io_dtype="f32", delta_mode="direct", seed=611)
    inp = W.gen_scan_inputs(spec)
    if kind == "general":
        inp["A"] = _break_identity(inp["A"], slice(None))
    elif kind == "special":
        inp["A"], _ = _special_power_A(1024, 16)
    check_bwd(ss, inp, "f32", label=f"bwd {kind} {'zoh' if zoh else 'euler'}", zoh=zoh)


@pytest.mark.parametrize("kind", ["power", "general", "mixed"])
def test_bidirectional_both_paths(ss, kind):
    spec = W.ScanSpec("powbi", 1, 16384, 1024, 16, io_dtype="f32", delta_mode="direct", seed=612)
    inp = W.gen_scan_inputs(spec)
    if kind == "general":
        inp["A"] = _break_identity(inp["A"], slice(None))
    elif kind == "mixed":
        inp["A"] = _break_identity(inp["A"], np.r_[0:256])
    check_bidir(ss, inp, "f32", dsel=np.array([0, 255, 256, 700, 1023]), label=f"bidir {kind}")


def test_power_and_general_agree_closely(ss):
    """The two paths differ by rounding only: on identical inputs up to the one-ulp change
    of A, their outputs agree to well within the fp32 bar."""
    spec = W.ScanSpec("powcmp", 2, 4096, 1024, 16, io_dtype="f32", delta_mode="direct", seed=613)
    inp = W.gen_scan_inputs(spec)
    g = to_dev(inp, "f32")
    y_pow = gpu_fwd(ss, g)
    g2 = dict(g)
    g2["A"] = torch.from_numpy(_break_identity(inp["A"], slice(None))).cuda()
    y_gen = gpu_fwd(ss, g2)
    torch.cuda.synchronize()
    e = maxrel(host(y_pow), host(y_gen))
    print(f"power vs general y maxrel {e:.2e}", flush=True)
    assert e <= TOL["f32"]


def _special_power_A(Dn, N):
    """A[d, n] = (n + 1) A[d, 0] exactly in fp32 on every channel, with A[d, 0] = -1 except
    on some channels of the first three workgroups (256 channels each): 0 on channels
    0, 37, .. of the first (no decay, an exact chain: that workgroup keeps the power path;
    for the zero-order hold the coefficient is Delta), -1e-3 on channels of the second (a
    memory far longer than the sequence, where the chain's rounding would grow with n: the
    workgroup must take the general decays) and +1e-4 on channels of the third (a growing
    state, general decays)."""
    a0 = np.full(Dn, -1.0, dtype=np.float32)
    a0[np.arange(0, 256, 37)] = np.float32(0.0)
    a0[256 + np.arange(3, 256, 17)] = np.float32(-1e-3)
    a0[512 + np.arange(5, 256, 41)] = np.float32(1e-4)
    k = np.arange(1, N + 1, dtype=np.float32)
    A = (k[None, :] * a0[:, None]).astype(np.float32)
    assert np.array_equal(A[:, 1:], np.float32(k[1:])[None, :] * A[:, :1])
    return A, np.flatnonzero(a0 != -1.0)


@pytest.mark.parametrize("zoh", [False, True], ids=["euler", "zoh"])
@pytest.mark.parametrize("N", [8, 16, 64])
@pytest.mark.parametrize("shape", list(SHAPES), ids=str)
@pytest.mark.parametrize("kind", ["power", "general", "mixed"])
def test_power_path_special_channels(ss, kind, shape, N, zoh):
    """fp32 I/O, both write terms: workgroups with channels of A[d, 0] = 0, -1e-3 and +1e-4
    beside the usual -1 (see _special_power_A); "mixed" also breaks the identity on a fourth
    workgroup. The zero-order hold's power path forms every write coefficient from the
    first one and the geometric sum 1 + a_0 + ... + a_0^n (main pass and, chunked,
    aggregate pass). Without the gate on A[d, 0], the -1e-3 channels at d_state 64 on the
    short shape were 3.5e-4 from the oracle on the power path."""
    Bsz, L, Dn = SHAPES[shape]
    spec = W.ScanSpec("spow", Bsz, L, Dn, N, io_dtype="f32", delta_mode="direct", seed=700 + N)
    inp = W.gen_scan_inputs(spec)
    inp["A"], special = _special_power_A(Dn, N)
    if kind == "general":
        inp["A"] = _break_identity(inp["A"], slice(None))
    elif kind == "mixed":
        inp["A"] = _break_identity(inp["A"], np.r_[768:1024])
    dsel = np.unique(np.r_[[0, 255, 256, 511, 512, Dn - 1], special])
    _per_state_errors(ss, inp, "f32", f"{'zoh' if zoh else 'euler'} {kind} {shape} N{N}", dsel=dsel, zoh=zoh)


def test_zoh_power_path_long_workload(ss):
    """The long workload (B1 L131072 D2048 N16 bf16, 64 chunks) with the zero-order hold on
    the power path and on the general path, sampled channels."""
    spec = W.WORKLOADS["long"]
    inp = W.gen_scan_inputs(spec)
    dsel = np.array([0, 1, 63, 64, 255, 256, 1000, 1023, 1024, 2047])
    per_n = _per_state_errors(ss, inp, "bf16", "zoh long power", dsel=dsel, zoh=True)
    inp["A"] = _break_identity(inp["A"], slice(None))
    per_g = _per_state_errors(ss, inp, "bf16", "zoh long general", dsel=dsel, zoh=True)
    assert max(per_n) <= 10 * max(max(per_g), 1e-6), (per_n, per_g)
