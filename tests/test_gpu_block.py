"""GPU parity of the Mamba block (ss_block_fwd / ss_block_step: RMSNorm, MFMA
projections, conv + SiLU, the scan, gate and residual) against the fp64 block oracle
on the same seeded weights and inputs. The block shape is the Mamba(d_model=512,
d_state=16, d_conv=4, expand=2) example of the bembew.net page ("Code Example").
Tolerances as for the scan: max relative error (rms floor) 1e-4 with fp32 I/O and 2e-2
with bf16 I/O, on the output and on the carried states. With bf16 I/O the library keeps
every activation between the block's steps in fp32 and feeds it to the bf16 matrix
cores as two bf16 terms, so only the bf16 input, output and weights (the same values on
both sides) differ from the fp64 oracle's arithmetic; the carried states then agree to
about 1e-4."""
import numpy as np
import pytest
import torch

import oracle.block as ob
import workloads as W
from gpu_util import TOL, host, maxrel

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def ss():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import selective_state_space_73_amd as mod
    return mod


def dev_weights(w, io):
    tdt = torch.bfloat16 if io == "bf16" else torch.float32
    out = {}
    for k, v in w.items():
        t = torch.from_numpy(np.ascontiguousarray(v, np.float32)).cuda()
        out[k] = t.to(tdt) if k in ("W_in", "W_x", "W_dt", "W_out") else t
    return out


def run_case(ss, spec, *, states, L=None, Bsz=None, inplace=False, label=""):
    w = W.gen_block_weights(spec)
    x = W.gen_block_input(spec, batch=Bsz, seqlen=L)
    Bn, Ln, _ = x.shape
    st = W.gen_states(Bn, spec.d_inner, spec.d_state, seed=spec.seed + 3) if states else None
    g = dev_weights(w, spec.io_dtype)
    tdt = torch.bfloat16 if spec.io_dtype == "bf16" else torch.float32
    xd = torch.from_numpy(x).cuda().to(tdt)
    hs = torch.from_numpy(st["ssm_state"]).cuda() if states else None
    cs = torch.from_numpy(st["conv_state"]).cuda() if states else None
    out = ss.ss_block_fwd(xd, g, spec.rank, ssm_state=hs, conv_state=cs, out=xd if inplace else None)
    torch.cuda.synchronize()
    ro, rh, rc = ob.block_forward(x, w, spec.rank, st["ssm_state"] if states else None,
                                  st["conv_state"] if states else None)
    e = maxrel(host(out), ro)
    tol = TOL[spec.io_dtype]
    if states:
        eh, ec = maxrel(host(hs), rh), maxrel(host(cs), rc)
        print(f"{label} out maxrel {e:.3e} ssm_state {eh:.3e} conv_state {ec:.3e}", flush=True)
        assert eh <= tol and ec <= tol, (label, eh, ec)
    else:
        print(f"{label} out maxrel {e:.3e}", flush=True)
    assert e <= tol, (label, e)
    return e


@pytest.mark.parametrize("states", [False, True])
def test_block_fwd_f32(ss, states):
    run_case(ss, W.BLOCKS["block_f32"], states=states, label="block f32")


@pytest.mark.parametrize("states", [False, True])
def test_block_fwd_bf16(ss, states):
    run_case(ss, W.BLOCKS["block_bf16"], states=states, label="block bf16")


def test_block_fwd_in_place(ss):
    run_case(ss, W.BLOCKS["block_f32"], states=True, L=200, inplace=True, label="block in place")


@pytest.mark.parametrize("io", ["f32", "bf16"])
def test_block_fwd_ragged(ss, io):
    """Small and ragged: d_model 48, d_inner 96, N 8, rank 3, L 67 (chunk and tile edges)."""
    spec = W.BlockSpec("ragged", 3, 67, 48, expand=2, d_state=8, dt_rank=3, io_dtype=io, seed=777)
    run_case(ss, spec, states=True, label=f"block ragged {io}")


@pytest.mark.parametrize("io", ["f32", "bf16"])
def test_block_fwd_wide_tiles(ss, io):
    """Enough rows (batch 3 x 1500 tokens = 4500, not a multiple of 128) that the input
    projection takes the 128-wide GEMM tiles with a ragged last row of tiles, while the
    narrower projections keep the 64-wide ones; carried states checked for both I/O
    dtypes. (When the block rounded its activations to bf16 between steps, the bf16
    state here was 2.15e-2 from the fp64 block, mostly from the normalised input and
    the conv output; with fp32 activations and split bf16 operands it is about 1e-4.)"""
    spec = W.BLOCKS["block_f32" if io == "f32" else "block_bf16"]
    run_case(ss, spec, states=True, Bsz=3, L=1500, label=f"block wide tiles {io}")


@pytest.mark.parametrize("io", ["f32", "bf16"])
def test_block_fwd_long_sequence_states(ss, io):
    """B2 L8192 at d_model 512: the carried states after a long sequence (the scan's
    chunked path inside the block) for both I/O dtypes."""
    spec = W.BLOCKS["block_f32" if io == "f32" else "block_bf16"]
    run_case(ss, spec, states=True, Bsz=2, L=8192, label=f"block L8192 {io}")


@pytest.mark.parametrize("io", ["f32", "bf16"])
def test_block_fwd_split_k_elementwise_loads(ss, io):
    """d_model 1001: K of in_proj (1001) and of x_proj (2002) is no multiple of the
    16-byte load chunk, so the projections load element by element, and with 200
    rows their grids are short enough that they split K (in_proj 4 ways, x_proj and
    out_proj 16 ways), summed by the reduce kernel, which also adds the residual."""
    spec = W.BlockSpec("splitk", 1, 200, 1001, io_dtype=io, seed=779)
    run_case(ss, spec, states=True, label=f"block split-K element loads {io}")


def test_block_fwd_chunked_long(ss):
    """A long sequence with few channels takes the scan's chunked path inside the block."""
    spec = W.BlockSpec("longblock", 1, 8192, 64, expand=2, d_state=16, io_dtype="f32", seed=778)
    run_case(ss, spec, states=True, label="block chunked")


@pytest.mark.parametrize("io", ["f32", "bf16"])
def test_block_steps(ss, io):
    """Decode: ss_block_step from carried states against the oracle's step, and the
    steps against the forward over the same tokens."""
    spec = W.BLOCKS["block_f32" if io == "f32" else "block_bf16"]
    w = W.gen_block_weights(spec)
    S, steps = 8, 6
    x = W.gen_block_input(spec, batch=S, seqlen=steps)
    st = W.gen_states(S, spec.d_inner, spec.d_state, seed=spec.seed + 5)
    g = dev_weights(w, io)
    tdt = torch.bfloat16 if io == "bf16" else torch.float32
    xd = torch.from_numpy(x).cuda().to(tdt)
    hs = torch.from_numpy(st["ssm_state"]).cuda()
    cs = torch.from_numpy(st["conv_state"]).cuda()
    hr, cr = st["ssm_state"].astype(np.float64), st["conv_state"].astype(np.float64)
    outs = []
    for t in range(steps):
        o = ss.ss_block_step(xd[:, t].contiguous(), g, spec.rank, hs, cs)
        ro, hr, cr = ob.block_step(x[:, t], w, spec.rank, hr, cr)
        e = maxrel(host(o), ro)
        assert e <= TOL[io], (t, e)
        outs.append(o)
    torch.cuda.synchronize()
    assert maxrel(host(hs), hr) <= TOL[io] and maxrel(host(cs), cr) <= TOL[io]
    # the same tokens through the forward from the same initial states
    hs2 = torch.from_numpy(st["ssm_state"]).cuda()
    cs2 = torch.from_numpy(st["conv_state"]).cuda()
    fw = ss.ss_block_fwd(xd, g, spec.rank, ssm_state=hs2, conv_state=cs2)
    torch.cuda.synchronize()
    assert maxrel(host(torch.stack(outs, 1)), host(fw)) <= TOL[io]


def test_block_train_width_sampled_rows(ss):
    """The training-width block (B8 L2048, d_model 2560, d_inner 5120, rank 160, bf16)
    on the GPU with carried states; the fp64 oracle on batch rows 0 and 7 (the block is
    independent across batch rows): output and both final states at the bf16 bar."""
    spec = W.BLOCKS["block_train"]
    w = W.gen_block_weights(spec)
    x = W.gen_block_input(spec)
    Bn = x.shape[0]
    st = W.gen_states(Bn, spec.d_inner, spec.d_state, seed=spec.seed + 3)
    g = dev_weights(w, "bf16")
    xd = torch.from_numpy(x).cuda().to(torch.bfloat16)
    hs = torch.from_numpy(st["ssm_state"]).cuda()
    cs = torch.from_numpy(st["conv_state"]).cuda()
    print("block_train: launching B8 L2048 d_model 2560", flush=True)
    out = ss.ss_block_fwd(xd, g, spec.rank, ssm_state=hs, conv_state=cs)
    torch.cuda.synchronize()
    for b in (0, Bn - 1):
        sl = slice(b, b + 1)
        ro, rh, rc = ob.block_forward(x[sl], w, spec.rank, st["ssm_state"][sl], st["conv_state"][sl])
        e, eh, ec = maxrel(host(out[sl]), ro), maxrel(host(hs[sl]), rh), maxrel(host(cs[sl]), rc)
        print(f"block_train row {b}: out {e:.3e} ssm_state {eh:.3e} conv_state {ec:.3e}", flush=True)
        assert e <= TOL["bf16"] and eh <= TOL["bf16"] and ec <= TOL["bf16"], (b, e, eh, ec)


@pytest.mark.parametrize("dm", [512, 2560])
def test_block_decode_64_streams(ss, dm):
    """64-stream block decode (bf16) at d_model 512 and 2560: three tokens from N(0,1)
    states against the oracle's steps."""
    spec = W.BLOCKS["block_bf16"] if dm == 512 else W.BLOCKS["block_train"]
    w = W.gen_block_weights(spec)
    S, steps = 64, 3
    x = W.gen_block_input(spec, batch=S, seqlen=steps)
    st = W.gen_states(S, spec.d_inner, spec.d_state, seed=spec.seed + 9)
    g = dev_weights(w, "bf16")
    xd = torch.from_numpy(x).cuda().to(torch.bfloat16)
    hs = torch.from_numpy(st["ssm_state"]).cuda()
    cs = torch.from_numpy(st["conv_state"]).cuda()
    hr, cr = st["ssm_state"].astype(np.float64), st["conv_state"].astype(np.float64)
    print(f"block decode: 64 streams, d_model {dm}", flush=True)
    for t in range(steps):
        o = ss.ss_block_step(xd[:, t].contiguous(), g, spec.rank, hs, cs)
        ro, hr, cr = ob.block_step(x[:, t], w, spec.rank, hr, cr)
        e = maxrel(host(o), ro)
        assert e <= TOL["bf16"], (t, e)
    torch.cuda.synchronize()
    eh, ec = maxrel(host(hs), hr), maxrel(host(cs), cr)
    print(f"block decode d_model {dm}: state {eh:.3e} conv {ec:.3e}", flush=True)
    assert eh <= TOL["bf16"] and ec <= TOL["bf16"]
