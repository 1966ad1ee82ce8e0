"""The C-ABI library loads, exports every symbol include/selscan.h declares, and
rejects bad arguments on the host before anything reaches the device. No
compute call is made, so these run without a GPU."""
import ctypes
import os
import re
import subprocess

import pytest

import selective_state_space_73_amd as ss

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "selscan.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"^\s*(?:const\s+)?[A-Za-z_][A-Za-z0-9_]*\s*\*?\s*([A-Za-z_][A-Za-z0-9_]*)\s*\(", text, flags=re.M)
    return sorted(set(n for n in names if n.startswith("ss_")))


def test_header_declares_the_boundary():
    assert declared_functions() == sorted(["ss_workspace_bytes", "ss_conv_scan_fwd", "ss_step", "ss_status_str",
                                           "ss_last_error", "ss_version", "ss_time_next_call",
                                           "ss_bwd_workspace_bytes", "ss_conv_scan_bwd", "ss_conv_scan_bidir_fwd",
                                           "ss_bidir_workspace_bytes", "ss_scan_plan", "ss_conv_scan_fwd_noalloc",
                                           "ss_block_workspace_bytes", "ss_block_fwd", "ss_block_step"])


def test_library_exports_every_declared_symbol():
    out = subprocess.run(["nm", "-D", "--defined-only", ss.LIB_PATH], capture_output=True, text=True, check=True).stdout
    exported = set(line.split()[-1] for line in out.splitlines() if line.strip())
    for name in declared_functions():
        assert name in exported, name
        assert getattr(ss.lib, name) is not None


def test_version_and_status_strings():
    assert ss.ss_version() == 5
    assert ss.lib.ss_status_str(0) == b"ok"
    assert b"workspace" in ss.lib.ss_status_str(3)


def test_struct_layout_matches_header():
    assert ctypes.sizeof(ss.ss_dims) == 40
    assert ctypes.sizeof(ss.ss_args) == 13 * ctypes.sizeof(ctypes.c_void_p)
    assert ctypes.sizeof(ss.ss_grads) == 15 * ctypes.sizeof(ctypes.c_void_p)
    assert ctypes.sizeof(ss.ss_block_dims) == 56
    assert ctypes.sizeof(ss.ss_block_weights) == 10 * ctypes.sizeof(ctypes.c_void_p)
    assert ctypes.sizeof(ss.ss_dir_args) == 8 * ctypes.sizeof(ctypes.c_void_p)
    assert ctypes.sizeof(ss.ss_plan) == 24


def _dims(**kw):
    d = dict(batch=2, seqlen=16, d_inner=64, d_state=16, io_dtype=ss.SS_F32)
    d.update(kw)
    return ss.make_dims(d["batch"], d["seqlen"], d["d_inner"], d["d_state"], d["io_dtype"], d.get("d_conv", 4))


def _fake_args(**kw):
    # fake but well aligned, non-overlapping "device" addresses: validation only looks at them
    base = 1 << 40
    a = {}
    for i, name in enumerate(["x", "conv_w", "conv_b", "delta", "delta_bias", "A", "B", "C", "Dskip", "z", "y",
                              "ssm_state", "conv_state"]):
        a[name] = base + i * (1 << 32)
    a.update(kw)
    return ss.ss_args(**a)


def _call(dims, args, ws=None, ws_bytes=0, step=False):
    if step:
        return ss.lib.ss_step(ctypes.byref(dims), ctypes.byref(args), None)
    return ss.lib.ss_conv_scan_fwd(ctypes.byref(dims), ctypes.byref(args), ws, ws_bytes, None)


@pytest.mark.parametrize("field", ["x", "delta", "A", "B", "C", "y"])
def test_null_required_pointer_rejected(field):
    assert _call(_dims(), _fake_args(**{field: None})) == 1
    assert field in ss.lib.ss_last_error().decode()


@pytest.mark.parametrize("kw,status", [
    (dict(batch=0), 1), (dict(seqlen=0), 1), (dict(d_inner=0), 1), (dict(d_inner=(1 << 26) + 1), 1),
    (dict(seqlen=1 << 31), 1), (dict(d_state=12), 2),
    (dict(d_state=128), 2), (dict(d_conv=3), 2), (dict(io_dtype=7), 2),
])
def test_bad_dims_rejected(kw, status):
    assert _call(_dims(**kw), _fake_args()) == status


@pytest.mark.parametrize("disc", [-1, 2, 7])
def test_unknown_discretization_rejected(disc):
    d = _dims()
    d.discretization = disc
    assert _call(d, _fake_args()) == 1
    assert "discretization" in ss.lib.ss_last_error().decode()


def test_discretization_field_layout():
    """The field sits where the header puts it, after io_dtype, and both rules are
    accepted by the size query (ZOH needs the same workspace as Euler)."""
    assert ss.ss_dims.discretization.offset == 36 and ctypes.sizeof(ss.ss_dims) == 40
    e = ss.make_dims(1, 8192, 64, 16, ss.SS_F32)
    z = ss.make_dims(1, 8192, 64, 16, ss.SS_F32, discretization=ss.SS_ZOH)
    assert ss.ss_workspace_bytes(e) == ss.ss_workspace_bytes(z) > 0


def test_misaligned_pointer_rejected():
    assert _call(_dims(), _fake_args(x=(1 << 40) + 2)) == 1
    assert "aligned" in ss.lib.ss_last_error().decode()
    assert _call(_dims(), _fake_args(ssm_state=(1 << 40) + 11 * (1 << 32) + 4)) == 1


def test_y_aliasing_an_input_rejected():
    a = _fake_args()
    a.y = a.x + 64
    assert _call(_dims(), a) == 1
    assert "overlaps" in ss.lib.ss_last_error().decode()


def test_conv_state_without_conv_rejected():
    assert _call(_dims(), _fake_args(conv_w=None)) == 1


def test_timing_events_are_consumed_by_a_failing_call():
    assert ss.lib.ss_time_next_call(None, None, None, None) == 0
    # a rejected call must not leave the events armed for the next call
    assert ss.lib.ss_time_next_call(1, 2, 3, 4) == 0
    assert _call(_dims(), _fake_args(x=None)) == 1
    assert ss.lib.ss_time_next_call(None, None, None, None) == 0


def test_step_requires_states():
    assert _call(_dims(), _fake_args(ssm_state=None), step=True) == 1
    assert _call(_dims(), _fake_args(conv_state=None), step=True) == 1


def test_workspace_query_and_check():
    # one batch row, few channels, long sequence: chunked, so a workspace is needed
    d = _dims(batch=1, seqlen=1 << 14, d_inner=64)
    need = ss.ss_workspace_bytes(d)
    assert need > 0
    assert _call(d, _fake_args(), None, 0) == 3
    assert _call(d, _fake_args(), 1 << 45, need - 1) == 3
    assert ss.ss_workspace_bytes(_dims(batch=0)) == 0


def _scan_ws(B, L, D, N, nc):
    """Forward workspace for nc chunks: a slot per chunk of end states S [B, nc, D, N]
    and summed steps [B, nc, D], copies of the initial state [B, D, N] and conv history
    [B, D, 3]."""
    a = lambda v: (v + 255) // 256 * 256  # noqa: E731
    if nc == 1:
        return 0
    return a(B * nc * D * N * 4) + a(B * nc * D * 4) + a(B * D * N * 4) + a(B * D * 3 * 4)


def test_forward_chunk_rules():
    """Host chunk rules, seen through the workspace size. One lane per channel takes
    whole 64-token tiles, aiming at 512 workgroups of 256 lanes. With d_state <= 16,
    when that gives fewer than 2048 waves holding a channel and the lane-quad kernels
    at least double them, the quad kernels run, chunked for about 2^18 lanes (four per
    channel) with chunks of at least 16 tokens and at most 128 chunks: batch 2 x 1024
    channels -> 32 chunks of 32 tokens (tiles: 16 chunks, 512 waves); one row of 64
    channels over 4096 tokens -> 128 chunks. One row of 256 channels over 24576 tokens
    keeps the tiles: 384 chunks hold 1536 waves, the quad cap of 128 chunks 2048.
    d_state 32 keeps the tiles: 2 rows x 4 groups -> 64 chunks, capped at 1024 / 64.
    The bidirectional passes keep the tile rule for every d_state."""
    assert ss.ss_workspace_bytes(ss.make_dims(2, 1024, 1024, 16, ss.SS_F32)) == _scan_ws(2, 1024, 1024, 16, 32)
    assert ss.ss_workspace_bytes(ss.make_dims(1, 4096, 64, 16, ss.SS_BF16)) == _scan_ws(1, 4096, 64, 16, 128)
    assert ss.ss_workspace_bytes(ss.make_dims(1, 24576, 256, 16, ss.SS_BF16)) == _scan_ws(1, 24576, 256, 16, 384)
    assert ss.ss_workspace_bytes(ss.make_dims(2, 1024, 1024, 32, ss.SS_F32)) == _scan_ws(2, 1024, 1024, 32, 16)
    a = lambda v: (v + 255) // 256 * 256  # noqa: E731
    assert ss.ss_bidir_workspace_bytes(ss.make_dims(2, 1024, 1024, 16, ss.SS_F32)) == \
        a(_scan_ws(2, 1024, 1024, 16, 16)) + 2 * 1024 * 1024 * 4
    # sequences shorter than two 16-token chunks stay in one chunk (no workspace)
    assert ss.ss_workspace_bytes(ss.make_dims(2, 31, 1024, 16, ss.SS_F32)) == 0


def test_scan_plan_matches_the_chunk_rules():
    """ss_scan_plan reports the chunking the workspace sizes above imply, per pass."""
    P = ss.ss_scan_plan
    F = dict(lane_quad=False, carry_correction=False)
    assert P(ss.make_dims(2, 1024, 1024, 16, ss.SS_F32)) == dict(nchunks=32, chunk_len=32, lane_quad=True,
                                                                 carry_correction=False)
    assert P(ss.make_dims(2, 1024, 1024, 16, ss.SS_F32), ss.SS_PASS_BIDIR) == dict(nchunks=16, chunk_len=64, **F)
    assert P(ss.make_dims(2, 1024, 1024, 16, ss.SS_F32), ss.SS_PASS_BWD) == dict(nchunks=16, chunk_len=64, **F)
    assert P(ss.make_dims(1, 24576, 256, 16, ss.SS_BF16)) == dict(nchunks=384, chunk_len=64, **F)
    # the long workload: 2048 channels = 8 workgroups, 64 chunks of 2048 tokens, whose
    # carries are added after the main pass (chunks of at least 1024 tokens)
    assert P(ss.make_dims(1, 131072, 2048, 16, ss.SS_BF16)) == dict(nchunks=64, chunk_len=2048, lane_quad=False,
                                                                    carry_correction=True)
    for pas in (ss.SS_PASS_BIDIR, ss.SS_PASS_BWD):
        assert not P(ss.make_dims(1, 131072, 2048, 16, ss.SS_BF16), pas)["carry_correction"]
    assert P(ss.make_dims(2, 65536, 1024, 16, ss.SS_F32)) == dict(nchunks=64, chunk_len=1024, lane_quad=False,
                                                                  carry_correction=True)
    assert P(ss.make_dims(1, 65536, 1024, 16, ss.SS_F32)) == dict(nchunks=128, chunk_len=512, **F)
    # the train workload: 4 chunks of 512 tokens, aggregate pass first
    assert P(ss.make_dims(8, 2048, 5120, 16, ss.SS_BF16)) == dict(nchunks=4, chunk_len=512, **F)
    # enough channels for the GPU: one chunk
    assert P(ss.make_dims(64, 2048, 5120, 16, ss.SS_BF16)) == dict(nchunks=1, chunk_len=2048, **F)
    for L, D, B in ((4096, 64, 1), (3001, 100, 2), (65536, 1024, 2), (65536, 1024, 1)):
        for pas in (ss.SS_PASS_FWD, ss.SS_PASS_BIDIR, ss.SS_PASS_BWD):
            p = P(ss.make_dims(B, L, D, 16, ss.SS_F32), pas)
            assert (p["nchunks"] - 1) * p["chunk_len"] < L <= p["nchunks"] * p["chunk_len"], (L, D, B, pas, p)


def test_scan_plan_rejects_bad_input():
    d = ss.make_dims(1, 64, 8, 16, ss.SS_F32)
    p = ss.ss_plan()
    assert ss.lib.ss_scan_plan(ctypes.byref(d), 3, ctypes.byref(p)) == 1
    assert ss.lib.ss_scan_plan(ctypes.byref(d), 0, None) == 1
    bad = ss.make_dims(1, 64, 8, 12, ss.SS_F32)
    assert ss.lib.ss_scan_plan(ctypes.byref(bad), 0, ctypes.byref(p)) == 2
    zero = ss.make_dims(1, 0, 8, 16, ss.SS_F32)
    assert ss.lib.ss_scan_plan(ctypes.byref(zero), 0, ctypes.byref(p)) == 1


def test_noalloc_rejects_dims_beyond_its_array():
    """The allocation-free forward takes its workspace from a built-in array of
    SS_NOALLOC_MAX_WORKSPACE bytes; dims needing more are rejected on the host."""
    text = open(HEADER).read()
    assert "#define SS_NOALLOC_MAX_WORKSPACE (16u << 20)" in text
    assert ss.NOALLOC_MAX_WORKSPACE == 16 << 20
    big = _dims(batch=1, seqlen=1 << 20, d_inner=4096, d_state=64)
    assert ss.ss_workspace_bytes(big) > ss.NOALLOC_MAX_WORKSPACE
    assert ss.lib.ss_conv_scan_fwd_noalloc(ctypes.byref(big), ctypes.byref(_fake_args()), None) == 3
    assert b"built-in array" in ss.lib.ss_last_error()
    # bad dims are reported as such, not as a workspace problem
    assert ss.lib.ss_conv_scan_fwd_noalloc(ctypes.byref(_dims(d_state=12)), ctypes.byref(_fake_args()), None) == 2
    # the bench workloads fit: long (B1 L131072 D2048) and train (B8 L2048 D5120)
    assert ss.ss_workspace_bytes(ss.make_dims(1, 131072, 2048, 16, ss.SS_BF16)) <= ss.NOALLOC_MAX_WORKSPACE
    assert ss.ss_workspace_bytes(ss.make_dims(8, 2048, 5120, 16, ss.SS_BF16)) <= ss.NOALLOC_MAX_WORKSPACE


def test_workspace_alignment_and_overlap_checked():
    d = _dims(batch=1, seqlen=1 << 14, d_inner=64)
    need = ss.ss_workspace_bytes(d)
    assert _call(d, _fake_args(), (1 << 45) + 4, need) == 1
    a = _fake_args()
    assert _call(d, a, a.x, need) == 1


# ----------------------------------------------------------------------------- bidirectional

def _fake_dir(**kw):
    base = 1 << 46
    r = {}
    for i, name in enumerate(["conv_w", "conv_b", "delta", "delta_bias", "A", "B", "C", "Dskip"]):
        r[name] = base + i * (1 << 32)
    r.update(kw)
    return ss.ss_dir_args(**r)


def _bidir(dims, args, rev, ws=None, ws_bytes=0):
    return ss.lib.ss_conv_scan_bidir_fwd(ctypes.byref(dims), ctypes.byref(args),
                                         ctypes.byref(rev) if rev is not None else None, ws, ws_bytes, None)


def test_bidir_rejects_states():
    assert _bidir(_dims(), _fake_args(conv_state=None), None) == 1
    assert "no states" in ss.lib.ss_last_error().decode()
    assert _bidir(_dims(), _fake_args(ssm_state=None), None) == 1


@pytest.mark.parametrize("field", ["delta", "A", "B", "C"])
def test_bidir_null_required_backward_parameter_rejected(field):
    a = _fake_args(ssm_state=None, conv_state=None)
    assert _bidir(_dims(), a, _fake_dir(**{field: None})) == 1
    err = ss.lib.ss_last_error().decode()
    assert "backward direction" in err and field in err


def test_bidir_backward_parameters_checked():
    a = _fake_args(ssm_state=None, conv_state=None)
    assert _bidir(_dims(), a, _fake_dir(A=(1 << 46) + 4 * (1 << 32) + 2)) == 1
    assert "aligned" in ss.lib.ss_last_error().decode()
    assert _bidir(_dims(), a, _fake_dir(B=a.y + 64)) == 1
    assert "overlaps" in ss.lib.ss_last_error().decode()
    # shared parameters, or separate ones, pass validation up to the workspace check
    d = _dims(batch=1, seqlen=1 << 14, d_inner=64)
    assert _bidir(d, a, None) == 3
    assert _bidir(d, a, _fake_dir()) == 3
    need = ss.ss_bidir_workspace_bytes(d)
    # the scan's workspace plus the forward pass's fp32 output
    assert need >= ss.ss_workspace_bytes(d) + 1 * (1 << 14) * 64 * 4
    assert _bidir(d, a, _fake_dir(), 1 << 45, need - 1) == 3
    assert _bidir(d, a, _fake_dir(), (1 << 45) + 4, need) == 1
    # an unchunked shape still needs the fp32 buffer
    assert ss.ss_bidir_workspace_bytes(_dims()) == 2 * 16 * 64 * 4 and ss.ss_workspace_bytes(_dims()) == 0
    assert ss.ss_bidir_workspace_bytes(_dims(batch=0)) == 0


def test_bidir_events_consumed_by_a_failing_call():
    assert ss.lib.ss_time_next_call(1, 2, 3, 4) == 0
    assert _bidir(_dims(), _fake_args(), None) == 1
    assert ss.lib.ss_time_next_call(None, None, None, None) == 0


# ----------------------------------------------------------------------------- backward

def _fake_grads(**kw):
    base = 1 << 44
    g = {}
    for i, name in enumerate(["dy", "dstate_final", "dconv_final", "dx", "ddelta", "dz", "dB", "dC", "dA", "dDskip",
                              "dconv_w", "dconv_b", "ddelta_bias", "dstate_init", "dconv_init"]):
        g[name] = base + i * (1 << 32)
    g.update(kw)
    return ss.ss_grads(**g)


def _bwd(dims, args, grads, ws=(1 << 47), ws_bytes=None):
    if ws_bytes is None:
        ws_bytes = ss.ss_bwd_workspace_bytes(dims)
    return ss.lib.ss_conv_scan_bwd(ctypes.byref(dims), ctypes.byref(args), ctypes.byref(grads), ws, ws_bytes, None)


def test_bwd_workspace_covers_checkpoints():
    d = _dims(batch=2, seqlen=4096, d_inner=64, d_state=16)
    # at least the state after every 4th token
    assert ss.ss_bwd_workspace_bytes(d) >= 2 * (4096 // 4) * 64 * 16 * 4
    assert ss.ss_bwd_workspace_bytes(_dims(batch=0)) == 0


@pytest.mark.parametrize("field", ["dy", "dx", "ddelta", "dB", "dC", "dA"])
def test_bwd_null_required_gradient_rejected(field):
    assert _bwd(_dims(), _fake_args(), _fake_grads(**{field: None})) == 1
    assert field in ss.lib.ss_last_error().decode()


def test_bwd_validates_zoh_like_euler_and_rejects_inconsistent_optional_pieces():
    z = ss.make_dims(2, 16, 64, 16, ss.SS_F32, discretization=ss.SS_ZOH)
    assert ss.ss_bwd_workspace_bytes(z) == ss.ss_bwd_workspace_bytes(_dims())
    assert _bwd(z, _fake_args(), _fake_grads(dz=None)) == 1
    assert _bwd(z, _fake_args(), _fake_grads(), ws_bytes=ss.ss_bwd_workspace_bytes(z) - 1) == 3
    assert _bwd(_dims(), _fake_args(), _fake_grads(dz=None)) == 1                 # z given, dz missing
    assert _bwd(_dims(), _fake_args(z=None), _fake_grads()) == 1                  # dz given, no z
    assert _bwd(_dims(), _fake_args(conv_w=None, conv_state=None), _fake_grads()) == 1   # conv grads, no conv


def test_bwd_rejects_overlaps_and_small_workspace():
    a, g = _fake_args(), _fake_grads()
    assert _bwd(_dims(), a, _fake_grads(dx=a.x + 4)) == 1
    assert "overlaps" in ss.lib.ss_last_error().decode()
    assert _bwd(_dims(), a, _fake_grads(dB=g.dC + 4)) == 1
    assert _bwd(_dims(), a, g, ws_bytes=ss.ss_bwd_workspace_bytes(_dims()) - 1) == 3
    assert _bwd(_dims(), a, g, ws=(1 << 47) + 8) == 1                               # misaligned workspace


# ----------------------------------------------------------------------------- block

def _bdims(**kw):
    d = dict(batch=2, seqlen=16, d_model=64, d_inner=128, d_state=16, dt_rank=4, io_dtype=ss.SS_F32, norm_eps=1e-5)
    d.update(kw)
    return ss.block_dims(d["batch"], d["seqlen"], d["d_model"], d["d_inner"], d["d_state"], d["dt_rank"],
                         d["io_dtype"], d["norm_eps"], d_conv=d.get("d_conv", 4))


def _bweights(**kw):
    base = 1 << 45
    w = {n: base + i * (1 << 32) for i, n in enumerate(["norm_w", "W_in", "conv_w", "conv_b", "W_x", "W_dt",
                                                         "dt_bias", "A", "Dskip", "W_out"])}
    w.update(kw)
    return ss.ss_block_weights(**w)


def _block(dims, w, x=(1 << 46), out=(1 << 46) + (1 << 40), h=None, c=None, step=False, ws=(1 << 47), ws_bytes=None):
    if ws_bytes is None:
        ws_bytes = ss.ss_block_workspace_bytes(dims, step)
    fn = ss.lib.ss_block_step if step else ss.lib.ss_block_fwd
    return fn(ctypes.byref(dims), ctypes.byref(w), x, out, h, c, ws, ws_bytes, None)


def test_block_workspace_size():
    """The block's activations (xn, xi, z, u, dr, B, C, delta, y; 256-byte aligned) plus
    the scan's workspace: M = 32 rows, d_model 64, d_inner 128, R 4, N 16, fp32."""
    a = lambda v: (v + 255) // 256 * 256  # noqa: E731
    M, dm, di, R, N, es = 32, 64, 128, 4, 16, 4
    acts = a(M * dm * es) + 5 * a(M * di * es) + a(M * R * es) + 2 * a(M * N * es)
    assert ss.ss_workspace_bytes(ss.make_dims(2, 16, 128, 16, ss.SS_F32)) == 0
    assert ss.ss_block_workspace_bytes(_bdims(), False) == acts
    # a long sequence adds the chunked scan's workspace
    long = _bdims(batch=1, seqlen=1 << 14)
    scan = ss.ss_workspace_bytes(ss.make_dims(1, 1 << 14, 128, 16, ss.SS_F32))
    assert scan > 0 and ss.ss_block_workspace_bytes(long, False) >= scan + (1 << 14) * 128 * 4 * 5
    assert ss.ss_block_workspace_bytes(_bdims(batch=0), False) == 0


@pytest.mark.parametrize("field", ["norm_w", "W_in", "conv_w", "W_x", "W_dt", "A", "W_out"])
def test_block_null_weight_rejected(field):
    assert _block(_bdims(), _bweights(**{field: None})) == 1
    assert field in ss.lib.ss_last_error().decode()


def test_block_rejects_bad_arguments():
    assert _block(_bdims(norm_eps=0.0), _bweights()) == 1
    assert _block(_bdims(d_state=12), _bweights()) == 2                      # the scan's own check
    assert _block(_bdims(d_conv=3), _bweights()) == 2
    assert _block(_bdims(), _bweights(W_in=(1 << 45) + 8)) == 1               # GEMM weight not 16-byte aligned
    assert _block(_bdims(), _bweights(), out=(1 << 46) + 64) == 1              # out partly overlaps x
    assert _block(_bdims(), _bweights(), step=True) == 1                       # the step needs both states
    assert _block(_bdims(), _bweights(), ws_bytes=ss.ss_block_workspace_bytes(_bdims(), False) - 1) == 3
