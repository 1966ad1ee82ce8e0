"""Python binding of libselscan (selective-scan S6 forward + decode step on gfx950).

Argument marshalling only: tensors are checked for device, dtype, shape and
contiguity, their data pointers and torch's current HIP stream are passed to
the C ABI declared in include/selscan.h, and every step of the computation
runs in the library's HIP kernels. There is no CPU fallback: importing the
package without a built ``libselscan.so`` raises.

Names follow the C ABI: ``ss_conv_scan_fwd``, ``ss_conv_scan_bwd``, ``ss_step``,
``ss_workspace_bytes``, ``ss_bwd_workspace_bytes``, ``ss_version``.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libselscan.so")

SS_F32, SS_BF16 = 0, 1
SS_EULER, SS_ZOH = 0, 1
STATUS = {0: "SS_OK", 1: "SS_ERR_INVALID_ARG", 2: "SS_ERR_UNSUPPORTED", 3: "SS_ERR_WORKSPACE", 4: "SS_ERR_HIP"}


class ss_dims(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int64), ("seqlen", ctypes.c_int64), ("d_inner", ctypes.c_int64),
                ("d_state", ctypes.c_int32), ("d_conv", ctypes.c_int32), ("io_dtype", ctypes.c_int32),
                ("discretization", ctypes.c_int32)]


_vp = ctypes.c_void_p


class ss_args(ctypes.Structure):
    _fields_ = [(n, _vp) for n in ("x", "conv_w", "conv_b", "delta", "delta_bias", "A", "B", "C", "Dskip",
                                   "z", "y", "ssm_state", "conv_state")]


class ss_plan(ctypes.Structure):
    _fields_ = [("nchunks", ctypes.c_int64), ("chunk_len", ctypes.c_int64), ("lane_quad", ctypes.c_int32),
                ("carry_correction", ctypes.c_int32)]


SS_PASS_FWD, SS_PASS_BIDIR, SS_PASS_BWD = 0, 1, 2


class ss_dir_args(ctypes.Structure):
    _fields_ = [(n, _vp) for n in ("conv_w", "conv_b", "delta", "delta_bias", "A", "B", "C", "Dskip")]


class ss_grads(ctypes.Structure):
    _fields_ = [(n, _vp) for n in ("dy", "dstate_final", "dconv_final", "dx", "ddelta", "dz", "dB", "dC", "dA",
                                   "dDskip", "dconv_w", "dconv_b", "ddelta_bias", "dstate_init", "dconv_init")]


class ss_block_dims(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int64), ("seqlen", ctypes.c_int64), ("d_model", ctypes.c_int64),
                ("d_inner", ctypes.c_int64), ("d_state", ctypes.c_int32), ("d_conv", ctypes.c_int32),
                ("dt_rank", ctypes.c_int32), ("io_dtype", ctypes.c_int32), ("discretization", ctypes.c_int32),
                ("norm_eps", ctypes.c_float)]


class ss_block_weights(ctypes.Structure):
    _fields_ = [(n, _vp) for n in ("norm_w", "W_in", "conv_w", "conv_b", "W_x", "W_dt", "dt_bias", "A", "Dskip",
                                   "W_out")]


class SelscanError(RuntimeError):
    def __init__(self, status: int, detail: str):
        super().__init__(f"{STATUS.get(status, status)}: {detail}")
        self.status = status


def _load() -> ctypes.CDLL:
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is not built: run __graft_entry__.build() (hipcc, gfx950)")
    lib = ctypes.CDLL(LIB_PATH)
    lib.ss_workspace_bytes.argtypes = [ctypes.POINTER(ss_dims)]
    lib.ss_workspace_bytes.restype = ctypes.c_size_t
    lib.ss_scan_plan.argtypes = [ctypes.POINTER(ss_dims), ctypes.c_int32, ctypes.POINTER(ss_plan)]
    lib.ss_scan_plan.restype = ctypes.c_int
    lib.ss_conv_scan_fwd.argtypes = [ctypes.POINTER(ss_dims), ctypes.POINTER(ss_args), _vp, ctypes.c_size_t, _vp]
    lib.ss_conv_scan_fwd.restype = ctypes.c_int
    lib.ss_conv_scan_fwd_noalloc.argtypes = [ctypes.POINTER(ss_dims), ctypes.POINTER(ss_args), _vp]
    lib.ss_conv_scan_fwd_noalloc.restype = ctypes.c_int
    lib.ss_conv_scan_bidir_fwd.argtypes = [ctypes.POINTER(ss_dims), ctypes.POINTER(ss_args),
                                           ctypes.POINTER(ss_dir_args), _vp, ctypes.c_size_t, _vp]
    lib.ss_conv_scan_bidir_fwd.restype = ctypes.c_int
    lib.ss_bidir_workspace_bytes.argtypes = [ctypes.POINTER(ss_dims)]
    lib.ss_bidir_workspace_bytes.restype = ctypes.c_size_t
    lib.ss_step.argtypes = [ctypes.POINTER(ss_dims), ctypes.POINTER(ss_args), _vp]
    lib.ss_step.restype = ctypes.c_int
    lib.ss_status_str.argtypes = [ctypes.c_int]
    lib.ss_status_str.restype = ctypes.c_char_p
    lib.ss_last_error.argtypes = []
    lib.ss_last_error.restype = ctypes.c_char_p
    lib.ss_version.argtypes = []
    lib.ss_version.restype = ctypes.c_int
    lib.ss_time_next_call.argtypes = [_vp, _vp, _vp, _vp]
    lib.ss_time_next_call.restype = ctypes.c_int
    lib.ss_bwd_workspace_bytes.argtypes = [ctypes.POINTER(ss_dims)]
    lib.ss_bwd_workspace_bytes.restype = ctypes.c_size_t
    lib.ss_conv_scan_bwd.argtypes = [ctypes.POINTER(ss_dims), ctypes.POINTER(ss_args), ctypes.POINTER(ss_grads), _vp,
                                     ctypes.c_size_t, _vp]
    lib.ss_conv_scan_bwd.restype = ctypes.c_int
    lib.ss_block_workspace_bytes.argtypes = [ctypes.POINTER(ss_block_dims), ctypes.c_int]
    lib.ss_block_workspace_bytes.restype = ctypes.c_size_t
    for name in ("ss_block_fwd", "ss_block_step"):
        fn = getattr(lib, name)
        fn.argtypes = [ctypes.POINTER(ss_block_dims), ctypes.POINTER(ss_block_weights), _vp, _vp, _vp, _vp, _vp,
                       ctypes.c_size_t, _vp]
        fn.restype = ctypes.c_int
    return lib


lib = _load()


def ss_version() -> int:
    return lib.ss_version()


def ss_time_next_call(agg_start=None, agg_stop=None, main_start=None, main_stop=None) -> None:
    """Arm hipEvent_t handles (ints) to be recorded around the kernels of the next
    ss_conv_scan_fwd / ss_conv_scan_bidir_fwd / ss_conv_scan_bwd / ss_step call on this
    thread (profiling)."""
    lib.ss_time_next_call(agg_start, agg_stop, main_start, main_stop)


def _check(status: int):
    if status != 0:
        raise SelscanError(status, lib.ss_last_error().decode())


def _io_dtype(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return SS_F32
    if t.dtype == torch.bfloat16:
        return SS_BF16
    raise TypeError(f"I/O tensors must be float32 or bfloat16, got {t.dtype}")


def _ptr(t: Optional[torch.Tensor], shape=None, dtype=None, name="") -> Optional[int]:
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    return t.data_ptr()


def make_dims(batch: int, seqlen: int, d_inner: int, d_state: int, io_dtype: int, d_conv: int = 4,
              discretization: int = SS_EULER) -> ss_dims:
    return ss_dims(batch, seqlen, d_inner, d_state, d_conv, io_dtype, discretization)


def ss_workspace_bytes(dims: ss_dims) -> int:
    return int(lib.ss_workspace_bytes(ctypes.byref(dims)))


def ss_scan_plan(dims: ss_dims, pass_: int = SS_PASS_FWD) -> dict:
    """How a call with these dims splits the sequence: {"nchunks", "chunk_len",
    "lane_quad", "carry_correction"} (pass_: SS_PASS_FWD, SS_PASS_BIDIR or SS_PASS_BWD)."""
    p = ss_plan()
    _check(lib.ss_scan_plan(ctypes.byref(dims), int(pass_), ctypes.byref(p)))
    return {"nchunks": int(p.nchunks), "chunk_len": int(p.chunk_len), "lane_quad": bool(p.lane_quad),
            "carry_correction": bool(p.carry_correction)}


def _stream_handle(stream) -> Optional[int]:
    s = torch.cuda.current_stream() if stream is None else stream
    return s.cuda_stream or None


def _build_args(x, delta, A, B, C, conv_w, conv_b, delta_bias, D, z, y, ssm_state, conv_state,
                lead, dims: ss_dims):
    io = x.dtype
    Dn, N, K = dims.d_inner, dims.d_state, dims.d_conv
    lead_bd = lead[:1] + (Dn,)
    return ss_args(
        x=_ptr(x, lead + (Dn,), io, "x"), conv_w=_ptr(conv_w, (Dn, K), torch.float32, "conv_w"),
        conv_b=_ptr(conv_b, (Dn,), torch.float32, "conv_b"), delta=_ptr(delta, lead + (Dn,), io, "delta"),
        delta_bias=_ptr(delta_bias, (Dn,), torch.float32, "delta_bias"), A=_ptr(A, (Dn, N), torch.float32, "A"),
        B=_ptr(B, lead + (N,), io, "B"), C=_ptr(C, lead + (N,), io, "C"), Dskip=_ptr(D, (Dn,), torch.float32, "D"),
        z=_ptr(z, lead + (Dn,), io, "z"), y=_ptr(y, lead + (Dn,), io, "y"),
        ssm_state=_ptr(ssm_state, lead_bd + (N,), torch.float32, "ssm_state"),
        conv_state=_ptr(conv_state, lead_bd + (K - 1,), torch.float32, "conv_state"))


def ss_conv_scan_fwd(x: torch.Tensor, delta: torch.Tensor, A: torch.Tensor, B: torch.Tensor, C: torch.Tensor, *,
                     conv_w: Optional[torch.Tensor] = None, conv_b: Optional[torch.Tensor] = None,
                     delta_bias: Optional[torch.Tensor] = None, D: Optional[torch.Tensor] = None,
                     z: Optional[torch.Tensor] = None, ssm_state: Optional[torch.Tensor] = None,
                     conv_state: Optional[torch.Tensor] = None, y: Optional[torch.Tensor] = None,
                     workspace: Optional[torch.Tensor] = None, zoh: bool = False, stream=None) -> torch.Tensor:
    """Full-sequence forward. x/delta/z: [B,L,D]; B/C: [B,L,N] (float32 or bfloat16, one dtype);
    A [D,N], conv_w [D,4], conv_b/delta_bias/D [D] float32; ssm_state [B,D,N] and conv_state [B,D,3]
    float32, updated in place when given. zoh=True selects the zero-order-hold write term
    (exp(Delta A) - 1) / A instead of Euler's Delta. Returns y [B,L,D] in the I/O dtype.
    Asynchronous on the current stream."""
    if x.dim() != 3:
        raise ValueError("x must be [batch, seqlen, d_inner]")
    Bsz, L, Dn = x.shape
    dims = make_dims(Bsz, L, Dn, A.shape[1] if A.dim() == 2 else 0, _io_dtype(x),
                     discretization=SS_ZOH if zoh else SS_EULER)
    if y is None:
        y = torch.empty_like(x)
    args = _build_args(x, delta, A, B, C, conv_w, conv_b, delta_bias, D, z, y, ssm_state, conv_state,
                       (Bsz, L), dims)
    need = ss_workspace_bytes(dims)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=x.device)
    elif workspace.numel() < need:
        raise ValueError(f"workspace has {workspace.numel()} bytes, {need} needed")
    _check(lib.ss_conv_scan_fwd(ctypes.byref(dims), ctypes.byref(args), workspace.data_ptr() if need else None,
                                workspace.numel(), _stream_handle(stream)))
    return y


class PreparedCall:
    """One C-ABI call with its argument structures built and validated once: calling the
    object re-issues it on the same tensors (whose contents the caller may change in
    place between calls) at the cost of one ctypes call. The tensors are kept alive by
    the object. Built by prepare_conv_scan_fwd."""

    def __init__(self, fn, dims, args, ws, ws_bytes, stream, keep):
        self._fn, self._dims, self._args = fn, dims, args
        self._ws, self._ws_bytes, self._stream = ws, ws_bytes, stream
        self._dref, self._aref = ctypes.byref(dims), ctypes.byref(args)
        self._keep = keep

    def __call__(self):
        _check(self._fn(self._dref, self._aref, self._ws, self._ws_bytes, self._stream))
        return self._keep["y"]


def prepare_conv_scan_fwd(x: torch.Tensor, delta: torch.Tensor, A: torch.Tensor, B: torch.Tensor, C: torch.Tensor, *,
                          conv_w: Optional[torch.Tensor] = None, conv_b: Optional[torch.Tensor] = None,
                          delta_bias: Optional[torch.Tensor] = None, D: Optional[torch.Tensor] = None,
                          z: Optional[torch.Tensor] = None, ssm_state: Optional[torch.Tensor] = None,
                          conv_state: Optional[torch.Tensor] = None, y: Optional[torch.Tensor] = None,
                          workspace: Optional[torch.Tensor] = None, zoh: bool = False, stream=None) -> PreparedCall:
    """ss_conv_scan_fwd prepared for repeated calls on the same tensors (arguments as for
    ss_conv_scan_fwd; the stream is fixed at preparation). Returns a PreparedCall whose
    call enqueues the forward and returns y."""
    if x.dim() != 3:
        raise ValueError("x must be [batch, seqlen, d_inner]")
    Bsz, L, Dn = x.shape
    dims = make_dims(Bsz, L, Dn, A.shape[1] if A.dim() == 2 else 0, _io_dtype(x),
                     discretization=SS_ZOH if zoh else SS_EULER)
    if y is None:
        y = torch.empty_like(x)
    args = _build_args(x, delta, A, B, C, conv_w, conv_b, delta_bias, D, z, y, ssm_state, conv_state,
                       (Bsz, L), dims)
    need = ss_workspace_bytes(dims)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=x.device)
    elif workspace.numel() < need:
        raise ValueError(f"workspace has {workspace.numel()} bytes, {need} needed")
    keep = dict(x=x, delta=delta, A=A, B=B, C=C, conv_w=conv_w, conv_b=conv_b, delta_bias=delta_bias, D=D, z=z,
                y=y, ssm_state=ssm_state, conv_state=conv_state, workspace=workspace)
    return PreparedCall(lib.ss_conv_scan_fwd, dims, args, workspace.data_ptr() if need else None,
                        workspace.numel(), _stream_handle(stream), keep)


NOALLOC_MAX_WORKSPACE = 16 << 20   # SS_NOALLOC_MAX_WORKSPACE


def ss_conv_scan_fwd_noalloc(x: torch.Tensor, delta: torch.Tensor, A: torch.Tensor, B: torch.Tensor,
                             C: torch.Tensor, *, conv_w: Optional[torch.Tensor] = None,
                             conv_b: Optional[torch.Tensor] = None, delta_bias: Optional[torch.Tensor] = None,
                             D: Optional[torch.Tensor] = None, z: Optional[torch.Tensor] = None,
                             ssm_state: Optional[torch.Tensor] = None, conv_state: Optional[torch.Tensor] = None,
                             y: Optional[torch.Tensor] = None, zoh: bool = False, stream=None) -> torch.Tensor:
    """ss_conv_scan_fwd with the library's built-in device workspace (no workspace
    argument; the C call allocates nothing). Pass y to keep this wrapper from
    allocating the output as well."""
    if x.dim() != 3:
        raise ValueError("x must be [batch, seqlen, d_inner]")
    Bsz, L, Dn = x.shape
    dims = make_dims(Bsz, L, Dn, A.shape[1] if A.dim() == 2 else 0, _io_dtype(x),
                     discretization=SS_ZOH if zoh else SS_EULER)
    if y is None:
        y = torch.empty_like(x)
    args = _build_args(x, delta, A, B, C, conv_w, conv_b, delta_bias, D, z, y, ssm_state, conv_state,
                       (Bsz, L), dims)
    _check(lib.ss_conv_scan_fwd_noalloc(ctypes.byref(dims), ctypes.byref(args), _stream_handle(stream)))
    return y


DIR_KEYS = ("conv_w", "conv_b", "delta", "delta_bias", "A", "B", "C", "D")


def ss_bidir_workspace_bytes(dims: ss_dims) -> int:
    return int(lib.ss_bidir_workspace_bytes(ctypes.byref(dims)))


def ss_conv_scan_bidir_fwd(x: torch.Tensor, delta: torch.Tensor, A: torch.Tensor, B: torch.Tensor,
                           C: torch.Tensor, *, conv_w: Optional[torch.Tensor] = None,
                           conv_b: Optional[torch.Tensor] = None, delta_bias: Optional[torch.Tensor] = None,
                           D: Optional[torch.Tensor] = None, z: Optional[torch.Tensor] = None,
                           rev: Optional[dict] = None, y: Optional[torch.Tensor] = None,
                           workspace: Optional[torch.Tensor] = None, zoh: bool = False, stream=None) -> torch.Tensor:
    """Bidirectional scan: the forward scan plus the same layer over the time-reversed
    sequence, y = (y_fwd + y_bwd) * SiLU(z). Arguments as for ss_conv_scan_fwd (no
    states); rev: the backward direction's own tensors keyed by DIR_KEYS (delta, A, B,
    C required, the others absent = not used), or None to share the forward's."""
    if x.dim() != 3:
        raise ValueError("x must be [batch, seqlen, d_inner]")
    Bsz, L, Dn = x.shape
    dims = make_dims(Bsz, L, Dn, A.shape[1] if A.dim() == 2 else 0, _io_dtype(x),
                     discretization=SS_ZOH if zoh else SS_EULER)
    if y is None:
        y = torch.empty_like(x)
    args = _build_args(x, delta, A, B, C, conv_w, conv_b, delta_bias, D, z, y, None, None, (Bsz, L), dims)
    rargs = None
    if rev is not None:
        unknown = set(rev) - set(DIR_KEYS)
        if unknown:
            raise ValueError(f"unknown keys in rev: {sorted(unknown)}")
        for k in ("delta", "A", "B", "C"):
            if rev.get(k) is None:
                raise ValueError(f"rev[{k!r}] is required")
        r = _build_args(x, rev["delta"], rev["A"], rev["B"], rev["C"], rev.get("conv_w"), rev.get("conv_b"),
                        rev.get("delta_bias"), rev.get("D"), None, y, None, None, (Bsz, L), dims)
        rargs = ss_dir_args(conv_w=r.conv_w, conv_b=r.conv_b, delta=r.delta, delta_bias=r.delta_bias, A=r.A,
                            B=r.B, C=r.C, Dskip=r.Dskip)
    need = ss_bidir_workspace_bytes(dims)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=x.device)
    elif workspace.numel() < need:
        raise ValueError(f"workspace has {workspace.numel()} bytes, {need} needed")
    _check(lib.ss_conv_scan_bidir_fwd(ctypes.byref(dims), ctypes.byref(args),
                                      ctypes.byref(rargs) if rargs is not None else None,
                                      workspace.data_ptr() if need else None, workspace.numel(),
                                      _stream_handle(stream)))
    return y


def ss_step(x: torch.Tensor, delta: torch.Tensor, A: torch.Tensor, B: torch.Tensor, C: torch.Tensor,
            ssm_state: torch.Tensor, *, conv_state: Optional[torch.Tensor] = None,
            conv_w: Optional[torch.Tensor] = None, conv_b: Optional[torch.Tensor] = None,
            delta_bias: Optional[torch.Tensor] = None, D: Optional[torch.Tensor] = None,
            z: Optional[torch.Tensor] = None, y: Optional[torch.Tensor] = None, zoh: bool = False,
            stream=None) -> torch.Tensor:
    """One decode step. x/delta/z: [S,D]; B/C: [S,N]; ssm_state [S,D,N] and conv_state [S,D,3]
    float32, updated in place. zoh as for ss_conv_scan_fwd. Returns y [S,D]."""
    if x.dim() != 2:
        raise ValueError("x must be [streams, d_inner]")
    S, Dn = x.shape
    dims = make_dims(S, 1, Dn, A.shape[1] if A.dim() == 2 else 0, _io_dtype(x),
                     discretization=SS_ZOH if zoh else SS_EULER)
    if y is None:
        y = torch.empty_like(x)
    args = _build_args(x, delta, A, B, C, conv_w, conv_b, delta_bias, D, z, y, ssm_state, conv_state, (S,), dims)
    _check(lib.ss_step(ctypes.byref(dims), ctypes.byref(args), _stream_handle(stream)))
    return y


def ss_bwd_workspace_bytes(dims: ss_dims) -> int:
    return int(lib.ss_bwd_workspace_bytes(ctypes.byref(dims)))


def ss_conv_scan_bwd(x: torch.Tensor, delta: torch.Tensor, A: torch.Tensor, B: torch.Tensor, C: torch.Tensor,
                     dy: torch.Tensor, *, conv_w: Optional[torch.Tensor] = None, conv_b: Optional[torch.Tensor] = None,
                     delta_bias: Optional[torch.Tensor] = None, D: Optional[torch.Tensor] = None,
                     z: Optional[torch.Tensor] = None, ssm_state: Optional[torch.Tensor] = None,
                     conv_state: Optional[torch.Tensor] = None, dstate_final: Optional[torch.Tensor] = None,
                     dconv_final: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None,
                     zoh: bool = False, stream=None) -> dict:
    """Backward of ss_conv_scan_fwd for the same inputs; ssm_state / conv_state are the
    forward's INITIAL states (read only). dy [B,L,D] in the I/O dtype; dstate_final
    [B,D,N] and dconv_final [B,D,3] float32 are the gradients of the returned states.
    Returns a dict of new tensors: dx, ddelta (I/O dtype), dB, dC, dA (float32), and
    where the input exists dz, dD, dconv_w, dconv_b, ddelta_bias (float32); always
    dstate_init and, with the conv, dconv_init (float32). Asynchronous on the stream."""
    if x.dim() != 3:
        raise ValueError("x must be [batch, seqlen, d_inner]")
    Bsz, L, Dn = x.shape
    N = A.shape[1] if A.dim() == 2 else 0
    dims = make_dims(Bsz, L, Dn, N, _io_dtype(x), discretization=SS_ZOH if zoh else SS_EULER)
    args = _build_args(x, delta, A, B, C, conv_w, conv_b, delta_bias, D, z, None, ssm_state, conv_state,
                       (Bsz, L), dims)
    dev = x.device
    f32 = dict(dtype=torch.float32, device=dev)
    out = {"dx": torch.empty_like(x), "ddelta": torch.empty_like(x), "dB": torch.empty(Bsz, L, N, **f32),
           "dC": torch.empty(Bsz, L, N, **f32), "dA": torch.empty(Dn, N, **f32),
           "dstate_init": torch.empty(Bsz, Dn, N, **f32)}
    if z is not None:
        out["dz"] = torch.empty_like(x)
    if D is not None:
        out["dD"] = torch.empty(Dn, **f32)
    if delta_bias is not None:
        out["ddelta_bias"] = torch.empty(Dn, **f32)
    if conv_w is not None:
        out["dconv_w"] = torch.empty(Dn, 4, **f32)
        out["dconv_init"] = torch.empty(Bsz, Dn, 3, **f32)
        if conv_b is not None:
            out["dconv_b"] = torch.empty(Dn, **f32)
    K = dims.d_conv
    g = ss_grads(dy=_ptr(dy, (Bsz, L, Dn), x.dtype, "dy"),
                 dstate_final=_ptr(dstate_final, (Bsz, Dn, N), torch.float32, "dstate_final"),
                 dconv_final=_ptr(dconv_final, (Bsz, Dn, K - 1), torch.float32, "dconv_final"),
                 **{k: (out[k].data_ptr() if k in out else None) for k in
                    ("dx", "ddelta", "dz", "dB", "dC", "dA", "dconv_w", "dconv_b", "ddelta_bias", "dstate_init",
                     "dconv_init")},
                 dDskip=out["dD"].data_ptr() if "dD" in out else None)
    need = ss_bwd_workspace_bytes(dims)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    elif workspace.numel() < need:
        raise ValueError(f"workspace has {workspace.numel()} bytes, {need} needed")
    _check(lib.ss_conv_scan_bwd(ctypes.byref(dims), ctypes.byref(args), ctypes.byref(g), workspace.data_ptr(),
                                workspace.numel(), _stream_handle(stream)))
    return out


BLOCK_WEIGHTS = ("norm_w", "W_in", "conv_w", "conv_b", "W_x", "W_dt", "dt_bias", "A", "D", "W_out")


def block_dims(batch: int, seqlen: int, d_model: int, d_inner: int, d_state: int, dt_rank: int, io_dtype: int,
               norm_eps: float = 1e-5, discretization: int = SS_EULER, d_conv: int = 4) -> ss_block_dims:
    return ss_block_dims(batch, seqlen, d_model, d_inner, d_state, d_conv, dt_rank, io_dtype, discretization,
                         norm_eps)


def ss_block_workspace_bytes(dims: ss_block_dims, step: bool = False) -> int:
    return int(lib.ss_block_workspace_bytes(ctypes.byref(dims), int(bool(step))))


def _block_call(step, x, W, dt_rank, ssm_state, conv_state, out, workspace, norm_eps, zoh, stream):
    io = x.dtype
    if step:
        if x.dim() != 2:
            raise ValueError("x must be [streams, d_model]")
        Bsz, dm = x.shape
        L = 1
    else:
        if x.dim() != 3:
            raise ValueError("x must be [batch, seqlen, d_model]")
        Bsz, L, dm = x.shape
    di = W["W_in"].shape[0] // 2
    N = W["A"].shape[1]
    dims = block_dims(Bsz, L, dm, di, N, dt_rank, _io_dtype(x), norm_eps, SS_ZOH if zoh else SS_EULER)
    f32 = torch.float32
    w = ss_block_weights(
        norm_w=_ptr(W["norm_w"], (dm,), f32, "norm_w"), W_in=_ptr(W["W_in"], (2 * di, dm), io, "W_in"),
        conv_w=_ptr(W["conv_w"], (di, 4), f32, "conv_w"), conv_b=_ptr(W.get("conv_b"), (di,), f32, "conv_b"),
        W_x=_ptr(W["W_x"], (dt_rank + 2 * N, di), io, "W_x"), W_dt=_ptr(W["W_dt"], (di, dt_rank), io, "W_dt"),
        dt_bias=_ptr(W.get("dt_bias"), (di,), f32, "dt_bias"), A=_ptr(W["A"], (di, N), f32, "A"),
        Dskip=_ptr(W.get("D"), (di,), f32, "D"), W_out=_ptr(W["W_out"], (dm, di), io, "W_out"))
    if out is None:
        out = torch.empty_like(x)
    need = ss_block_workspace_bytes(dims, step)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=x.device)
    elif workspace.numel() < need:
        raise ValueError(f"workspace has {workspace.numel()} bytes, {need} needed")
    fn = lib.ss_block_step if step else lib.ss_block_fwd
    _check(fn(ctypes.byref(dims), ctypes.byref(w), _ptr(x, None, io, "x"), _ptr(out, tuple(x.shape), io, "out"),
              _ptr(ssm_state, (Bsz, di, N), f32, "ssm_state"), _ptr(conv_state, (Bsz, di, 3), f32, "conv_state"),
              workspace.data_ptr(), workspace.numel(), _stream_handle(stream)))
    return out


def ss_block_fwd(x: torch.Tensor, W: dict, dt_rank: int, *, ssm_state: Optional[torch.Tensor] = None,
                 conv_state: Optional[torch.Tensor] = None, out: Optional[torch.Tensor] = None,
                 workspace: Optional[torch.Tensor] = None, norm_eps: float = 1e-5, zoh: bool = False,
                 stream=None) -> torch.Tensor:
    """Mamba block forward: x [B,L,d_model] (float32 or bfloat16) -> out, same shape.
    W: device tensors named as BLOCK_WEIGHTS (GEMM weights in the I/O dtype, the rest
    float32; conv_b, dt_bias and D optional). ssm_state [B,Di,N] / conv_state [B,Di,3]
    float32 are read and updated when given."""
    return _block_call(False, x, W, dt_rank, ssm_state, conv_state, out, workspace, norm_eps, zoh, stream)


def ss_block_step(x: torch.Tensor, W: dict, dt_rank: int, ssm_state: torch.Tensor, conv_state: torch.Tensor, *,
                  out: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None,
                  norm_eps: float = 1e-5, zoh: bool = False, stream=None) -> torch.Tensor:
    """One decode token per stream through the block: x [S,d_model] -> out [S,d_model];
    both states required and updated in place."""
    return _block_call(True, x, W, dt_rank, ssm_state, conv_state, out, workspace, norm_eps, zoh, stream)


__all__ = ["ss_conv_scan_bidir_fwd", "ss_bidir_workspace_bytes", "ss_dir_args", "DIR_KEYS", "ss_block_fwd", "ss_block_step", "ss_block_workspace_bytes", "block_dims", "ss_block_dims",
           "ss_block_weights", "BLOCK_WEIGHTS", "ss_conv_scan_fwd", "ss_conv_scan_fwd_noalloc", "prepare_conv_scan_fwd", "PreparedCall", "NOALLOC_MAX_WORKSPACE",
           "ss_conv_scan_bwd", "ss_bwd_workspace_bytes", "ss_grads", "ss_step", "ss_workspace_bytes", "ss_scan_plan", "ss_plan",
           "SS_PASS_FWD", "SS_PASS_BIDIR", "SS_PASS_BWD", "ss_version", "ss_time_next_call", "make_dims", "ss_dims", "ss_args",
           "SelscanError", "SS_F32", "SS_BF16", "SS_EULER", "SS_ZOH", "LIB_PATH", "lib"]
