"""Helpers shared by the GPU parity tests: move seeded inputs to the device,
call the HIP library through its C ABI binding, call the oracle on the same
values, and compare."""
from __future__ import annotations

import numpy as np
import torch

import oracle
import workloads as W

TOL = {"f32": 1e-4, "bf16": 2e-2}   # max relative error vs the fp64 oracle, per I/O dtype
IO_KEYS = ("x", "delta", "z", "B", "C")
PARAM_KEYS = ("conv_w", "conv_b", "delta_bias", "A", "D")


def maxrel(g, r) -> float:
    """max_i |g_i - r_i| / max(|r_i|, rms(r)): elementwise relative error with the
    reference's rms as the floor for elements near zero."""
    g = np.asarray(g, np.float64)
    r = np.asarray(r, np.float64)
    if r.size == 0:
        return 0.0
    floor = max(float(np.sqrt(np.mean(r * r))), 1e-30)
    return float(np.max(np.abs(g - r) / np.maximum(np.abs(r), floor)))


def to_dev(inp: dict, io: str, dev="cuda") -> dict:
    tdt = torch.bfloat16 if io == "bf16" else torch.float32
    out = {}
    for k, v in inp.items():
        if v is None:
            out[k] = None
        elif k in IO_KEYS:
            out[k] = torch.from_numpy(np.ascontiguousarray(v, np.float32)).to(dev).to(tdt)
        else:
            out[k] = torch.from_numpy(np.ascontiguousarray(v, np.float32)).to(dev)
    return out


def gpu_fwd(ss, g: dict, ssm_state=None, conv_state=None, flags=None, zoh=False):
    f = dict(conv=True, gate=True, skip=True, bias=True)
    f.update(flags or {})
    return ss.ss_conv_scan_fwd(
        g["x"], g["delta"], g["A"], g["B"], g["C"],
        conv_w=g["conv_w"] if f["conv"] else None, conv_b=g["conv_b"] if f["conv"] else None,
        delta_bias=g["delta_bias"] if f["bias"] else None, D=g["D"] if f["skip"] else None,
        z=g["z"] if f["gate"] else None, ssm_state=ssm_state, conv_state=conv_state if f["conv"] else None,
        zoh=zoh)


def oracle_fwd(inp: dict, ssm_state=None, conv_state=None, flags=None, dsel=None, zoh=False):
    """Oracle on all channels, or on the channel subset dsel (the recurrences of
    different channels are independent)."""
    f = dict(conv=True, gate=True, skip=True, bias=True)
    f.update(flags or {})
    def sel_bld(a):
        return a if dsel is None else a[:, :, dsel]
    def sel_d(a):
        return a if dsel is None else a[dsel]
    def sel_bd(a):
        return None if a is None else (a if dsel is None else a[:, dsel])
    return oracle.conv_scan_fwd(
        sel_bld(inp["x"]), sel_bld(inp["delta"]), sel_d(inp["A"]), inp["B"], inp["C"],
        conv_w=sel_d(inp["conv_w"]) if f["conv"] else None, conv_b=sel_d(inp["conv_b"]) if f["conv"] else None,
        delta_bias=sel_d(inp["delta_bias"]) if f["bias"] else None, D=sel_d(inp["D"]) if f["skip"] else None,
        z=sel_bld(inp["z"]) if f["gate"] else None, ssm_state=sel_bd(ssm_state),
        conv_state=sel_bd(conv_state) if f["conv"] else None, zoh=zoh)


def host(t: torch.Tensor) -> np.ndarray:
    return t.float().cpu().numpy()


def check_fwd(ss, spec, *, seed=None, shape=None, states=False, flags=None, dsel=None, label="", zoh=False):
    """One ss_conv_scan_fwd call on seeded inputs against the oracle (all channels,
    or the subset dsel): y and ssm_state to the dtype's tolerance, conv history exact."""
    shape = shape or {}
    inp = W.gen_scan_inputs(spec, seed=seed, **shape)
    return check_inputs(ss, inp, spec.io_dtype, states=states, flags=flags, dsel=dsel, label=label, zoh=zoh)


def check_inputs(ss, inp, io, *, states=False, flags=None, dsel=None, label="", zoh=False, state_tol=None):
    Bsz, L, Dn = inp["x"].shape
    N = inp["A"].shape[1]
    st = W.gen_states(Bsz, Dn, N) if states else None
    g = to_dev(inp, io)
    hs = torch.from_numpy(st["ssm_state"]).cuda() if states else None
    cs = torch.from_numpy(st["conv_state"]).cuda() if states else None
    y = gpu_fwd(ss, g, hs, cs, flags, zoh=zoh)
    torch.cuda.synchronize()
    yr, hr, cr = oracle_fwd(inp, st["ssm_state"] if states else None, st["conv_state"] if states else None,
                            flags, dsel, zoh=zoh)
    yg = host(y) if dsel is None else host(y[:, :, torch.as_tensor(dsel, device=y.device)])
    tol = TOL[io]
    e = maxrel(yg, yr)
    print(f"{label} y maxrel {e:.3e}", flush=True)
    assert e <= tol, (label, e)
    if states:
        hg = host(hs) if dsel is None else host(hs)[:, dsel]
        eh = maxrel(hg, hr)
        assert eh <= (state_tol or tol), (label, "ssm_state", eh)
        if (flags or {}).get("conv", True):
            cg = host(cs) if dsel is None else host(cs)[:, dsel]
            assert np.array_equal(cg.astype(np.float64), cr), (label, "conv_state")
    return e
