"""Independent pins of the fp64 block oracle (oracle/block.py).

* an independent implementation of the whole block in torch float64 ops
  (torch.nn.functional.linear / rms_norm / conv1d, the recurrence written over
  torch tensors) compared element by element;
* W_out = 0 leaves the residual: out == x exactly;
* W_x = 0 switches the SSM's input and readout off (B = C = 0): out is
  x + (D u SiLU(z)) W_out^T, with u from torch's conv1d;
* L decode steps from the carried states reproduce the forward.
Each takes the block-oracle module so that mutated copies can be checked too.
"""
from __future__ import annotations

import numpy as np
import torch
import torch.nn.functional as F

import workloads as W
from pins import relerr

SPEC = W.BlockSpec("pin", 2, 9, 16, expand=2, d_state=4, dt_rank=3, io_dtype="f32", seed=4242)


def case(seed=0, L=9):
    rng = np.random.default_rng(seed)
    w = W.gen_block_weights(SPEC, seed=seed + 1)
    w = {k: np.asarray(v, np.float64) for k, v in w.items()}
    w["A"] = -rng.uniform(0.2, 3.0, w["A"].shape)
    w["D"] = rng.standard_normal(w["D"].shape)
    x = rng.standard_normal((2, L, SPEC.d_model))
    st = dict(ssm_state=rng.standard_normal((2, SPEC.d_inner, SPEC.d_state)),
              conv_state=rng.standard_normal((2, SPEC.d_inner, 3)))
    return w, x, st


def torch_block(w, x, R, ssm_state, conv_state):
    t = {k: torch.tensor(v, dtype=torch.float64) for k, v in w.items()}
    xt = torch.tensor(x, dtype=torch.float64)
    Bsz, L, dm = xt.shape
    di = t["W_in"].shape[0] // 2
    N = t["A"].shape[1]
    xn = F.rms_norm(xt, (dm,), weight=t["norm_w"], eps=1e-5)
    xi = F.linear(xn, t["W_in"][:di])
    z = F.linear(xn, t["W_in"][di:])
    hist = torch.tensor(conv_state, dtype=torch.float64)                         # [B, D, 3]
    full = torch.cat([hist, xi.transpose(1, 2)], dim=2)                          # [B, D, L+3]
    c = F.conv1d(full, t["conv_w"].unsqueeze(1), t["conv_b"], groups=di).transpose(1, 2)
    u = F.silu(c)
    dr = F.linear(u, t["W_x"][:R])
    Bm = F.linear(u, t["W_x"][R:R + N])
    Cm = F.linear(u, t["W_x"][R + N:])
    dt = F.softplus(F.linear(dr, t["W_dt"], t["dt_bias"]), threshold=1000.0)
    h = torch.tensor(ssm_state, dtype=torch.float64)
    ys = []
    for s in range(L):
        h = torch.exp(dt[:, s, :, None] * t["A"]) * h + (dt[:, s] * u[:, s])[:, :, None] * Bm[:, s, None, :]
        ys.append((h * Cm[:, s, None, :]).sum(-1) + t["D"] * u[:, s])
    y = torch.stack(ys, 1) * F.silu(z)
    out = xt + F.linear(y, t["W_out"])
    return out.numpy(), h.numpy(), full[:, :, L:].numpy()


def pin_block_torch(ob, seed=1):
    w, x, st = case(seed)
    out, h, cs = ob.block_forward(x, w, SPEC.rank, **st)
    ro, rh, rc = torch_block(w, x, SPEC.rank, **st)
    assert relerr(out, ro) < 1e-11, relerr(out, ro)
    # the history holds in_proj outputs, which two BLAS paths round differently
    assert relerr(h, rh) < 1e-11 and relerr(cs, rc) < 1e-13


def pin_block_residual_only(ob, seed=2):
    w, x, st = case(seed)
    w["W_out"] = np.zeros_like(w["W_out"])
    out, _, _ = ob.block_forward(x, w, SPEC.rank, **st)
    assert np.array_equal(out, x)


def pin_block_ssm_off(ob, seed=3):
    w, x, st = case(seed)
    w["W_x"] = np.zeros_like(w["W_x"])
    out, _, _ = ob.block_forward(x, w, SPEC.rank, **st)
    t = {k: torch.tensor(v, dtype=torch.float64) for k, v in w.items()}
    xt = torch.tensor(x, dtype=torch.float64)
    di = SPEC.d_inner
    xn = F.rms_norm(xt, (SPEC.d_model,), weight=t["norm_w"], eps=1e-5)
    full = torch.cat([torch.tensor(st["conv_state"]), F.linear(xn, t["W_in"][:di]).transpose(1, 2)], dim=2)
    u = F.silu(F.conv1d(full, t["conv_w"].unsqueeze(1), t["conv_b"], groups=di).transpose(1, 2))
    ref = xt + F.linear(t["D"] * u * F.silu(F.linear(xn, t["W_in"][di:])), t["W_out"])
    assert relerr(out, ref.numpy()) < 1e-12


def pin_block_steps_match_forward(ob, seed=4):
    w, x, st = case(seed, L=6)
    out, h, cs = ob.block_forward(x, w, SPEC.rank, **st)
    hs, css = st["ssm_state"], st["conv_state"]
    outs = []
    for s in range(6):
        o, hs, css = ob.block_step(x[:, s], w, SPEC.rank, hs, css)
        outs.append(o)
    assert relerr(np.stack(outs, 1), out) < 1e-13 and relerr(hs, h) < 1e-13 and relerr(css, cs) < 1e-13


BLOCK_PINS = [pin_block_torch, pin_block_residual_only, pin_block_ssm_off, pin_block_steps_match_forward]
