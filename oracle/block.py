"""fp64 oracle of the Mamba block around the selective scan (forward and decode step).

TEST INFRASTRUCTURE ONLY (like the rest of this package): the tests, the smoke
check and the benchmark's CPU baseline may use it; the HIP library never does.

The block, as the pages describe it (bembew.net "Overview of Mamba (SSM) Model",
"How the Mamba Block Works"; ozercemkelahmet.com "Mamba", "The block"; inferensys.com
"Mamba", block list; ai360xpert.com "Mamba", "What the Mamba block looks like"):
a linear projection widens the input into a main branch and a gate branch; the
main branch goes through a short causal depthwise conv and SiLU and then the
selective SSM, whose step size, B and C are small linear projections of that
branch (ai360xpert.com "The selection mechanism": a small learned linear
projection W_Delta; ozercemkelahmet.com "What selective means", "Step 3"); the SSM
output (with its D skip) is gated by SiLU of the gate branch and projected back to
the model width; blocks are stacked with a normalisation and a residual connection.

Readings where the pages are silent (each is a plain choice, also stated where the
library documents the block):
  * pre-norm residual: out = x + out_proj(block(norm(x)));
  * the normalisation is RMSNorm with a learned scale, eps 1e-5;
  * the step size is low rank: delta = W_dt (W_x_delta u) with the bias of W_dt
    inside the softplus (the scan's delta_bias); rank R given by the caller;
  * in_proj, x_proj and out_proj have no bias.

Weights (row-major, as y = v @ W.T):
  norm_w [d_model]; W_in [2*d_inner, d_model] (rows 0..d_inner-1 give the main
  branch, the rest the gate z); conv_w [d_inner, 4], conv_b [d_inner];
  W_x [R + 2N, d_inner] (rows: delta, then B, then C); W_dt [d_inner, R];
  dt_bias [d_inner]; A [d_inner, N]; D [d_inner]; W_out [d_model, d_inner].
The scan itself is the C oracle's conv_scan_fwd / step (pinned on its own); u is
computed here (conv + SiLU) because x_proj reads it, and the scan runs with the
conv off on u.
"""
from __future__ import annotations

import numpy as np

from . import default as _scan

NORM_EPS = 1e-5


def rms_norm(x, w, eps=NORM_EPS):
    x = np.asarray(x, np.float64)
    return x / np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + eps) * np.asarray(w, np.float64)


def silu(v):
    return v / (1.0 + np.exp(-v))


def conv_silu(xi, conv_w, conv_b, conv_state=None):
    """Causal depthwise conv (width K, tap K-1 on the current token) over the history
    plus the sequence, then SiLU. xi [B,L,D]; conv_state [B,D,K-1] or None (zeros).
    Returns (u [B,L,D], the new history [B,D,K-1])."""
    xi = np.asarray(xi, np.float64)
    Bsz, L, D = xi.shape
    K = conv_w.shape[1]
    hist = np.zeros((Bsz, K - 1, D)) if conv_state is None else np.transpose(np.asarray(conv_state, np.float64), (0, 2, 1))
    full = np.concatenate([hist, xi], axis=1)                     # [B, L+K-1, D]
    c = np.broadcast_to(np.asarray(conv_b, np.float64), (Bsz, L, D)).copy()
    for k in range(K):
        c += conv_w[:, k] * full[:, k:k + L, :]
    return silu(c), np.ascontiguousarray(np.transpose(full[:, L:, :], (0, 2, 1)))


def block_forward(x, W, R, ssm_state=None, conv_state=None):
    """Block forward over a sequence. x [B,L,d_model]; W: dict of the weights above.
    ssm_state [B,d_inner,N], conv_state [B,d_inner,K-1] (None: zero). Returns
    (out [B,L,d_model], final ssm_state, final conv_state) in float64."""
    x = np.asarray(x, np.float64)
    Bsz, L, _ = x.shape
    Din = W["W_in"].shape[0] // 2
    N = W["A"].shape[1]
    xn = rms_norm(x, W["norm_w"])
    proj = xn @ np.asarray(W["W_in"], np.float64).T
    xi, z = proj[..., :Din], proj[..., Din:]
    u, cs = conv_silu(xi, W["conv_w"], W["conv_b"], conv_state)
    xp = u @ np.asarray(W["W_x"], np.float64).T
    dr, Bm, Cm = xp[..., :R], xp[..., R:R + N], xp[..., R + N:]
    delta = dr @ np.asarray(W["W_dt"], np.float64).T
    h0 = np.zeros((Bsz, Din, N)) if ssm_state is None else ssm_state
    y, hs, _ = _scan().conv_scan_fwd(u, delta, W["A"], Bm, Cm, delta_bias=W["dt_bias"], D=W["D"], z=z,
                                     ssm_state=h0)
    out = x + y @ np.asarray(W["W_out"], np.float64).T
    return out, hs, cs


def block_step(x, W, R, ssm_state, conv_state):
    """One decode token for every stream: x [S,d_model]; both states required.
    Returns (out [S,d_model], new ssm_state, new conv_state)."""
    out, hs, cs = block_forward(np.asarray(x, np.float64)[:, None, :], W, R, ssm_state, conv_state)
    return out[:, 0, :], hs, cs
