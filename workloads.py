"""Seeded synthetic inputs for the selective-scan (S6) forward path and its decode step.

This module only draws random numbers and rounds them to the I/O dtype. It
holds none of the method's arithmetic (no conv, softplus, discretisation,
recurrence or gate), so both the fp64 oracle under ``oracle/`` and the HIP
library can be fed from it without sharing any of the computation.

Workloads (shapes and value distributions are the ones named for each case):

* ``tiny``   batch 1, L=64, d_inner=8, d_state=4, fp32.
* ``block``  batch 2, L=1024, d_inner=1024 (d_model 512 x expand 2), d_state 16,
             fp32; the block shape of the ``Mamba(d_model=512, d_state=16,
             d_conv=4, expand=2)`` example on the bembew.net page ("Code Example").
* ``train``  batch 8, L=2048, d_inner 5120, d_state 16, bf16 x/delta/z/B/C.
* ``long``   batch 1, L=131072, d_inner 2048, d_state 16, bf16.
* ``decode`` 64 streams x 32 layers, d_inner 8192, d_state 16, 256 steps,
             bf16 token inputs, fp32 SSM and conv state.

Value recipe (draw order conv_w, conv_b, b_delta, A, D, x, delta, z, B, C):

* ``tiny``/``block``: x, z, B, C, delta ~ N(0,1); b_delta[d] = inverse-softplus of
  a log-uniform draw in [1e-3, 1e-1]; A[d,n] = -(n+1); D = 1;
  conv_w ~ U(-0.5, 0.5); conv_b = 0.
* ``train``/``long``/``decode``: x, z, B, C ~ N(0,1); a step size drawn
  log-uniform in [1e-3, 1e-1] per element and stored as its inverse-softplus
  in the I/O dtype, b_delta = 0; D ~ N(0,1); A[d,n] = -(n+1);
  conv_w ~ U(-0.5, 0.5); conv_b = 0.

A[d,n] = -(n+1) is the A_log = log(1..N) initialisation of the slow PyTorch
reference on the ozercemkelahmet.com page ("A minimal selective scan in
PyTorch"). All values are returned as float32 arrays whose entries are
exactly representable in the I/O dtype (bf16 values are rounded to nearest
even), so widening them to float64 is exact.
"""
from __future__ import annotations

import dataclasses
from typing import Dict, Optional

import numpy as np

__all__ = [
    "ScanSpec", "WORKLOADS", "bf16_round", "bf16_bits", "gen_scan_inputs",
    "gen_states", "gen_decode_layer_params", "gen_decode_step_inputs",
    "DecodeSpec", "DECODE", "BlockSpec", "BLOCKS", "gen_block_weights", "gen_block_input",
]

SEED_BASE = 73000


@dataclasses.dataclass(frozen=True)
class ScanSpec:
    name: str
    batch: int
    seqlen: int
    d_inner: int
    d_state: int
    d_conv: int = 4
    io_dtype: str = "f32"          # "f32" | "bf16"
    delta_mode: str = "bias"       # "bias": delta~N(0,1) + inverse-softplus bias; "direct": log-uniform step stored as delta
    seed: int = SEED_BASE


@dataclasses.dataclass(frozen=True)
class DecodeSpec:
    name: str
    streams: int
    layers: int
    d_inner: int
    d_state: int
    steps: int
    pool: int = 16                 # distinct step-input sets per layer, used as step % pool
    d_conv: int = 4
    io_dtype: str = "bf16"
    seed: int = SEED_BASE + 4


WORKLOADS: Dict[str, ScanSpec] = {
    "tiny": ScanSpec("tiny", 1, 64, 8, 4, io_dtype="f32", delta_mode="bias", seed=SEED_BASE + 0),
    "block": ScanSpec("block", 2, 1024, 1024, 16, io_dtype="f32", delta_mode="bias", seed=SEED_BASE + 1),
    "train": ScanSpec("train", 8, 2048, 5120, 16, io_dtype="bf16", delta_mode="direct", seed=SEED_BASE + 2),
    "long": ScanSpec("long", 1, 131072, 2048, 16, io_dtype="bf16", delta_mode="direct", seed=SEED_BASE + 3),
}

DECODE = DecodeSpec("decode", streams=64, layers=32, d_inner=8192, d_state=16, steps=256)


def bf16_round(a: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bfloat16 (ties to even); return float32."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    bits = a.view(np.uint32)
    lsb = (bits >> np.uint32(16)) & np.uint32(1)
    rounded = (bits + np.uint32(0x7FFF) + lsb) & np.uint32(0xFFFF0000)
    return rounded.view(np.float32)


def bf16_bits(a: np.ndarray) -> np.ndarray:
    """Upper 16 bits of float32 values that are already bf16-representable."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    return (a.view(np.uint32) >> np.uint32(16)).astype(np.uint16)


def _to_io(a: np.ndarray, io_dtype: str) -> np.ndarray:
    a = np.asarray(a, dtype=np.float32)
    if io_dtype == "bf16":
        return bf16_round(a)
    if io_dtype == "f32":
        return a
    raise ValueError(f"unknown io dtype {io_dtype!r}")


def _normal(rng: np.random.Generator, shape) -> np.ndarray:
    return rng.standard_normal(size=shape, dtype=np.float32)


def _log_uniform(rng: np.random.Generator, shape, lo=1e-3, hi=1e-1) -> np.ndarray:
    return np.exp(rng.uniform(np.log(lo), np.log(hi), size=shape))


def _inv_softplus(s: np.ndarray) -> np.ndarray:
    # the value v whose softplus is s: v = log(exp(s) - 1)
    return np.log(np.expm1(np.asarray(s, dtype=np.float64)))


def _params(rng: np.random.Generator, d_inner: int, d_state: int, d_conv: int,
            delta_mode: str) -> Dict[str, np.ndarray]:
    conv_w = rng.uniform(-0.5, 0.5, size=(d_inner, d_conv)).astype(np.float32)
    conv_b = np.zeros(d_inner, dtype=np.float32)
    if delta_mode == "bias":
        delta_bias = _inv_softplus(_log_uniform(rng, d_inner)).astype(np.float32)
    else:
        delta_bias = np.zeros(d_inner, dtype=np.float32)
    A = -np.broadcast_to(np.arange(1, d_state + 1, dtype=np.float32), (d_inner, d_state)).copy()
    if delta_mode == "bias":
        Dskip = np.ones(d_inner, dtype=np.float32)
    else:
        Dskip = _normal(rng, d_inner)
    return dict(conv_w=conv_w, conv_b=conv_b, delta_bias=delta_bias, A=A, D=Dskip)


def gen_scan_inputs(spec: ScanSpec, seed: Optional[int] = None,
                    batch: Optional[int] = None, seqlen: Optional[int] = None,
                    d_inner: Optional[int] = None, d_state: Optional[int] = None) -> Dict[str, np.ndarray]:
    """Draw one full-sequence workload. Shape overrides allow ragged test cases
    drawn with the same distributions. Returns float32 arrays:
    conv_w [D,K], conv_b [D], delta_bias [D], A [D,N], D [D], x/delta/z [B,L,D], B/C [B,L,N]."""
    Bsz = spec.batch if batch is None else batch
    L = spec.seqlen if seqlen is None else seqlen
    Dn = spec.d_inner if d_inner is None else d_inner
    N = spec.d_state if d_state is None else d_state
    rng = np.random.default_rng(spec.seed if seed is None else seed)
    out = _params(rng, Dn, N, spec.d_conv, spec.delta_mode)
    out["x"] = _to_io(_normal(rng, (Bsz, L, Dn)), spec.io_dtype)
    if spec.delta_mode == "bias":
        out["delta"] = _to_io(_normal(rng, (Bsz, L, Dn)), spec.io_dtype)
    else:
        out["delta"] = _to_io(_inv_softplus(_log_uniform(rng, (Bsz, L, Dn))), spec.io_dtype)
    out["z"] = _to_io(_normal(rng, (Bsz, L, Dn)), spec.io_dtype)
    out["B"] = _to_io(_normal(rng, (Bsz, L, N)), spec.io_dtype)
    out["C"] = _to_io(_normal(rng, (Bsz, L, N)), spec.io_dtype)
    return out


def gen_states(batch: int, d_inner: int, d_state: int, d_conv: int = 4,
               seed: int = SEED_BASE + 100) -> Dict[str, np.ndarray]:
    """N(0,1) initial SSM state [B,D,N] and conv history [B,D,K-1] (float32)."""
    rng = np.random.default_rng(seed)
    return dict(ssm_state=_normal(rng, (batch, d_inner, d_state)),
                conv_state=_normal(rng, (batch, d_inner, d_conv - 1)))


def gen_decode_layer_params(spec: DecodeSpec, layer: int) -> Dict[str, np.ndarray]:
    """Per-layer parameters of the decode workload (each layer has its own)."""
    rng = np.random.default_rng([spec.seed, layer, 0])
    return _params(rng, spec.d_inner, spec.d_state, spec.d_conv, "direct")


def gen_decode_step_inputs(spec: DecodeSpec, layer: int, slot: int,
                           streams: Optional[int] = None) -> Dict[str, np.ndarray]:
    """Single-token inputs of one pool slot of one layer: x/delta/z [S,D], B/C [S,N]."""
    S = spec.streams if streams is None else streams
    rng = np.random.default_rng([spec.seed, layer, 1 + slot])
    D, N = spec.d_inner, spec.d_state
    return dict(
        x=_to_io(_normal(rng, (S, D)), spec.io_dtype),
        delta=_to_io(_inv_softplus(_log_uniform(rng, (S, D))), spec.io_dtype),
        z=_to_io(_normal(rng, (S, D)), spec.io_dtype),
        B=_to_io(_normal(rng, (S, N)), spec.io_dtype),
        C=_to_io(_normal(rng, (S, N)), spec.io_dtype),
    )


# ---------------------------------------------------------------------------
# The Mamba block around the scan: seeded random weights of the block's shape
# (the Mamba(d_model=512, d_state=16, d_conv=4, expand=2) example on the bembew.net
# page, "Code Example") and its input. Draws only; the block's arithmetic lives in
# the oracle and in the library.

@dataclasses.dataclass(frozen=True)
class BlockSpec:
    name: str
    batch: int
    seqlen: int
    d_model: int
    expand: int = 2
    d_state: int = 16
    d_conv: int = 4
    dt_rank: int = 0               # 0: ceil(d_model / 16)
    io_dtype: str = "f32"
    seed: int = SEED_BASE + 10

    @property
    def d_inner(self) -> int:
        return self.expand * self.d_model

    @property
    def rank(self) -> int:
        return self.dt_rank or -(-self.d_model // 16)


BLOCKS: Dict[str, BlockSpec] = {
    "block_f32": BlockSpec("block_f32", 2, 1024, 512, io_dtype="f32", seed=SEED_BASE + 10),
    "block_bf16": BlockSpec("block_bf16", 2, 1024, 512, io_dtype="bf16", seed=SEED_BASE + 11),
    # training-shaped block: d_inner 5120 as the train workload
    "block_train": BlockSpec("block_train", 8, 2048, 2560, io_dtype="bf16", seed=SEED_BASE + 12),
}


def gen_block_weights(spec: BlockSpec, seed: Optional[int] = None) -> Dict[str, np.ndarray]:
    """Random-init weights (float32 arrays; GEMM weights rounded to the I/O dtype):
    norm_w ~ 1 + 0.1 N(0,1); W_in [2 d_inner, d_model] ~ N(0, 1/d_model);
    conv_w ~ U(-0.5, 0.5), conv_b ~ U(-0.1, 0.1); W_x [R + 2N, d_inner] ~ N(0, 1/d_inner);
    W_dt [d_inner, R] ~ N(0, 1/R) / 2; dt_bias = inverse-softplus of a log-uniform draw
    in [1e-3, 1e-1]; A = -(n+1); D = 1; W_out [d_model, d_inner] ~ N(0, 1/d_inner)."""
    rng = np.random.default_rng([spec.seed if seed is None else seed, 7])
    dm, di, N, R = spec.d_model, spec.d_inner, spec.d_state, spec.rank
    io = spec.io_dtype
    W = dict(
        norm_w=(1.0 + 0.1 * _normal(rng, dm)).astype(np.float32),
        W_in=_to_io(_normal(rng, (2 * di, dm)) / np.float32(np.sqrt(dm)), io),
        conv_w=rng.uniform(-0.5, 0.5, size=(di, spec.d_conv)).astype(np.float32),
        conv_b=rng.uniform(-0.1, 0.1, size=di).astype(np.float32),
        W_x=_to_io(_normal(rng, (R + 2 * N, di)) / np.float32(np.sqrt(di)), io),
        W_dt=_to_io(_normal(rng, (di, R)) / np.float32(2.0 * np.sqrt(R)), io),
        dt_bias=_inv_softplus(_log_uniform(rng, di)).astype(np.float32),
        A=-np.broadcast_to(np.arange(1, N + 1, dtype=np.float32), (di, N)).copy(),
        D=np.ones(di, dtype=np.float32),
        W_out=_to_io(_normal(rng, (dm, di)) / np.float32(np.sqrt(di)), io),
    )
    return W


def gen_block_input(spec: BlockSpec, seed: Optional[int] = None, batch: Optional[int] = None,
                    seqlen: Optional[int] = None) -> np.ndarray:
    """x [B, L, d_model] ~ N(0,1) in the I/O dtype (float32 array)."""
    rng = np.random.default_rng([spec.seed if seed is None else seed, 8])
    Bsz = spec.batch if batch is None else batch
    L = spec.seqlen if seqlen is None else seqlen
    return _to_io(_normal(rng, (Bsz, L, spec.d_model)), spec.io_dtype)
