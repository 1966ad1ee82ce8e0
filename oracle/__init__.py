"""fp64 CPU oracle for the selective-scan (S6) forward path, its decode step, its
backward (gradients of every input) and the bidirectional scan.

TEST INFRASTRUCTURE ONLY: the tests, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this package; the HIP library
and its Python binding never do. It shares no code with them.

The computation lives in ``selscan_oracle.c`` (plain C, fp64, one sequential
loop per channel, OpenMP across independent channels). This wrapper only
builds that file with gcc, widens arrays to float64 and marshals pointers.

Pinned by ``tests/test_oracle_pins.py`` (closed form, LTI convolution,
worked example, limits, conv impulse / library conv, gate and skip,
softplus through a cumulative sum; for the zero-order-hold variant: Van Loan
``expm``, equilibrium, composition of steps; for the bidirectional scan: the
unrolled two-sided closed form, a two-sided LTI convolution by ``numpy.fft`` and
the mirror symmetry) and ``tests/test_oracle_mutants.py``.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading
from typing import Optional

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "selscan_oracle.c")
LIB = os.path.join(HERE, "liboracle.so")

_lock = threading.Lock()


def build(src: str = SRC, out: str = LIB, extra_flags=()) -> str:
    """Compile the oracle with gcc (fp64, no fast-math)."""
    cmd = ["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c11", "-Wall",
           *extra_flags, "-o", out + ".tmp", src, "-lm"]
    subprocess.run(cmd, check=True, capture_output=True, text=True)
    os.replace(out + ".tmp", out)
    return out


def _stale(lib: str, src: str) -> bool:
    return (not os.path.exists(lib)) or os.path.getmtime(lib) < os.path.getmtime(src)


_dp = ctypes.POINTER(ctypes.c_double)


class Oracle:
    """Handle on one compiled oracle library (the default one, or a test mutant)."""

    def __init__(self, path: Optional[str] = None):
        if path is None:
            with _lock:
                if _stale(LIB, SRC):
                    build()
            path = LIB
        self.path = path
        lib = ctypes.CDLL(path)
        args = [ctypes.c_int64] * 5 + [_dp] * 13 + [ctypes.c_int, ctypes.c_int]
        lib.oracle_conv_scan_fwd.argtypes = args
        lib.oracle_conv_scan_fwd.restype = ctypes.c_int
        lib.oracle_step.argtypes = [ctypes.c_int64] * 4 + [_dp] * 13 + [ctypes.c_int, ctypes.c_int]
        lib.oracle_step.restype = ctypes.c_int
        lib.oracle_conv_scan_bwd.argtypes = [ctypes.c_int64] * 5 + [_dp] * 27 + [ctypes.c_int, ctypes.c_int]
        lib.oracle_conv_scan_bwd.restype = ctypes.c_int
        lib.oracle_conv_scan_bidir.argtypes = [ctypes.c_int64] * 5 + [_dp] * 19 + [ctypes.c_int, ctypes.c_int]
        lib.oracle_conv_scan_bidir.restype = ctypes.c_int
        self._lib = lib

    @staticmethod
    def _in(a, shape=None):
        if a is None:
            return None, None
        arr = np.ascontiguousarray(np.asarray(a, dtype=np.float64))
        if shape is not None and arr.shape != tuple(shape):
            raise ValueError(f"shape {arr.shape} != {tuple(shape)}")
        return arr, arr.ctypes.data_as(_dp)

    def conv_scan_fwd(self, x, delta, A, B, C, *, conv_w=None, conv_b=None, delta_bias=None,
                      D=None, z=None, ssm_state=None, conv_state=None, zoh: bool = False,
                      nthreads: int = 0):
        """Full-sequence forward (zoh=True: zero-order-hold write term instead of Euler). x/delta/z: [B,L,D]; B/C: [B,L,N]; A: [D,N];
        conv_w: [D,K]; conv_b/delta_bias/D: [D]; ssm_state: [B,D,N]; conv_state: [B,D,K-1].
        Returns (y [B,L,D], final ssm_state or None, final conv_state or None), float64."""
        x = np.asarray(x)
        Bsz, L, Dn = x.shape
        N = np.asarray(A).shape[1]
        K = np.asarray(conv_w).shape[1] if conv_w is not None else 4
        keep = []
        def p(a, shape=None):
            arr, ptr = self._in(a, shape)
            keep.append(arr)
            return ptr
        y = np.zeros((Bsz, L, Dn), dtype=np.float64)
        hs = None if ssm_state is None else np.array(ssm_state, dtype=np.float64, copy=True, order="C")
        cs = None if conv_state is None else np.array(conv_state, dtype=np.float64, copy=True, order="C")
        rc = self._lib.oracle_conv_scan_fwd(
            Bsz, L, Dn, N, K,
            p(x), p(conv_w, (Dn, K) if conv_w is not None else None), p(conv_b, (Dn,) if conv_b is not None else None),
            p(delta, (Bsz, L, Dn)), p(delta_bias, (Dn,) if delta_bias is not None else None), p(A, (Dn, N)),
            p(B, (Bsz, L, N)), p(C, (Bsz, L, N)), p(D, (Dn,) if D is not None else None),
            p(z, (Bsz, L, Dn) if z is not None else None),
            y.ctypes.data_as(_dp),
            None if hs is None else hs.ctypes.data_as(_dp),
            None if cs is None else cs.ctypes.data_as(_dp),
            int(bool(zoh)), int(nthreads))
        if rc != 0:
            raise ValueError("oracle rejected its arguments")
        return y, hs, cs

    def step(self, x, delta, A, B, C, ssm_state, *, conv_w=None, conv_b=None, delta_bias=None,
             D=None, z=None, conv_state=None, zoh: bool = False, nthreads: int = 0):
        """One decode step. x/delta/z: [S,D]; B/C: [S,N]; states required (conv_state when conv_w).
        Returns (y [S,D], new ssm_state, new conv_state or None)."""
        x = np.asarray(x)
        S, Dn = x.shape
        y, hs, cs = self.conv_scan_fwd(
            x[:, None, :], np.asarray(delta)[:, None, :], A, np.asarray(B)[:, None, :],
            np.asarray(C)[:, None, :], conv_w=conv_w, conv_b=conv_b, delta_bias=delta_bias, D=D,
            z=None if z is None else np.asarray(z)[:, None, :], ssm_state=ssm_state,
            conv_state=conv_state, zoh=zoh, nthreads=nthreads)
        return y[:, 0, :], hs, cs


    def conv_scan_bwd(self, x, delta, A, B, C, dy, *, conv_w=None, conv_b=None, delta_bias=None, D=None,
                      z=None, ssm_state=None, conv_state=None, dstate_final=None, dconv_final=None,
                      zoh: bool = False, nthreads: int = 0):
        """Gradients through conv_scan_fwd of sum(dy * out) + sum(dstate_final * h_final)
        + sum(dconv_final * conv_history_final). ssm_state / conv_state are the INITIAL
        states (None = zero). Returns a dict: dx, ddelta, dB, dC, dA, and where the
        corresponding input exists dz, dD, dconv_w, dconv_b, ddelta_bias, dstate_init,
        dconv_init (float64)."""
        x = np.asarray(x)
        Bsz, L, Dn = x.shape
        N = np.asarray(A).shape[1]
        K = np.asarray(conv_w).shape[1] if conv_w is not None else 4
        keep = []

        def p(a, shape=None):
            arr, ptr = self._in(a, shape)
            keep.append(arr)
            return ptr

        def out(shape, cond=True):
            if not cond:
                return None, None
            arr = np.zeros(shape, dtype=np.float64)
            return arr, arr.ctypes.data_as(_dp)

        conv = conv_w is not None
        g = {}
        names = [("dx", (Bsz, L, Dn), True), ("ddelta", (Bsz, L, Dn), True), ("dz", (Bsz, L, Dn), z is not None),
                 ("dB", (Bsz, L, N), True), ("dC", (Bsz, L, N), True), ("dA", (Dn, N), True),
                 ("dD", (Dn,), D is not None), ("dconv_w", (Dn, K), conv), ("dconv_b", (Dn,), conv and conv_b is not None),
                 ("ddelta_bias", (Dn,), delta_bias is not None), ("dstate_init", (Bsz, Dn, N), True),
                 ("dconv_init", (Bsz, Dn, K - 1), conv)]
        ptrs = {}
        for name, shape, cond in names:
            arr, ptr = out(shape, cond)
            if arr is not None:
                g[name] = arr
            ptrs[name] = ptr
        rc = self._lib.oracle_conv_scan_bwd(
            Bsz, L, Dn, N, K,
            p(x), p(conv_w, (Dn, K) if conv else None), p(conv_b, (Dn,) if conv_b is not None else None),
            p(delta, (Bsz, L, Dn)), p(delta_bias, (Dn,) if delta_bias is not None else None), p(A, (Dn, N)),
            p(B, (Bsz, L, N)), p(C, (Bsz, L, N)), p(D, (Dn,) if D is not None else None),
            p(z, (Bsz, L, Dn) if z is not None else None),
            p(ssm_state, (Bsz, Dn, N) if ssm_state is not None else None),
            p(conv_state, (Bsz, Dn, K - 1) if conv_state is not None else None),
            p(dy, (Bsz, L, Dn)), p(dstate_final, (Bsz, Dn, N) if dstate_final is not None else None),
            p(dconv_final, (Bsz, Dn, K - 1) if dconv_final is not None else None),
            *[ptrs[n] for n, _, _ in names], int(bool(zoh)), int(nthreads))
        if rc != 0:
            raise ValueError("oracle rejected its arguments")
        return g


    BIDIR_KEYS = ("conv_w", "conv_b", "delta", "delta_bias", "A", "B", "C", "D")

    def conv_scan_bidir(self, x, delta, A, B, C, *, conv_w=None, conv_b=None, delta_bias=None, D=None,
                        z=None, rev: Optional[dict] = None, zoh: bool = False, nthreads: int = 0):
        """Bidirectional scan: the forward scan plus the same layer over the
        time-reversed sequence, pre-gate outputs summed, then the SiLU(z) gate.
        The arguments are the forward direction's; rev holds the backward
        direction's own parameters (keys BIDIR_KEYS; delta, A, B and C required, the
        others absent = not used), or None to share the forward's. Zero initial
        states. Returns y [B,L,D] float64."""
        x = np.asarray(x)
        Bsz, L, Dn = x.shape
        N = np.asarray(A).shape[1]
        fwd = dict(conv_w=conv_w, conv_b=conv_b, delta=delta, delta_bias=delta_bias, A=A, B=B, C=C, D=D)
        if rev is None:
            rev = fwd
        elif set(rev) - set(self.BIDIR_KEYS):
            raise ValueError(f"unknown keys in rev: {sorted(set(rev) - set(self.BIDIR_KEYS))}")
        cw = [q["conv_w"] for q in (fwd, rev) if q.get("conv_w") is not None]
        K = np.asarray(cw[0]).shape[1] if cw else 4
        keep = []

        def p(a, shape=None):
            arr, ptr = self._in(a, shape)
            keep.append(arr)
            return ptr

        def params(q):
            opt = lambda k, shape: p(q.get(k), shape if q.get(k) is not None else None)  # noqa: E731
            return [opt("conv_w", (Dn, K)), opt("conv_b", (Dn,)), p(q["delta"], (Bsz, L, Dn)),
                    opt("delta_bias", (Dn,)), p(q["A"], (Dn, N)), p(q["B"], (Bsz, L, N)), p(q["C"], (Bsz, L, N)),
                    opt("D", (Dn,))]

        y = np.zeros((Bsz, L, Dn), dtype=np.float64)
        rc = self._lib.oracle_conv_scan_bidir(
            Bsz, L, Dn, N, K, p(x), p(z, (Bsz, L, Dn) if z is not None else None), y.ctypes.data_as(_dp),
            *params(fwd), *params(rev), int(bool(zoh)), int(nthreads))
        if rc != 0:
            raise ValueError("oracle rejected its arguments")
        return y


_default: Optional[Oracle] = None


def default() -> Oracle:
    global _default
    if _default is None:
        _default = Oracle()
    return _default


def conv_scan_fwd(*args, **kwargs):
    return default().conv_scan_fwd(*args, **kwargs)


def step(*args, **kwargs):
    return default().step(*args, **kwargs)


def conv_scan_bwd(*args, **kwargs):
    return default().conv_scan_bwd(*args, **kwargs)


def conv_scan_bidir(*args, **kwargs):
    return default().conv_scan_bidir(*args, **kwargs)
