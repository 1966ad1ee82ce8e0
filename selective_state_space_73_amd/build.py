"""Build libselscan.so in-tree with hipcc for gfx950 (device code) and the host C ABI."""
from __future__ import annotations

import glob
import hashlib
import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libselscan.so")
# kernel units (one per I/O dtype and write rule, plus the block's elementwise kernels;
# compiled in parallel) + the C ABI layer and the block pipeline (host code, hipBLASLt)
KERNEL_UNITS = sorted(glob.glob(os.path.join(CSRC, "selscan_*.hip")))
SOURCES = KERNEL_UNITS + [os.path.join(CSRC, "selscan_api.cpp"), os.path.join(CSRC, "selscan_block.cpp")]
HEADERS = [os.path.join(CSRC, "selscan_device.h"), os.path.join(CSRC, "selscan_bwd.h"),
           os.path.join(CSRC, "selscan_block.h"), os.path.join(CSRC, "selscan_internal.h"),
           os.path.join(INCLUDE, "selscan.h")]
LIBS = ["-L/opt/rocm/lib", "-lhipblaslt", "-Wl,-rpath,/opt/rocm/lib"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
# packed fp32 instructions are disabled for all device code
DEVICE_FLAGS = ["-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]
COMMON = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", "-I", INCLUDE, "-I", CSRC,
          "-Wall", "-Wno-unused-command-line-argument"]


def _run(cmd):
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError("build step failed: " + " ".join(cmd))
    return r


def kernel_digest() -> str:
    """sha256 over the sources that decide what a launch does (the kernels' code,
    launch constants and the chunking rule of the C ABI layer), so that measurements
    taken on one build can be matched to it later."""
    h = hashlib.sha256()
    for path in sorted(SOURCES + HEADERS[:4]):
        with open(path, "rb") as f:
            h.update(os.path.basename(path).encode() + b"\0" + f.read())
    return h.hexdigest()


def build(verbose: bool = False, jobs: int = 0) -> str:
    """Compile every source (in parallel) and link libselscan.so next to this file.
    Always rebuilds."""
    objdir = os.path.join(PKG, "_build")
    os.makedirs(objdir, exist_ok=True)
    cmds, objs = [], []
    for src in SOURCES:
        obj = os.path.join(objdir, os.path.basename(src) + ".o")
        cmd = [HIPCC, *COMMON, *DEVICE_FLAGS, "-c", src, "-o", obj]
        if src.endswith(".cpp"):
            cmd = [HIPCC, *COMMON, "-x", "hip", *DEVICE_FLAGS, "-c", src, "-o", obj]
        if verbose:
            print(" ".join(cmd))
        cmds.append(cmd)
        objs.append(obj)
    jobs = jobs or min(len(cmds), os.cpu_count() or 1, 16)
    with ThreadPoolExecutor(max_workers=jobs) as ex:
        for _ in ex.map(_run, cmds):
            pass
    tmp = LIB + ".tmp"
    _run([HIPCC, "-shared", "-fPIC", f"--offload-arch={ARCH}", "-o", tmp, *objs, *LIBS])
    os.replace(tmp, LIB)
    return LIB


def is_stale() -> bool:
    if not os.path.exists(LIB):
        return True
    t = os.path.getmtime(LIB)
    return any(os.path.getmtime(s) > t for s in SOURCES + HEADERS)


if __name__ == "__main__":
    print(build(verbose=True))
