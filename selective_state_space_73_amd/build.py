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
# the benchmark's calibration kernels (include/selscan_probes.h), a library of their own
PROBE_LIB = os.path.join(PKG, "libselscan_probes.so")
PROBE_SOURCES = [os.path.join(PKG, "csrc", "probes.hip")]
# kernel units (one per I/O dtype and write rule, plus the block's kernels; compiled in
# parallel) + the C ABI layer and the block pipeline (host code)
KERNEL_UNITS = sorted(glob.glob(os.path.join(CSRC, "selscan_*.hip")))
SOURCES = KERNEL_UNITS + [os.path.join(CSRC, "selscan_api.cpp"), os.path.join(CSRC, "selscan_block.cpp")]
HEADERS = [os.path.join(CSRC, "selscan_device.h"), os.path.join(CSRC, "selscan_bwd.h"),
           os.path.join(CSRC, "selscan_block.h"), os.path.join(CSRC, "selscan_gemm.h"),
           os.path.join(CSRC, "selscan_internal.h"), os.path.join(INCLUDE, "selscan.h")]
LIBS = []

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
# packed fp32 instructions are disabled for all device code. Fully unrolled loops
# (#pragma unroll) may be large: the zero-order-hold backward at d_state 64 exceeds
# the compiler's default size limit for them, and a loop left rolled indexes its
# per-state arrays at run time and moves them to scratch memory.
DEVICE_FLAGS = ["-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", "-mllvm", "-pragma-unroll-threshold=200000"]
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
    for path in sorted(SOURCES + HEADERS[:5]):
        with open(path, "rb") as f:
            h.update(os.path.basename(path).encode() + b"\0" + f.read())
    return h.hexdigest()


OBJDIR = os.path.join(PKG, "_build")
RESOURCES = os.path.join(OBJDIR, "kernel_resources.txt")


def build(verbose: bool = False, jobs: int = 0) -> str:
    """Compile every source (in parallel) and link libselscan.so next to this file.
    Always rebuilds. The compiler's per-kernel resource report (registers, scratch,
    spills, occupancy) of the kernel units is kept in _build/kernel_resources.txt."""
    os.makedirs(OBJDIR, exist_ok=True)
    cmds, objs = [], []
    for src in SOURCES:
        obj = os.path.join(OBJDIR, os.path.basename(src) + ".o")
        cmd = [HIPCC, *COMMON, *DEVICE_FLAGS, "-Rpass-analysis=kernel-resource-usage", "-c", src, "-o", obj]
        if src.endswith(".cpp"):
            cmd = [HIPCC, *COMMON, "-x", "hip", *DEVICE_FLAGS, "-c", src, "-o", obj]
        if verbose:
            print(" ".join(cmd))
        cmds.append(cmd)
        objs.append(obj)
    probe_objs = []
    for src in PROBE_SOURCES:
        obj = os.path.join(OBJDIR, os.path.basename(src) + ".o")
        cmds.append([HIPCC, *COMMON, *DEVICE_FLAGS, "-c", src, "-o", obj])
        probe_objs.append(obj)
    jobs = jobs or min(len(cmds), os.cpu_count() or 1, 16)
    with ThreadPoolExecutor(max_workers=jobs) as ex:
        reports = [r.stderr for r in ex.map(_run, cmds)]
    with open(RESOURCES, "w") as f:
        f.write("\n".join(reports[:len(objs)]))
    tmp = LIB + ".tmp"
    _run([HIPCC, "-shared", "-fPIC", f"--offload-arch={ARCH}", "-o", tmp, *objs, *LIBS])
    os.replace(tmp, LIB)
    tmp = PROBE_LIB + ".tmp"
    _run([HIPCC, "-shared", "-fPIC", f"--offload-arch={ARCH}", "-o", tmp, *probe_objs])
    os.replace(tmp, PROBE_LIB)
    return LIB


def kernel_resources(path: str = RESOURCES) -> dict:
    """Per-kernel resource usage from the last build's report: mangled name ->
    {"vgpr", "agpr", "scratch" (bytes per lane), "vgpr_spill", "occupancy"}."""
    import re
    out, cur = {}, None
    keys = {"VGPRs": "vgpr", "AGPRs": "agpr", "ScratchSize [bytes/lane]": "scratch", "VGPRs Spill": "vgpr_spill",
            "Occupancy [waves/SIMD]": "occupancy"}
    with open(path) as f:
        for line in f:
            m = re.search(r"remark:\s+Function Name: (\S+)", line)
            if m:
                cur = out.setdefault(m.group(1), {})
                continue
            m = re.search(r"remark:\s+([A-Za-z ]+(?:\[[^\]]*\])?): (\d+) \[", line)
            if m and cur is not None and m.group(1).strip() in keys:
                cur[keys[m.group(1).strip()]] = int(m.group(2))
    return out


def is_stale() -> bool:
    if not os.path.exists(LIB):
        return True
    t = os.path.getmtime(LIB)
    return any(os.path.getmtime(s) > t for s in SOURCES + HEADERS)


if __name__ == "__main__":
    print(build(verbose=True))
