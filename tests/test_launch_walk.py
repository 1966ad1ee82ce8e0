"""CPU: the host-side launch walk (tests/walk/). The block pipeline runs on the host
against fake device address ranges with its kernel launchers replaced by recorders, and
every recorded launch's address ranges are checked against the buffers they must stay
in, at the training-width block (B8 L2048 d_model 2560), 64-stream block decode at
d_model 512 and 2560, and the shapes the GPU tests use; the aggregate pass's row, tile
and LDS-row indices are checked for every d_state with 4- and 8-row groups in both scan
directions. A planted mistake (a workspace registered 4 KiB short) must be reported."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
WALK = os.path.join(ROOT, "tests", "walk")
CSRC = os.path.join(ROOT, "selective_state_space_73_amd", "csrc")
ROCM = "/opt/rocm"


@pytest.fixture(scope="module")
def walk_bin(tmp_path_factory):
    if shutil.which("g++") is None or not os.path.isdir(os.path.join(ROCM, "include", "hip")):
        pytest.skip("needs g++ and the HIP headers")
    out = str(tmp_path_factory.mktemp("walk") / "walk")
    cmd = ["g++", "-std=c++17", "-O1", "-D__HIP_PLATFORM_AMD__", "-I", os.path.join(ROCM, "include"),
           "-I", os.path.join(ROOT, "include"), "-I", CSRC, "-I", WALK,
           os.path.join(WALK, "block_walk.cpp"), os.path.join(WALK, "mock_launch.cpp"),
           os.path.join(CSRC, "selscan_api.cpp"), os.path.join(CSRC, "selscan_block.cpp"),
           "-L", os.path.join(ROCM, "lib"), "-lamdhip64", f"-Wl,-rpath,{os.path.join(ROCM, 'lib')}", "-o", out]
    subprocess.run(cmd, check=True, capture_output=True, text=True)
    return out


def test_every_launch_stays_in_its_buffers(walk_bin):
    r = subprocess.run([walk_bin], capture_output=True, text=True, timeout=300)
    print(r.stdout[-3000:])
    assert r.returncode == 0, r.stdout[-3000:]
    assert "ok: 0 violation(s)" in r.stdout
    assert "block_train B8 L2048 d2560" in r.stdout and "decode S64 d2560 bf16" in r.stdout
    assert r.stdout.count("in bounds") >= 9 * 5 * 2 * 2


def test_planted_overrun_is_reported(walk_bin):
    r = subprocess.run([walk_bin, "--plant"], capture_output=True, text=True, timeout=300)
    assert r.returncode == 1
    assert "run past workspace" in r.stdout
