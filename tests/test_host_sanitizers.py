"""The host side of the C ABI (argument validation in abi.cpp, decode planning in plan.cpp)
built with AddressSanitizer and UndefinedBehaviorSanitizer and driven on the CPU.

No device code is built: the kernel launchers are host stand-ins (tests/sanitize/stubs.cpp)
that check the invariants each kernel relies on. The driver (tests/sanitize/driver.cpp) calls
every entry point with valid shapes (which must be accepted, with the workspace and table sizes
the *_bytes queries report), with each of them made wrong in one argument (which must be
rejected with the documented status), and with pseudo-random arguments (any documented status,
always with a message). An out-of-bounds access, a signed overflow or any other undefined
behaviour aborts the run."""

from __future__ import annotations

import shutil
import subprocess
from pathlib import Path

import pytest

ROOT = Path(__file__).resolve().parents[1]
CSRC = ROOT / "sliding_window_global_amd" / "csrc"
HIP_INCLUDE = Path("/opt/rocm/include")


@pytest.mark.skipif(shutil.which("g++") is None or not (HIP_INCLUDE / "hip" / "hip_runtime.h").exists(),
                    reason="needs g++ and the HIP headers")
def test_abi_validation_under_asan_ubsan(tmp_path):
    exe = tmp_path / "drive"
    cmd = ["g++", "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
           "-D__HIP_PLATFORM_AMD__", f"-I{HIP_INCLUDE}", f"-I{ROOT / 'include'}", f"-I{CSRC}",
           str(CSRC / "abi.cpp"), str(CSRC / "plan.cpp"),
           str(ROOT / "tests" / "sanitize" / "stubs.cpp"), str(ROOT / "tests" / "sanitize" / "driver.cpp"),
           "-o", str(exe)]
    build = subprocess.run(cmd, capture_output=True, text=True, timeout=600)
    assert build.returncode == 0, build.stderr[-4000:]
    run = subprocess.run([str(exe)], capture_output=True, text=True, timeout=600,
                         env={"ASAN_OPTIONS": "abort_on_error=0:halt_on_error=1",
                              "UBSAN_OPTIONS": "print_stacktrace=1:halt_on_error=1"})
    assert run.returncode == 0, (run.stdout + run.stderr)[-4000:]
    assert "host sanitizer drive ok" in run.stdout
