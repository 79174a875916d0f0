"""Host-only check of the persistent NS loop's list scheduler: compiles
tests/ns_schedule_check.cpp with the library's ns_schedule.cpp (plain C++,
no HIP) and runs it.  See the checker's header for what it verifies."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "newton_schulz_muon_amd", "csrc")


# The second build runs the same checker under AddressSanitizer and
# UndefinedBehaviorSanitizer (host code only: the scheduler is plain C++).
SANITIZE = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", "-g"]


@pytest.mark.parametrize("flags", [[], SANITIZE], ids=["plain", "asan_ubsan"])
def test_schedule_invariants(tmp_path, flags):
    cxx = shutil.which("g++")
    if cxx is None:
        pytest.skip("g++ not available")
    exe = str(tmp_path / "ns_schedule_check")
    build = subprocess.run([cxx, "-std=c++17", "-O2", "-Wall", "-Werror", *flags, "-I", CSRC,
                            os.path.join(ROOT, "tests", "ns_schedule_check.cpp"),
                            os.path.join(CSRC, "ns_schedule.cpp"), "-o", exe],
                           capture_output=True, text=True)
    assert build.returncode == 0, build.stderr
    run = subprocess.run([exe], capture_output=True, text=True, timeout=300)
    assert run.returncode == 0 and run.stdout.strip().endswith("ALL OK"), run.stdout[-2000:]
