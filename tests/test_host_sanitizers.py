"""The host layer (parameter validation, planning, workspace layout, the C
ABI's host checks) built with g++ under AddressSanitizer and
UndefinedBehaviorSanitizer and driven by a seeded sweep of valid and hostile
parameter sets (tests/host/plan_sanitize.cpp). Any report aborts the sweep.
CPU only: no GPU code is compiled."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "decode_gsa_amd", "csrc")


@pytest.fixture(scope="module")
def sweep(tmp_path_factory):
    gxx = shutil.which("g++")
    if gxx is None:
        pytest.skip("g++ not found")
    exe = str(tmp_path_factory.mktemp("san") / "plan_sanitize")
    cmd = [gxx, "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-static-libasan",
           "-I", os.path.join(ROOT, "include"), "-I", CSRC,
           os.path.join(ROOT, "tests", "host", "plan_sanitize.cpp"), os.path.join(CSRC, "gsa_plan.cpp"),
           "-o", exe]
    r = subprocess.run(cmd, capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stderr
    return exe


@pytest.mark.parametrize("seed", [1, 2, 3])
def test_planner_under_asan_ubsan(sweep, seed):
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    r = subprocess.run([sweep, "200000", str(seed)], capture_output=True, text=True, timeout=300, env=env)
    assert r.returncode == 0, r.stderr[-4000:]
    assert r.stdout.startswith("ok "), r.stdout
    accepted = int(r.stdout.split()[3])
    assert accepted > 20000, r.stdout   # the sweep reaches the planners' accepting paths
