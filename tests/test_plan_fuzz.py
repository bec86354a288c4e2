"""fd_plan under the host sanitizers (no GPU): tests/native/fuzz_plan.cpp
drives the planner sources with random and hostile problems and options,
built with g++ -fsanitize=address,undefined. A signed overflow, an
out-of-bounds read or a malformed accepted plan fails the run."""
import os
import shutil
import subprocess

import pytest

from tests.conftest import ROOT

CSRC = os.path.join(ROOT, "decode_attention_fd_amd", "csrc")
GEN = os.path.join(ROOT, "_build", "gen")          # fd_occupancy.inc, written by the library build
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")


@pytest.mark.skipif(shutil.which("g++") is None, reason="needs g++")
@pytest.mark.skipif(not os.path.exists(os.path.join(GEN, "fd_occupancy.inc")),
                    reason="needs the library build's generated occupancy table")
def test_planner_under_sanitizers(tmp_path):
    exe = tmp_path / "fuzz_plan"
    native = os.path.join(ROOT, "tests", "native")
    subprocess.run(["g++", "-std=c++17", "-O1", "-g", "-fsanitize=address,undefined",
                    "-fno-sanitize-recover=all", "-D__HIP_PLATFORM_AMD__",
                    f"-I{os.path.join(ROOT, 'include')}", f"-I{CSRC}", f"-I{GEN}", f"-I{ROCM}/include",
                    os.path.join(native, "fuzz_plan.cpp"), os.path.join(native, "plan_stubs.cpp"),
                    os.path.join(CSRC, "plan.cpp"), os.path.join(CSRC, "api.cpp"),
                    f"-L{ROCM}/lib", "-lamdhip64", f"-Wl,-rpath,{ROCM}/lib", "-o", str(exe)],
                   check=True, timeout=300)
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0", UBSAN_OPTIONS="print_stacktrace=1")
    r = subprocess.run([str(exe), "200000"], capture_output=True, text=True, env=env, timeout=600)
    assert r.returncode == 0, r.stdout[-2000:] + r.stderr[-4000:]
    ok, rejected = (int(v) for v in r.stdout.split()[1::2])
    assert ok + rejected == 200000 and ok > 5000           # the planner's rules did run
