"""The planner's and the oracle's host code under AddressSanitizer and
UndefinedBehaviorSanitizer: tests/sanitize/plan_sanitize.cpp is built with g++
(host code only; no GPU code is compiled or run) from fsdp_sharded_state_amd/
csrc/fs_plan.cpp and oracle/fs_oracle.c and runs the exhaustive tiny layouts
(compared with the oracle element by element), re-shard planning, the
workload shapes and the error paths.  Any out-of-bounds access, leak, signed
overflow or other undefined behaviour aborts the run."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "tests", "sanitize", "plan_sanitize.cpp")


@pytest.fixture(scope="module")
def driver(tmp_path_factory):
    if not shutil.which("g++") or not shutil.which("gcc"):
        pytest.skip("no host compiler")
    out = tmp_path_factory.mktemp("sanitize")
    oracle_o = str(out / "fs_oracle.o")
    san = ["-fsanitize=address,undefined", "-fno-sanitize-recover=undefined", "-fno-omit-frame-pointer", "-g", "-O1"]
    subprocess.run(["gcc", "-std=c11", "-ffp-contract=off", *san, "-c", os.path.join(ROOT, "oracle", "fs_oracle.c"),
                    "-o", oracle_o], check=True)
    exe = str(out / "plan_sanitize")
    r = subprocess.run(["g++", "-std=c++17", "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include", *san, SRC,
                        os.path.join(ROOT, "fsdp_sharded_state_amd", "csrc", "fs_plan.cpp"), oracle_o, "-lm",
                        "-o", exe], capture_output=True, text=True)
    if r.returncode != 0 and "hip_runtime_api.h" in r.stderr:
        pytest.skip("HIP headers not available for a host build")
    assert r.returncode == 0, r.stderr
    return exe


def test_planner_and_oracle_clean_under_asan_ubsan(driver):
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0:exitcode=3:verify_asan_link_order=0",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1:exitcode=4")
    r = subprocess.run([driver], capture_output=True, text=True, env=env, timeout=600)
    assert r.returncode == 0, r.stdout[-2000:] + r.stderr[-4000:]
    assert "runtime error" not in r.stderr and "AddressSanitizer" not in r.stderr, r.stderr[-4000:]
    assert r.stdout.strip().startswith("ok:"), r.stdout
