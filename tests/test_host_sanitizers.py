"""The host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU
only): libgdn's C ABI (gdn_host.cpp, with launch stubs that check every
workspace region and unit map handed to the kernels) driven by a fuzzer over
descriptors, offsets, flags and sizes, and the fp64 oracle driven over small
ragged problems and its invalid arguments. Both are built with g++ / gcc
alone; no device code is involved."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", "-g", "-O1"]


def _build_and_run(tmp_path, cmd, exe, extra_env=None):
    subprocess.run(cmd + ["-o", str(tmp_path / exe)], check=True, capture_output=True, text=True)
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0", UBSAN_OPTIONS="print_stacktrace=1",
               **(extra_env or {}))
    env.pop("LD_PRELOAD", None)
    r = subprocess.run([str(tmp_path / exe)], capture_output=True, text=True, env=env, timeout=300)
    assert r.returncode == 0, r.stdout[-2000:] + r.stderr[-4000:]
    return r.stdout


@pytest.mark.skipif(shutil.which("g++") is None, reason="needs g++")
def test_host_abi_fuzz_under_sanitizers(tmp_path):
    csrc = os.path.join(ROOT, "chunked_gated_delta_05_amd", "csrc")
    cmd = ["g++", "-std=c++17", *SAN, "-D__HIP_PLATFORM_AMD__", "-I", os.path.join(ROOT, "include"), "-I", csrc,
           "-I", "/opt/rocm/include", os.path.join(csrc, "gdn_host.cpp"),
           os.path.join(ROOT, "tests", "sanitize", "launch_stub.cpp"),
           os.path.join(ROOT, "tests", "sanitize", "fuzz_host.cpp")]
    out = _build_and_run(tmp_path, cmd, "fuzz_host")
    print(out)
    assert "statuses:" in out


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")
def test_oracle_under_sanitizers(tmp_path):
    cmd = ["gcc", "-std=c99", *SAN, "-fopenmp", os.path.join(ROOT, "oracle", "gdn_oracle.c"),
           os.path.join(ROOT, "tests", "sanitize", "oracle_driver.c"), "-lm"]
    out = _build_and_run(tmp_path, cmd, "oracle_driver", {"OMP_NUM_THREADS": "2"})
    assert "oracle driver: ok" in out
