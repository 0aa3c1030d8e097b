"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

* The float64 oracle (oracle/gdn_oracle*.c) compiled into tests/sanitize/oracle_driver.c and run
  over small, ragged, empty and gate-limit inputs and over sizes it must reject.
* The C ABI's argument validation (gated_deltanet_linear_delta_amd/csrc/api.cpp) compiled by the
  host compiler with the kernel launchers replaced by host-only stand-ins
  (tests/sanitize/launch_stubs.cpp) and driven through every entry point with valid and invalid
  arguments and a grid of sizes up to INT_MAX (tests/sanitize/abi_driver.cpp).

Any sanitizer report aborts the program, which fails the test."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=undefined", "-g", "-O1"]
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")


def run(cmd, env_extra, timeout=300):
    env = dict(os.environ, **env_extra)
    p = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, env=env, timeout=timeout)
    return p.returncode, p.stdout.decode(errors="replace")


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not available")
def test_oracle_under_sanitizers(tmp_path):
    exe = str(tmp_path / "oracle_driver")
    srcs = [os.path.join(ROOT, "tests", "sanitize", "oracle_driver.c")] + \
           [os.path.join(ROOT, "oracle", f) for f in ("gdn_oracle.c", "gdn_oracle_bwd.c", "gdn_oracle_kda.c")]
    rc, out = run(["gcc", "-std=c11", "-Wall", "-Wextra", "-fopenmp"] + SAN + srcs + ["-lm", "-o", exe], {})
    assert rc == 0, out
    rc, out = run([exe], {"ASAN_OPTIONS": "detect_leaks=1:abort_on_error=1"})
    assert rc == 0 and "oracle driver: ok" in out, out


@pytest.mark.skipif(shutil.which("g++") is None or not os.path.exists(os.path.join(ROCM, "include", "hip")),
                    reason="g++ or the HIP headers not available")
def test_abi_validation_under_sanitizers(tmp_path):
    exe = str(tmp_path / "abi_driver")
    csrc = os.path.join(ROOT, "gated_deltanet_linear_delta_amd", "csrc")
    srcs = [os.path.join(ROOT, "tests", "sanitize", "abi_driver.cpp"), os.path.join(csrc, "api.cpp"),
            os.path.join(ROOT, "tests", "sanitize", "launch_stubs.cpp")]
    cmd = ["g++", "-std=c++17", "-Wall", "-D__HIP_PLATFORM_AMD__", "-I", os.path.join(ROCM, "include"),
           "-I", os.path.join(ROOT, "include"), "-I", csrc] + SAN + srcs + \
          ["-L", os.path.join(ROCM, "lib"), f"-Wl,-rpath,{os.path.join(ROCM, 'lib')}", "-lamdhip64", "-o", exe]
    rc, out = run(cmd, {})
    assert rc == 0, out
    # the HIP runtime keeps process-lifetime allocations, so leak checking stays off here
    rc, out = run([exe], {"ASAN_OPTIONS": "detect_leaks=0:abort_on_error=1"})
    assert rc == 0 and "abi driver: ok" in out, out
