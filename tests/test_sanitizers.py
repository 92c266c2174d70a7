"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only):

* the oracle (oracle/oracle.c), compiled into tests/sanitize/oracle_driver.c,
  runs every routine on inputs with the routing and encoding edge cases;
* libmxg's C ABI layer (csrc/api.cpp), linked with host-only stand-ins for
  its launchers and for the two HIP calls of the MXG_VALIDATE check
  (tests/sanitize/abi_stubs.cpp), is driven through every entry point by
  tests/sanitize/abi_driver.cpp.

Each program must exit 0 with no sanitizer report (errors abort:
-fno-sanitize-recover=all; leaks are reported by LeakSanitizer)."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = os.path.join(ROOT, "tests", "sanitize")
CSRC = os.path.join(ROOT, "fp4_grouped_gemm_quantize_amd", "csrc")
FLAGS = ["-O1", "-g", "-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer"]
HIP_INCLUDE = "/opt/rocm/include"


def run(cmd, cwd, timeout=240):
    res = subprocess.run(cmd, cwd=cwd, capture_output=True, text=True, timeout=timeout)
    return res.returncode, res.stdout + res.stderr


def check_clean(exe, tmp_path):
    rc, out = run([exe], tmp_path)
    assert rc == 0, out[-4000:]
    for marker in ("runtime error", "ERROR: AddressSanitizer", "ERROR: LeakSanitizer"):
        assert marker not in out, out[-4000:]
    return out


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not installed")
def test_oracle_under_sanitizers(tmp_path):
    exe = str(tmp_path / "oracle_driver")
    rc, out = run(["gcc", "-std=c11", *FLAGS, "-ffp-contract=off", os.path.join(SAN, "oracle_driver.c"), "-o", exe,
                   "-lm"], tmp_path)
    assert rc == 0, out
    assert "fails 0" in check_clean(exe, tmp_path)


@pytest.mark.skipif(shutil.which("g++") is None or not os.path.isdir(HIP_INCLUDE),
                    reason="g++ or the HIP headers not installed")
def test_abi_layer_under_sanitizers(tmp_path):
    exe = str(tmp_path / "abi_driver")
    rc, out = run(["g++", "-std=c++17", *FLAGS, "-D__HIP_PLATFORM_AMD__", "-I", HIP_INCLUDE, "-I",
                   os.path.join(ROOT, "include"), "-I", CSRC, "-I", SAN, os.path.join(CSRC, "api.cpp"),
                   os.path.join(SAN, "abi_stubs.cpp"), os.path.join(SAN, "abi_driver.cpp"), "-o", exe], tmp_path)
    assert rc == 0, out
    assert "fails 0" in check_clean(exe, tmp_path)
