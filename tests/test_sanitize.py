"""The library's host code (planner, C ABI) and the oracle built with
AddressSanitizer and UndefinedBehaviorSanitizer (g++ / gcc, host code only: the
kernel launchers and the HIP runtime are replaced by stand-ins that count and fail
any call), driven through random and invalid inputs.  Any sanitizer report fails
the test."""
import os
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(ROOT, "paged_kv_attention_ragged_amd", "csrc")
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", "-g", "-O1"]
ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0:halt_on_error=1",
           UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")


def build_and_run(tmp_path, cmd, exe, args=()):
    subprocess.check_call(cmd + ["-o", str(tmp_path / exe)])
    r = subprocess.run([str(tmp_path / exe)] + list(args), capture_output=True, text=True, env=ENV, timeout=600)
    out = r.stdout + r.stderr
    assert r.returncode == 0 and "runtime error" not in out and "AddressSanitizer" not in out, out[-4000:]
    return out


def test_planner_and_host_abi_under_sanitizers(tmp_path):
    cmd = (["g++", "-std=c++17"] + SAN + ["-D__HIP_PLATFORM_AMD__", "-I", "/opt/rocm/include",
                                          "-I", os.path.join(ROOT, "include"), "-I", CSRC,
                                          os.path.join(HERE, "sanitize", "planner_fuzz.cpp"),
                                          os.path.join(HERE, "sanitize", "hip_stubs.cpp"),
                                          os.path.join(CSRC, "rpa_schedule.cpp"), os.path.join(CSRC, "rpa_api.cpp")])
    out = build_and_run(tmp_path, cmd, "planner_fuzz", ["300"])
    assert "0 failures, 0 HIP calls" in out


def test_oracle_under_sanitizers(tmp_path):
    cmd = (["gcc", "-std=c11", "-pthread", "-ffp-contract=off"] + SAN +
           [os.path.join(HERE, "sanitize", "oracle_fuzz.c"), os.path.join(ROOT, "oracle", "rpa_oracle.c"), "-lm"])
    out = build_and_run(tmp_path, cmd, "oracle_fuzz")
    assert "0 failures" in out
