"""The plan code (stft_log_mel_amd/csrc/lm_plan.cpp: argument checks,
window, twiddles, mel filterbank, blocked and lane tables) built for the host
alone under AddressSanitizer and UndefinedBehaviorSanitizer, and driven by
tests/host_sanitize/plan_driver.cpp over every transform size and option,
including invalid arguments.  Any out-of-bounds access, leak or undefined
behaviour aborts the driver.  CPU only: no GPU code is built or run."""
from __future__ import annotations

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CLANG = "/opt/rocm/llvm/bin/clang++"


def _compiler():
    for c in (CLANG, shutil.which("clang++")):
        if c and os.path.exists(c):
            return c
    return None


def test_plan_code_under_address_and_undefined_behaviour_sanitizers(tmp_path):
    cxx = _compiler()
    if cxx is None:
        pytest.skip("no clang++ for the host sanitizer build")
    exe = tmp_path / "plan_driver"
    cmd = [cxx, "-std=c++17", "-O1", "-g", "-w", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
           "-fno-omit-frame-pointer", "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include",
           "-I" + os.path.join(ROOT, "include"), "-I" + os.path.join(ROOT, "stft_log_mel_amd", "csrc"),
           "-x", "c++", os.path.join(ROOT, "stft_log_mel_amd", "csrc", "lm_plan.cpp"),
           "-x", "c++", os.path.join(ROOT, "tests", "host_sanitize", "plan_driver.cpp"), "-o", str(exe)]
    b = subprocess.run(cmd, capture_output=True, text=True, timeout=300)
    if b.returncode != 0 and ("asan" in b.stderr.lower() and "cannot find" in b.stderr.lower()):
        pytest.skip("sanitizer runtime not installed")
    assert b.returncode == 0, b.stderr[-3000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0:exitcode=23",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=300, env=env)
    assert r.returncode == 0, (r.stdout[-2000:], r.stderr[-4000:])
    assert "160 plans, 0 failed checks" in r.stdout
    assert "runtime error" not in r.stderr and "ERROR: AddressSanitizer" not in r.stderr
