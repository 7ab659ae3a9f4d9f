"""AddressSanitizer and UndefinedBehaviorSanitizer run on the CPU.

tests/sanitize/driver.cpp is compiled with g++ / gcc (host code only; no
GPU code is built here) together with the C ABI's host code
(quantized_recurrent_state_amd/csrc/leapq_abi.cpp, its kernel launchers
replaced by tests/sanitize/launch_stubs.cpp, which launch nothing) and the
oracle (oracle/leapq_oracle.c), all under -fsanitize=address,undefined with
recovery off.  The driver takes every entry point through valid and invalid
arguments and every oracle routine through two windows of small inputs; the
test passes when it exits 0 with no sanitizer report.
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", "-g", "-O1"]


@pytest.mark.skipif(shutil.which("g++") is None or shutil.which("gcc") is None, reason="needs gcc and g++")
def test_abi_and_oracle_under_asan_ubsan(tmp_path):
    csrc = os.path.join(ROOT, "quantized_recurrent_state_amd", "csrc")
    inc = ["-I" + os.path.join(ROOT, "include"), "-I" + csrc, "-I/opt/rocm/include", "-D__HIP_PLATFORM_AMD__"]
    objs = []
    units = [("g++", os.path.join(csrc, "leapq_abi.cpp"), ["-std=c++17"]),
             ("g++", os.path.join(ROOT, "tests", "sanitize", "launch_stubs.cpp"), ["-std=c++17"]),
             ("g++", os.path.join(ROOT, "tests", "sanitize", "driver.cpp"), ["-std=c++17"]),
             ("gcc", os.path.join(ROOT, "oracle", "leapq_oracle.c"), ["-std=c11", "-ffp-contract=off"])]
    for cc, src, extra in units:
        obj = os.path.join(tmp_path, os.path.basename(src) + ".o")
        r = subprocess.run([cc, *SAN, *extra, *inc, "-c", src, "-o", obj], capture_output=True, text=True)
        assert r.returncode == 0, r.stderr[-3000:]
        objs.append(obj)
    exe = os.path.join(tmp_path, "driver")
    r = subprocess.run(["g++", *SAN, *objs, "-o", exe, "-lm"], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-3000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0", UBSAN_OPTIONS="print_stacktrace=1")
    env.pop("LD_PRELOAD", None)
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=600)
    out = r.stdout + r.stderr
    print(out[-2000:])
    assert r.returncode == 0, out[-4000:]
    assert "AddressSanitizer" not in out and "runtime error" not in out, out[-4000:]
    assert "0 failed checks" in out
