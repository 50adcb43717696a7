"""The C ABI's argument validation under AddressSanitizer and UndefinedBehaviorSanitizer,
on the host: capi.cpp and the attention split plan (attn_plan.cpp) built with g++ and
linked against stub launchers (tests/capi_host_check.cpp) that only record calls. Every
entry point runs with valid arguments, with one bad argument at a time and with sizes
near the int limits; the program exits non-zero on a wrong status, an unexpected launch
or any sanitizer report. No GPU needed."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "block_sparse_long_spot_amd", "csrc")


@pytest.mark.skipif(shutil.which("g++") is None, reason="needs g++")
def test_capi_validation_under_sanitizers(tmp_path):
    exe = str(tmp_path / "capi_host_check")
    cmd = ["g++", "-std=c++17", "-g", "-O1", "-fno-omit-frame-pointer",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
           "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include", f"-I{os.path.join(ROOT, 'include')}",
           f"-I{CSRC}", os.path.join(ROOT, "tests", "capi_host_check.cpp"),
           os.path.join(CSRC, "capi.cpp"), os.path.join(CSRC, "attn_plan.cpp"), "-o", exe]
    b = subprocess.run(cmd, capture_output=True, text=True, timeout=300)
    assert b.returncode == 0, b.stderr[-4000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1")
    r = subprocess.run([exe], capture_output=True, text=True, timeout=120, env=env)
    assert r.returncode == 0, (r.stdout + r.stderr)[-4000:]
    assert "passed: 0 failure(s)" in r.stdout
