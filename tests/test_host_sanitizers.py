"""The host-only half of the C ABI built with the address and undefined-behaviour sanitizers.

csrc/host.cpp (argument validation, the static mask generators, the index bookkeeping) has no
device code, so it is compiled here with the host compiler, instrumented, and driven by
tests/host/host_check.cpp over valid and invalid arguments with edge values.  No GPU is needed.
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "sparse_attention_diffusion_block_amd", "csrc")
ROCM_INCLUDE = "/opt/rocm/include"


@pytest.mark.skipif(shutil.which("g++") is None or not os.path.isdir(ROCM_INCLUDE),
                    reason="needs g++ and the HIP runtime headers")
def test_host_code_under_asan_and_ubsan(tmp_path):
    exe = tmp_path / "host_check"
    sanitize = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer"]
    cmd = ["g++", "-std=c++17", "-O1", "-g", *sanitize, "-D__HIP_PLATFORM_AMD__", f"-I{ROCM_INCLUDE}", f"-I{CSRC}",
           os.path.join(CSRC, "host.cpp"), os.path.join(ROOT, "tests", "host", "host_check.cpp"), "-o", str(exe)]
    build = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    assert build.returncode == 0, build.stdout
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0", UBSAN_OPTIONS="print_stacktrace=1")
    run = subprocess.run([str(exe)], stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True, env=env, timeout=300)
    assert run.returncode == 0, run.stdout
    assert "host checks passed" in run.stdout
