"""The C-ABI layer (abi.cpp) built for the host with AddressSanitizer and
UndefinedBehaviorSanitizer, linked against stub launchers that record calls
(tests/asan/), and driven through every entry point of include/qgemm.h:
invalid arguments return their status without a launch, valid ones reach one
launcher.  Host code only; no GPU is needed."""
import os
import shutil
import subprocess

import pytest

from conftest import ROOT

ROCM = "/opt/rocm"


@pytest.mark.skipif(shutil.which("g++") is None or not os.path.isdir(os.path.join(ROCM, "include", "hip")),
                    reason="needs g++ and the HIP headers")
def test_abi_layer_under_host_sanitizers(tmp_path):
    exe = tmp_path / "abi_driver"
    cmd = ["g++", "-std=c++17", "-g", "-O1", "-fsanitize=address,undefined", "-fno-omit-frame-pointer",
           "-fno-sanitize-recover=undefined", "-D__HIP_PLATFORM_AMD__",
           "-I", os.path.join(ROCM, "include"),
           "-I", os.path.join(ROOT, "weight_only_quantized_w4a16_amd", "csrc"),
           os.path.join(ROOT, "weight_only_quantized_w4a16_amd", "csrc", "abi.cpp"),
           os.path.join(ROOT, "tests", "asan", "stub_launchers.cpp"),
           os.path.join(ROOT, "tests", "asan", "abi_driver.cpp"),
           "-L", os.path.join(ROCM, "lib"), "-lamdhip64", "-Wl,-rpath," + os.path.join(ROCM, "lib"),
           "-o", str(exe)]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-4000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0", UBSAN_OPTIONS="print_stacktrace=1")
    r = subprocess.run([str(exe)], capture_output=True, text=True, env=env, timeout=120)
    assert r.returncode == 0, (r.stdout + r.stderr)[-4000:]
    assert "abi driver ok" in r.stdout
