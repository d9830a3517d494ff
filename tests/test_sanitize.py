"""The C-ABI's host-side validation under AddressSanitizer and UndefinedBehaviorSanitizer.

tests/sanitize/abi_checks.cpp drives every entry point with arguments it must reject
(null, misaligned and overlapping pointers, sizes whose products overflow, problems beyond
the kernels' limits or the decode scratch) and with empty problems. It is linked with
api.cpp compiled by g++ with -fsanitize=address,undefined (host code only) and with the
HIP objects of the library's own build. No call reaches the GPU.
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "differential_attention_causal_amd", "csrc")
BUILD = os.path.join(ROOT, "_build")
KERNELS = ["lambda.hip", "fwd_fp32.hip", "fwd_bf16.hip", "decode.hip", "bwd.hip", "append.hip",
           "gemm.hip", "scratch.hip"]


def _objects():
    objs = [os.path.join(BUILD, k + ".o") for k in KERNELS]
    if not all(os.path.exists(o) for o in objs):
        from differential_attention_causal_amd import build
        build.build()
    return objs


@pytest.mark.skipif(shutil.which("g++") is None or not os.path.isdir("/opt/rocm/include"),
                    reason="needs g++ and the ROCm headers")
def test_abi_validation_under_asan_and_ubsan(tmp_path):
    objs = _objects()
    inc = ["-I", os.path.join(ROOT, "include"), "-I", CSRC, "-I", "/opt/rocm/include",
           "-D__HIP_PLATFORM_AMD__"]
    san = ["-fsanitize=address,undefined", "-fno-sanitize-recover=undefined",
           "-fno-omit-frame-pointer"]
    api_o = str(tmp_path / "api_san.o")
    drv_o = str(tmp_path / "abi_checks.o")
    exe = str(tmp_path / "abi_checks")
    for src, obj in ((os.path.join(CSRC, "api.cpp"), api_o),
                     (os.path.join(ROOT, "tests", "sanitize", "abi_checks.cpp"), drv_o)):
        r = subprocess.run(["g++", "-std=c++17", "-O1", "-g"] + san + inc + ["-c", src, "-o", obj],
                           capture_output=True, text=True)
        assert r.returncode == 0, r.stderr
    r = subprocess.run(["g++"] + san + [drv_o, api_o] + objs +
                       ["-L/opt/rocm/lib", "-lamdhip64", "-lrocprofiler-sdk-roctx", "-Wl,-rpath,/opt/rocm/lib",
                        "-o", exe],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1", HIP_VISIBLE_DEVICES="")
    env.pop("LD_PRELOAD", None)
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=120)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "abi checks passed" in r.stdout
    assert "runtime error" not in r.stderr and "AddressSanitizer" not in r.stderr, r.stderr
