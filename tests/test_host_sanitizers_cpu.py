"""The host code of the C ABI under AddressSanitizer and UndefinedBehaviorSanitizer.

csrc/api.cpp (the argument validation of every entry point) and csrc/safetensors.cpp (the
file reader) are built with g++ -fsanitize=address,undefined (and the standard library's
own bounds assertions), host code only, and linked
with tests/c/launch_stubs.cpp in place of the kernel launchers, so no device is involved.
tests/c/host_fuzz.cpp then drives them with random and extreme layer descriptions (sizes
near the int32 and int64 limits, overlapping and out-of-range token ranges, null and
misaligned pointers, launch failures) and with well-formed, hand-written malformed and
randomly damaged safetensors files.  Besides the sanitizers' own findings it checks that
a rejected call launches nothing, that every launch receives geometry the kernels accept,
that entry points agree with veda_layer_check, and that well-formed files read back
exactly.  Any finding aborts the program (-fno-sanitize-recover=all).
"""
import os
import re
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")
CSRC = os.path.join(ROOT, "block_sparse_attention_predictor_amd", "csrc")

pytestmark = pytest.mark.skipif(
    shutil.which("g++") is None or not os.path.exists(os.path.join(ROCM, "include", "hip", "hip_runtime.h")),
    reason="needs g++ and the HIP runtime headers")


@pytest.fixture(scope="module")
def fuzz_exe(tmp_path_factory):
    exe = str(tmp_path_factory.mktemp("hostsan") / "host_fuzz")
    sources = [os.path.join(CSRC, "api.cpp"), os.path.join(CSRC, "safetensors.cpp"),
               os.path.join(ROOT, "tests", "c", "launch_stubs.cpp"), os.path.join(ROOT, "tests", "c", "host_fuzz.cpp")]
    flags = ["-std=c++17", "-O1", "-g", "-Wall", "-Wextra", "-Werror", "-fno-omit-frame-pointer",
             "-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-D_GLIBCXX_ASSERTIONS", "-D__HIP_PLATFORM_AMD__",
             "-I", os.path.join(ROOT, "include"), "-isystem", os.path.join(ROCM, "include")]
    r = subprocess.run(["g++", *flags, *sources, "-o", exe], capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stderr[-4000:]
    return exe


@pytest.mark.parametrize("seed", [1, 2, 3])
def test_host_code_under_sanitizers(fuzz_exe, tmp_path, seed):
    env = dict(os.environ)
    env["ASAN_OPTIONS"] = "detect_leaks=1:abort_on_error=1"
    env["UBSAN_OPTIONS"] = "print_stacktrace=1"
    r = subprocess.run([fuzz_exe, str(tmp_path), str(seed), "40000", "600"], capture_output=True, text=True,
                       timeout=300, env=env)
    assert r.returncode == 0, (r.stdout + r.stderr)[-4000:]
    # the run reached both halves with a real mix of accepted and rejected inputs
    m = re.search(r"layers: (\d+) valid for attention, (\d+) rejected; (\d+) launches", r.stdout)
    assert m and int(m[1]) > 10000 and int(m[2]) > 10000 and int(m[3]) > 100000, r.stdout
    m = re.search(r"damaged: (\d+) rejected, (\d+) still well formed", r.stdout)
    assert m and int(m[1]) > 300 and int(m[2]) > 10, r.stdout
    m = re.search(r"checks: (\d+)", r.stdout)
    assert m and int(m[1]) > 1000000, r.stdout
