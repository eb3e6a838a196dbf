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


# Plausible mistakes, each re-inserted into a temporary copy of one host source: the fuzzer
# must fail on every one of them (a sanitizer report, a launch stand-in's precondition or
# one of its own properties).
MUTATIONS = {
    "ceil_div_overflows": ("api.cpp", "int64_t ceil_div(int64_t a, int64_t b) { return a / b + (a % b != 0); }",
                           "int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }"),
    "missing_index_check": ("api.cpp", "  if (!idx && D.Ktot != D.Tk) return VEDA_EINVAL;", ""),
    "dense_overlap_unchecked": ("api.cpp", "      if (overlap(dense[i], dense[j])) return VEDA_ERANGE;", "      ;"),
    "nul_accepted": ("safetensors.cpp", "          } else if (cp == 0) {", "          } else if (cp == 0xFFFFFFFF) {"),
}


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_fuzzer_catches_planted_mistakes(tmp_path, name):
    fname, old, new = MUTATIONS[name]
    sources = {f: open(os.path.join(CSRC, f)).read() for f in ("api.cpp", "safetensors.cpp", "common.h")}
    assert sources[fname].count(old) == 1, "mutation site not found"
    sources[fname] = sources[fname].replace(old, new)
    # the copies keep their relative includes: <tmp>/pkg/csrc/*.cpp -> <tmp>/include/veda.h
    csrc = tmp_path / "pkg" / "csrc"
    csrc.mkdir(parents=True)
    for f, text in sources.items():
        (csrc / f).write_text(text)
    (tmp_path / "include").mkdir()
    (tmp_path / "include" / "veda.h").write_text(open(os.path.join(ROOT, "include", "veda.h")).read())
    exe = str(tmp_path / "host_fuzz")
    flags = ["-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
             "-fno-sanitize-recover=all", "-D__HIP_PLATFORM_AMD__", "-I", str(tmp_path / "include"),
             "-isystem", os.path.join(ROCM, "include")]
    stubs = [os.path.join(ROOT, "tests", "c", "launch_stubs.cpp"), os.path.join(ROOT, "tests", "c", "host_fuzz.cpp")]
    # the stand-ins include common.h by a path relative to tests/c; point them at the copy
    for s in stubs:
        text = open(s).read().replace("../../block_sparse_attention_predictor_amd/csrc/common.h",
                                      str(csrc / "common.h")).replace("../../include/veda.h",
                                                                      str(tmp_path / "include" / "veda.h"))
        (tmp_path / os.path.basename(s)).write_text(text)
    shutil.copy(os.path.join(ROOT, "tests", "c", "launch_stubs.h"), tmp_path / "launch_stubs.h")
    r = subprocess.run(["g++", *flags, str(csrc / "api.cpp"), str(csrc / "safetensors.cpp"),
                        str(tmp_path / "launch_stubs.cpp"), str(tmp_path / "host_fuzz.cpp"), "-o", exe],
                       capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stderr[-4000:]
    files = tmp_path / "files"
    files.mkdir()
    r = subprocess.run([exe, str(files), "1", "40000", "50"], capture_output=True, text=True, timeout=300)
    assert r.returncode != 0, "the planted mistake went unnoticed:\n" + r.stdout[-2000:]
