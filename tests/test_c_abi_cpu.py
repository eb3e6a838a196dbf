"""The boundary from plain C: tests/c/abi_check.c includes only include/veda.h, is built
with gcc as strict C99 (warnings as errors) against libveda.so, and runs the host-side
entry points and the compute calls' validation failures, none of which touches a device."""
import os
import shutil
import subprocess

import pytest

from block_sparse_attention_predictor_amd import binding as Bnd

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

pytestmark = pytest.mark.skipif(not os.path.exists(Bnd.lib_path) or shutil.which("gcc") is None,
                                reason="needs libveda.so (run __graft_entry__.build()) and gcc")


def test_c99_program_links_and_passes(tmp_path):
    lib_dir = os.path.dirname(Bnd.lib_path)
    exe = str(tmp_path / "abi_check")
    build = subprocess.run(
        ["gcc", "-std=c99", "-Wall", "-Wextra", "-Werror", "-pedantic",
         "-I", os.path.join(ROOT, "include"), os.path.join(ROOT, "tests", "c", "abi_check.c"),
         "-L", lib_dir, "-lveda", f"-Wl,-rpath,{lib_dir}", "-o", exe],
        capture_output=True, text=True, timeout=120)
    assert build.returncode == 0, build.stderr
    run = subprocess.run([exe], capture_output=True, text=True, timeout=120)
    assert run.returncode == 0, run.stdout + run.stderr
    assert "FAIL" not in run.stdout and run.stdout.count(" ok ") >= 12
