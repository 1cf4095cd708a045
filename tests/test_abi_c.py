"""The C boundary from C: tests/c_abi_check.c includes include/la.h as C99,
links libla.so and makes only calls that need no GPU (queries and calls that
fail argument validation). CPU only."""
import os
import shutil
import subprocess

import pytest

import non_causal_linear_amd as la

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_c_program_compiles_links_and_runs(tmp_path):
    cc = shutil.which("gcc") or shutil.which("cc")
    if cc is None:
        pytest.skip("no C compiler")
    if not os.path.exists(la.LIB_PATH):
        from non_causal_linear_amd import build
        build.build()
    libdir = os.path.dirname(la.LIB_PATH)
    exe = str(tmp_path / "c_abi_check")
    cmd = [cc, "-std=c99", "-Wall", "-Werror", "-I", os.path.join(ROOT, "include"),
           os.path.join(ROOT, "tests", "c_abi_check.c"), "-o", exe, libdir + "/libla.so",
           "-Wl,-rpath," + libdir, "-Wl,--allow-shlib-undefined", "-lm"]
    res = subprocess.run(cmd, capture_output=True, text=True)
    assert res.returncode == 0, res.stdout + res.stderr
    run = subprocess.run([exe], capture_output=True, text=True, timeout=120)
    assert run.returncode == 0, run.stdout + run.stderr
    assert "c abi ok" in run.stdout
