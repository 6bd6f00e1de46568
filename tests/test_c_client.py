"""The boundary from C: a C99 program (tests/c/abi_client.c) includes the
public headers with warnings as errors, links libaxr.so and exercises the
host-side calls (codebook, validation before any device call)."""

import os
import shutil
import subprocess

import pytest

import lut_attention_scoring_amd as axr

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_c99_client(tmp_path):
    cc = shutil.which("gcc") or shutil.which("cc")
    if cc is None:
        pytest.skip("no C compiler")
    libdir = os.path.dirname(axr.LIB_PATH)
    exe = tmp_path / "abi_client"
    cmd = [cc, "-std=c99", "-Wall", "-Wextra", "-Werror", "-I", os.path.join(ROOT, "include"),
           os.path.join(ROOT, "tests", "c", "abi_client.c"), "-L", libdir, "-laxr",
           f"-Wl,-rpath,{libdir}", "-lm", "-o", str(exe)]
    build = subprocess.run(cmd, capture_output=True, text=True, timeout=300)
    assert build.returncode == 0, build.stderr
    run = subprocess.run([str(exe)], capture_output=True, text=True, timeout=300)
    lines = run.stdout.strip().splitlines()
    assert run.returncode == 0, run.stdout + run.stderr
    assert len(lines) == 9 and all(l.startswith("ok ") for l in lines), run.stdout
