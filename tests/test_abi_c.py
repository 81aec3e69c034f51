"""The C ABI from plain C: tests/c/abi_host_check.c is compiled with gcc
against include/dsa_indexer.h and linked to the built library, then run (it
makes host-only calls, no device work)."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LIBDIR = os.path.join(ROOT, "sparse_attention_token_02_amd")


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not available")
def test_c_program_uses_the_abi(tmp_path):
    import torch  # noqa: F401  (same HIP runtime as the Python binding loads)
    exe = tmp_path / "abi_host_check"
    cmd = ["gcc", "-std=c11", "-Wall", "-Werror", "-I", os.path.join(ROOT, "include"),
           os.path.join(ROOT, "tests", "c", "abi_host_check.c"), "-L", LIBDIR, "-ldsa_indexer",
           "-Wl,-rpath," + LIBDIR, "-o", str(exe)]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    run = subprocess.run([str(exe)], capture_output=True, text=True, timeout=120)
    assert run.returncode == 0, run.stderr
    assert run.stdout.strip() == "ok"
