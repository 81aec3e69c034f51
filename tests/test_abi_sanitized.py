"""The host side of the C ABI under AddressSanitizer and UndefinedBehavior-
Sanitizer, with the workspace layout checks compiled in (DSA_DEBUG_BOUNDS).
abi.cpp is rebuilt with the sanitizers on its host code only (hipcc
-Xarch_host), linked with the library's other (unsanitized) objects, and
tests/c/abi_host_check.c, compiled with clang and the same sanitizers, runs
against it: host-only calls, no device work.  CPU only."""
import glob
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "sparse_attention_token_02_amd", "csrc")
OBJDIR = os.path.join(ROOT, "_build", "dsa_indexer")
HIPCC = "/opt/rocm/bin/hipcc"
CLANG = "/opt/rocm/llvm/bin/clang"
SAN = ["address", "undefined"]


def _host_san_flags():
    flags = []
    for s in SAN:
        flags += ["-Xarch_host", f"-fsanitize={s}"]
    return flags + ["-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer"]


@pytest.mark.skipif(not (os.path.exists(HIPCC) and os.path.exists(CLANG)), reason="ROCm compilers not available")
def test_c_abi_host_paths_under_asan_and_ubsan(tmp_path):
    objs = [os.path.join(OBJDIR, f"{n}.hip.o") for n in ("prefill", "decode", "overlap", "attention")]
    if not all(os.path.exists(o) for o in objs):
        pytest.skip("library objects not built (run the package build first)")
    abi_o = tmp_path / "abi_san.o"
    cmd = [HIPCC, "-O1", "-g", "-std=c++17", "-fPIC", "--offload-arch=gfx950", "-x", "hip",
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", "-DDSA_DEBUG_BOUNDS",
           "-Wno-unused-command-line-argument", *_host_san_flags(),
           "-I", os.path.join(ROOT, "include"), "-I", CSRC, "-c", os.path.join(CSRC, "abi.cpp"), "-o", str(abi_o)]
    r = subprocess.run(cmd, capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, r.stderr[-3000:]
    lib = tmp_path / "libdsa_indexer.so"
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", str(lib), str(abi_o), *objs,
           "-L/opt/rocm/lib", "-lrocprofiler-sdk-roctx", "-Wl,-rpath,/opt/rocm/lib"]
    r = subprocess.run(cmd, capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, r.stderr[-3000:]
    exe = tmp_path / "abi_host_check_san"
    cmd = [CLANG, "-std=c11", "-g", "-O1", "-Wall", "-Werror", *[f"-fsanitize={s}" for s in SAN],
           "-fno-sanitize-recover=undefined", "-I", os.path.join(ROOT, "include"),
           os.path.join(ROOT, "tests", "c", "abi_host_check.c"), "-L", str(tmp_path), "-ldsa_indexer",
           "-Wl,-rpath," + str(tmp_path), "-o", str(exe)]
    r = subprocess.run(cmd, capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stderr[-3000:]
    env = dict(os.environ)
    # the HIP runtime's own allocations outlive main(); leaks are not what this checks
    env["ASAN_OPTIONS"] = "detect_leaks=0:halt_on_error=1:abort_on_error=0"
    env["UBSAN_OPTIONS"] = "halt_on_error=1:print_stacktrace=1"
    run = subprocess.run([str(exe)], capture_output=True, text=True, timeout=300, env=env)
    assert run.returncode == 0, (run.stdout[-2000:], run.stderr[-4000:])
    assert run.stdout.strip() == "ok"
    assert "runtime error" not in run.stderr and "AddressSanitizer" not in run.stderr, run.stderr[-4000:]
