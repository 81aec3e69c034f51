"""Builds the gfx950 HIP library ``libdsa_indexer.so`` in this package directory.

    python -m sparse_attention_token_02_amd.build [--jobs N]

Every translation unit is compiled with hipcc for gfx950 only; packed fp32
instructions are disabled for device code.
"""
from __future__ import annotations

import argparse
import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
OUT = os.path.join(PKG, "libdsa_indexer.so")
SOURCES = ["abi.cpp", "prefill.hip", "decode.hip", "overlap.hip", "attention.hip"]
# measured device peaks (matrix-core and HBM microbenchmarks), for the benchmark
PEAK_OUT = os.path.join(PKG, "libdsa_peak.so")
PEAK_SOURCES = ["peak.hip"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
# The decode score kernel's one-lane claims on a shared counter must stay
# single atomics whose results are read several loads later; the atomic
# optimizer would turn each into a wave reduction that is waited for at once.
PER_SOURCE = {"decode.hip": ["-mllvm", "-amdgpu-atomic-optimizer-strategy=None"]}
# roctx (per-layer ranges in the schedule drivers), from the ROCm install
ROCTX_LIBS = ("-L/opt/rocm/lib", "-lrocprofiler-sdk-roctx", "-Wl,-rpath,/opt/rocm/lib")
ARCH = "gfx950"

COMMON = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          # inputs are finite by contract: max(x, 0) needs no NaN-quieting instruction
          "-fno-honor-nans",
          "-Wno-unused-command-line-argument",
          "-I", os.path.join(ROOT, "include"), "-I", CSRC]


def _compile(src: str, obj_dir: str, extra: list[str]) -> str:
    obj = os.path.join(obj_dir, os.path.basename(src) + ".o")
    lang = ["-x", "hip"] if src.endswith(".cpp") else []
    # the host-only C-ABI layer checks caller values (a loss callback) for NaN
    host_only = ["-fhonor-nans"] if src == "abi.cpp" else []
    cmd = [HIPCC, *COMMON, *host_only, *PER_SOURCE.get(src, []), *extra, *lang, "-c", os.path.join(CSRC, src),
           "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    return obj


def _link(objs: list[str], out: str, libs: tuple[str, ...] = ()) -> str:
    tmp = out + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs, *libs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    shutil.move(tmp, out)
    return out


def build(jobs: int = 8, extra: list[str] | None = None, out: str = OUT, peak: bool = True) -> str:
    """Builds libdsa_indexer.so (to `out`) and, unless peak is False, libdsa_peak.so."""
    extra = list(extra or [])
    obj_dir = os.path.join(ROOT, "_build", "dsa_indexer")
    os.makedirs(obj_dir, exist_ok=True)
    srcs = SOURCES + (PEAK_SOURCES if peak else [])
    with ThreadPoolExecutor(max_workers=max(1, jobs)) as ex:
        objs = dict(zip(srcs, ex.map(lambda s: _compile(s, obj_dir, extra), srcs)))
    _link([objs[s] for s in SOURCES], out, ROCTX_LIBS)
    if peak:
        _link([objs[s] for s in PEAK_SOURCES], PEAK_OUT)
    return out


def main(argv=None) -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--jobs", type=int, default=min(8, os.cpu_count() or 1))
    args = ap.parse_args(argv)
    print(build(args.jobs))
    return 0


if __name__ == "__main__":
    sys.exit(main())
