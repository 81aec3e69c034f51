"""Binding of ``libdsa_peak.so``: measured device peaks (matrix cores, HBM)
that the benchmark reports its kernels against, next to the specification
sheet (declared in ``include/dsa_peak.h``).  Argument marshalling only."""
from __future__ import annotations

import ctypes
import os

import torch  # noqa: F401  (the HIP runtime torch loads; see the package binding)

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libdsa_peak.so")
EXPORTS = ("dsa_peak_mfma_fp8", "dsa_peak_mfma_bf16", "dsa_peak_hbm_read", "dsa_peak_hbm_copy")

if not os.path.exists(LIB_PATH):
    raise ImportError(f"{LIB_PATH} is missing: build it with `python -m sparse_attention_token_02_amd.build`")
_lib = ctypes.CDLL(LIB_PATH)
_d = ctypes.POINTER(ctypes.c_double)
_vp = ctypes.c_void_p
for _n in ("dsa_peak_mfma_fp8", "dsa_peak_mfma_bf16"):
    getattr(_lib, _n).restype = ctypes.c_int
    getattr(_lib, _n).argtypes = [ctypes.c_int, _d, _d, _vp]
_lib.dsa_peak_hbm_read.restype = ctypes.c_int
_lib.dsa_peak_hbm_read.argtypes = [_vp, ctypes.c_size_t, ctypes.c_int, _d, _vp]
_lib.dsa_peak_hbm_copy.restype = ctypes.c_int
_lib.dsa_peak_hbm_copy.argtypes = [_vp, _vp, ctypes.c_size_t, ctypes.c_int, _d, _vp]


def _stream(stream):
    return torch.cuda.current_stream().cuda_stream if stream is None else stream.cuda_stream


def _ok(rc, what):
    if rc != 0:
        raise RuntimeError(f"{what} failed with HIP error {rc}")


def mfma(dtype: str = "fp8", iters: int = 5, stream=None) -> tuple[float, float]:
    """(dense TFLOP/s, shader clock in MHz) of an MFMA-only kernel."""
    t, c = ctypes.c_double(0.0), ctypes.c_double(0.0)
    fn = _lib.dsa_peak_mfma_fp8 if dtype == "fp8" else _lib.dsa_peak_mfma_bf16
    _ok(fn(iters, ctypes.byref(t), ctypes.byref(c), _stream(stream)), f"mfma peak ({dtype})")
    return t.value, c.value


def hbm_read(buf, iters: int = 5, stream=None) -> float:
    """GB/s reading the whole contiguous device tensor `buf` once per launch."""
    g = ctypes.c_double(0.0)
    n = buf.numel() * buf.element_size() // 16 * 16
    _ok(_lib.dsa_peak_hbm_read(buf.data_ptr(), n, iters, ctypes.byref(g), _stream(stream)), "hbm read peak")
    return g.value


def hbm_copy(src, dst, iters: int = 5, stream=None) -> float:
    """GB/s (read + written bytes) copying `src` into `dst` (same byte size)."""
    g = ctypes.c_double(0.0)
    n = min(src.numel() * src.element_size(), dst.numel() * dst.element_size()) // 16 * 16
    _ok(_lib.dsa_peak_hbm_copy(src.data_ptr(), dst.data_ptr(), n, iters, ctypes.byref(g), _stream(stream)),
        "hbm copy peak")
    return g.value
