"""Device-side builder of the seeded synthetic inputs (same bytes as synth.gen).

Large workloads (hundreds of MB to GB of fp8 queries) are generated on the GPU
by ``libdsa_synth.so``; ``synth.gen`` rebuilds any subset of rows on the host
for the oracle, and the tests check that both agree bit for bit.
"""
from __future__ import annotations

import ctypes
import os
import shutil
import subprocess

import numpy as np

from . import gen

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libdsa_synth.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")


def build() -> str:
    src = os.path.join(_HERE, "csrc", "synth_gen.hip")
    tmp = LIB_PATH + ".tmp"
    cmd = [HIPCC, "-O3", "-std=c++17", "-fPIC", "-shared", "--offload-arch=gfx950",
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
           "-ffp-contract=off", "-Wno-unused-command-line-argument", src, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"synth build failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    shutil.move(tmp, LIB_PATH)
    return LIB_PATH


_lib = None


def _load():
    global _lib
    if _lib is None:
        import torch  # noqa: F401  (bind to torch's HIP runtime, see the package binding)
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} missing: run synth.gpu.build()")
        lib = ctypes.CDLL(LIB_PATH)
        vp, i32, i64, f32 = ctypes.c_void_p, ctypes.c_int, ctypes.c_longlong, ctypes.c_float
        lib.synth_gen_rows.restype = i32
        lib.synth_gen_rows.argtypes = [vp, i32, i64, i32, i32, vp, f32, f32, f32, vp, vp, vp]
        lib.synth_quant_rows_e4m3.restype = i32
        lib.synth_quant_rows_e4m3.argtypes = [vp, i32, i32, vp, vp, vp]
        lib.synth_bf16.restype = i32
        lib.synth_bf16.argtypes = [vp, i64, vp, vp]
        _lib = lib
    return _lib


class DeviceGen:
    """Generator state on one device (the normal table)."""

    def __init__(self, device="cuda"):
        import torch
        self.torch = torch
        self.device = torch.device(device)
        self.table = torch.from_numpy(gen.NORMAL_TABLE.copy()).to(self.device)
        self.lib = _load()

    def _stream(self):
        return self.torch.cuda.current_stream(self.device).cuda_stream

    def rows_f32(self, seed, name, nrows, ncols, *, row0=0, layers=0, rho=0.0, sigma=0.0, div=0.0, mult=None):
        """float32 [nrows, ncols] of stream ``name`` (layer recurrence if layers > 0)."""
        torch = self.torch
        bases = np.array([gen.stream_base(seed, gen.STREAM[name] * 1024 + l) for l in range(layers + 1)],
                         dtype=np.uint64)
        bd = torch.from_numpy(bases.view(np.int64)).to(self.device)
        out = torch.empty((nrows, ncols), dtype=torch.float32, device=self.device)
        m = None if mult is None else mult.contiguous()
        rc = self.lib.synth_gen_rows(bd.data_ptr(), layers, row0, nrows, ncols, self.table.data_ptr(),
                                     float(rho), float(sigma), float(div),
                                     None if m is None else m.data_ptr(), out.data_ptr(), self._stream())
        if rc:
            raise RuntimeError(f"synth_gen_rows failed ({rc})")
        return out

    def quant_e4m3(self, X):
        torch = self.torch
        R = X.shape[0]
        C = X.numel() // R
        codes = torch.empty(X.shape, dtype=torch.uint8, device=self.device)
        scales = torch.empty(R, dtype=torch.float32, device=self.device)
        rc = self.lib.synth_quant_rows_e4m3(X.data_ptr(), R, C, codes.data_ptr(), scales.data_ptr(), self._stream())
        if rc:
            raise RuntimeError(f"synth_quant_rows_e4m3 failed ({rc})")
        return codes, scales

    def bf16(self, X):
        torch = self.torch
        out = torch.empty(X.shape, dtype=torch.int16, device=self.device)
        rc = self.lib.synth_bf16(X.data_ptr(), X.numel(), out.data_ptr(), self._stream())
        if rc:
            raise RuntimeError(f"synth_bf16 failed ({rc})")
        return out

    # ---- workloads -------------------------------------------------------

    def prefill_inputs(self, cfg: dict) -> dict:
        """Device tensors of a prefill workload: q [L,H,D] (uint8 e4m3 or int16 bf16
        bits), q_scale [L] or None, k [L,D], k_scale [L] or None, w [L,H] int16 bf16 bits."""
        torch = self.torch
        L, H, D, seed = cfg["L"], cfg["H"], cfg["D"], cfg["seed"]
        heavy = gen.heavy_positions(seed, L, cfg.get("heavy_count", 0))
        mult = None
        if len(heavy):
            m = np.ones(L, dtype=np.float32)
            m[heavy] = np.float32(cfg["heavy_factor"])
            mult = torch.from_numpy(m).to(self.device)
        fp8 = cfg["dtype"] == "fp8"
        kdiv = 0.0 if fp8 else cfg["qk_div"]
        K = self.rows_f32(seed, "k", L, D, div=kdiv, mult=mult)
        out = {"heavy": heavy}
        if fp8:
            out["k"], out["k_scale"] = self.quant_e4m3(K)
        else:
            out["k"], out["k_scale"] = self.bf16(K), None
        del K
        # queries in row chunks to bound the float32 staging buffer
        if fp8:
            q = torch.empty((L, H, D), dtype=torch.uint8, device=self.device)
            qs = torch.empty(L, dtype=torch.float32, device=self.device)
        else:
            q = torch.empty((L, H, D), dtype=torch.int16, device=self.device)
            qs = None
        chunk = max(1, (1 << 27) // (H * D))
        for r0 in range(0, L, chunk):
            n = min(chunk, L - r0)
            Q = self.rows_f32(seed, "q", n, H * D, row0=r0, div=kdiv)
            if fp8:
                c, s = self.quant_e4m3(Q)
                q[r0:r0 + n] = c.view(n, H, D)
                qs[r0:r0 + n] = s
            else:
                q[r0:r0 + n] = self.bf16(Q).view(n, H, D)
            del Q
        out["q"], out["q_scale"] = q, qs
        W = self.rows_f32(seed, "w", L, H, div=cfg["w_div"])
        out["w"] = self.bf16(W)
        return out

    def decode_inputs(self, cfg: dict) -> dict:
        torch = self.torch
        B, Lmax, H, D, seed = cfg["B"], cfg["Lmax"], cfg["H"], cfg["D"], cfg["seed"]
        cache = torch.empty((B, Lmax, D), dtype=torch.uint8, device=self.device)
        ks = torch.empty((B, Lmax), dtype=torch.float32, device=self.device)
        for b in range(B):
            K = self.rows_f32(seed, "k", Lmax, D, row0=b * Lmax)
            c, s = self.quant_e4m3(K)
            cache[b] = c
            ks[b] = s
            del K
        q = self.bf16(self.rows_f32(seed, "q", B, H * D)).view(B, H, D)
        w = self.bf16(self.rows_f32(seed, "w", B, H, div=cfg["w_div"]))
        lens = torch.from_numpy(gen.decode_lens(cfg)).to(self.device)
        return {"cache": cache, "k_scale": ks, "q": q, "w": w, "lens": lens}

    def fs_layer_inputs(self, cfg: dict, layer: int) -> dict:
        torch = self.torch
        L, H, D, seed = cfg["L"], cfg["H"], cfg["D"], cfg["seed"]
        rs = dict(layers=layer, rho=cfg["rho"], sigma=cfg["sigma"])
        K = self.rows_f32(seed, "k", L, D, **rs)
        k, k_scale = self.quant_e4m3(K)
        del K
        q = torch.empty((L, H, D), dtype=torch.uint8, device=self.device)
        qs = torch.empty(L, dtype=torch.float32, device=self.device)
        chunk = max(1, (1 << 27) // (H * D))
        for r0 in range(0, L, chunk):
            n = min(chunk, L - r0)
            Q = self.rows_f32(seed, "q", n, H * D, row0=r0, **rs)
            c, s = self.quant_e4m3(Q)
            q[r0:r0 + n] = c.view(n, H, D)
            qs[r0:r0 + n] = s
            del Q
        W = self.rows_f32(seed, "w", L, H, div=cfg["w_div"], **rs)
        return {"q": q, "q_scale": qs, "k": k, "k_scale": k_scale, "w": self.bf16(W)}

    def fs_decode_layer_inputs(self, cfg: dict, layer: int) -> dict:
        torch = self.torch
        B, Lmax, H, D, seed = cfg["B"], cfg["Lmax"], cfg["H"], cfg["D"], cfg["seed"]
        rs = dict(layers=layer, rho=cfg["rho"], sigma=cfg["sigma"])
        cache = torch.empty((B, Lmax, D), dtype=torch.uint8, device=self.device)
        ks = torch.empty((B, Lmax), dtype=torch.float32, device=self.device)
        for b in range(B):
            K = self.rows_f32(seed, "k", Lmax, D, row0=b * Lmax, **rs)
            c, s = self.quant_e4m3(K)
            cache[b] = c
            ks[b] = s
            del K
        q = self.bf16(self.rows_f32(seed, "q", B, H * D, **rs)).view(B, H, D)
        w = self.bf16(self.rows_f32(seed, "w", B, H, div=cfg["w_div"], **rs))
        lens = torch.from_numpy(gen.decode_lens(cfg)).to(self.device)
        return {"cache": cache, "k_scale": ks, "q": q, "w": w, "lens": lens}

    def standin_latent(self, seed: int, which: int, B: int, Lmax: int):
        torch = self.torch
        out = torch.empty((B, Lmax, 576), dtype=torch.int16, device=self.device)
        for b in range(B):
            X = self.rows_f32(seed, "latent", Lmax, 576, row0=b * Lmax, layers=which, rho=0.0, sigma=1.0, div=4.0)
            out[b] = self.bf16(X)
            del X
        return out

    def standin_query(self, seed: int, layer: int, B: int):
        return self.bf16(self.rows_f32(seed, "qa", B, 576, layers=layer, rho=0.0, sigma=1.0, div=4.0))
