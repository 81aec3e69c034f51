"""Host (numpy) implementation of the seeded synthetic inputs.

Generator
---------
Every random number comes from SplitMix64 (Steele, Lea and Flood, "Fast
splittable pseudorandom number generators", OOPSLA 2014) used as a counter
based generator: element ``i`` of stream ``(seed, stream)`` is the ``i``-th
output of a SplitMix64 sequence whose state starts at
``mix64(seed * 2**32 + stream)``.  Any element can be produced on its own, so
the host can rebuild exactly the rows an oracle check needs while the device
builds the whole tensor (``synth.gpu``) and both agree bit for bit.

A standard normal draw is ``NORMAL_TABLE[h >> 48]``: the top 16 bits of the
hash pick one of 65536 equiprobable levels, the level value being the normal
quantile at the level's midpoint ((i + 0.5) / 65536).  Only table lookups,
IEEE-rounded float32 multiplies/adds/divides and integer bit operations follow,
so the host and the device produce identical bytes.

Formats
-------
* bf16: round-to-nearest-even of the float32 bit pattern.
* e4m3: OCP 8-bit floating point E4M3 ("e4m3fn": bias 7, no infinities,
  largest finite 448, S.1111.111 is NaN), round-to-nearest-even, saturating
  to +-448.  Per-token scale = amax / 448 in float32 (1 when amax is 0) and
  code = e4m3(x / scale).
"""
from __future__ import annotations

import math
from statistics import NormalDist

import numpy as np

__all__ = [
    "GAMMA", "mix64_int", "stream_base", "hash_u64", "NORMAL_TABLE", "normal_f32",
    "uniform_int", "bf16_bits", "e4m3_bits", "quant_rows_e4m3", "heavy_positions",
    "STREAM", "CONFIGS", "prefill_inputs", "decode_inputs", "fs_layer_inputs", "fs_decode_layer_inputs",
    "standin_latent", "standin_query",
    "fs_noise_rows", "decode_lens", "FS_PATTERNS", "ragged_decode_config",
]

MASK64 = (1 << 64) - 1
GAMMA = 0x9E3779B97F4A7C15
_M1 = 0xBF58476D1CE4E5B9
_M2 = 0x94D049BB133111EB


def mix64_int(z: int) -> int:
    """SplitMix64 output function on a Python int (mod 2**64)."""
    z &= MASK64
    z = ((z ^ (z >> 30)) * _M1) & MASK64
    z = ((z ^ (z >> 27)) * _M2) & MASK64
    return z ^ (z >> 31)


def stream_base(seed: int, stream: int) -> int:
    """Start state of stream ``stream`` under ``seed`` (both < 2**32)."""
    if not (0 <= seed < 2**32 and 0 <= stream < 2**32):
        raise ValueError("seed and stream must fit in 32 bits")
    return mix64_int((seed << 32) | stream)


def hash_u64(seed: int, stream: int, idx) -> np.ndarray:
    """64-bit hash of element(s) ``idx`` (uint64 array) of a stream."""
    idx = np.asarray(idx, dtype=np.uint64)
    with np.errstate(over="ignore"):
        z = np.uint64(stream_base(seed, stream)) + (idx + np.uint64(1)) * np.uint64(GAMMA)
        z = (z ^ (z >> np.uint64(30))) * np.uint64(_M1)
        z = (z ^ (z >> np.uint64(27))) * np.uint64(_M2)
        z = z ^ (z >> np.uint64(31))
    return z


def _normal_table() -> np.ndarray:
    nd = NormalDist()
    return np.array([nd.inv_cdf((i + 0.5) / 65536.0) for i in range(65536)], dtype=np.float32)


NORMAL_TABLE = _normal_table()


def normal_f32(seed: int, stream: int, idx) -> np.ndarray:
    """Standard-normal draws (float32) for elements ``idx`` of a stream."""
    h = hash_u64(seed, stream, idx)
    return NORMAL_TABLE[(h >> np.uint64(48)).astype(np.int64)]


def uniform_int(seed: int, stream: int, idx, lo: int, hi: int) -> np.ndarray:
    """Integers uniform on [lo, hi] (inclusive) for elements ``idx``."""
    span = hi - lo + 1
    if not (0 < span <= 2**31):
        raise ValueError("bad range")
    h = hash_u64(seed, stream, idx) >> np.uint64(32)
    return (lo + ((h * np.uint64(span)) >> np.uint64(32)).astype(np.int64)).astype(np.int64)


def bf16_bits(x) -> np.ndarray:
    """float32 -> bf16 bit pattern (uint16), round to nearest even.  Finite input."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    r = (u + np.uint64(0x7FFF) + ((u >> np.uint64(16)) & np.uint64(1))) >> np.uint64(16)
    return r.astype(np.uint16)


def e4m3_bits(x) -> np.ndarray:
    """float32 -> OCP e4m3fn code (uint8), round to nearest even, saturating."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.int64)
    sign = ((u >> 31) & 1) << 7
    a = u & 0x7FFFFFFF
    # normal range |x| >= 2**-6: keep 3 mantissa bits, round at bit 20
    r = a + 0x7FFFF + ((a >> 20) & 1)
    e = (r >> 23) - 127
    m = (r >> 20) & 7
    sat = (e > 8) | ((e == 8) & (m == 7))
    code_n = np.where(sat, 0x7E, ((e + 7) << 3) | m)
    # below 2**-6: multiples of 2**-9, scaling by 512 is exact in float32
    mag = (a.astype(np.uint32)).view(np.float32) * np.float32(512.0)
    code_s = np.rint(mag).astype(np.int64)
    code = np.where(a >= 0x3C800000, code_n, code_s)
    return (code | sign).astype(np.uint8)


def quant_rows_e4m3(X) -> tuple[np.ndarray, np.ndarray]:
    """Per-row e4m3 quantisation: returns (codes uint8 like X, scale float32 [rows])."""
    X = np.asarray(X, dtype=np.float32)
    X2 = X.reshape(X.shape[0], -1)
    amax = np.max(np.abs(X2), axis=1)
    scale = np.where(amax > 0, amax / np.float32(448.0), np.float32(1.0)).astype(np.float32)
    codes = e4m3_bits((X2 / scale[:, None]).astype(np.float32))
    return codes.reshape(X.shape), scale


# ----------------------------------------------------------------------------
# Workload recipes
# ----------------------------------------------------------------------------

# Stream ids: tensor id * 1024 + layer (the layer is 0 outside the layer-reuse workload).
STREAM = {"q": 1, "k": 2, "w": 3, "heavy": 4, "lens": 5, "latent": 6, "qa": 7}


def _sid(name: str, layer: int = 0) -> int:
    return STREAM[name] * 1024 + layer


def heavy_positions(seed: int, L: int, count: int) -> np.ndarray:
    """``count`` distinct key positions uniform over [0, L): the keys with the
    smallest hashes (position breaks hash ties).  Sorted ascending."""
    if count <= 0:
        return np.zeros(0, dtype=np.int64)
    h = hash_u64(seed, _sid("heavy"), np.arange(L, dtype=np.uint64))
    order = np.lexsort((np.arange(L), h))
    return np.sort(order[:count]).astype(np.int64)


_F32 = np.float32

CONFIGS = {
    # L=2048 single-layer bf16 prefill with 16 planted 4x keys
    "tiny": dict(kind="prefill", L=2048, H=8, D=64, topk=128, dtype="bf16", seed=0,
                 heavy_count=16, heavy_factor=4.0, qk_div=8.0, w_div=float(_F32(math.sqrt(8.0)))),
    # L=32768 fp8 prefill, 1% heavy keys at 3x
    "prefill_32k": dict(kind="prefill", L=32768, H=64, D=128, topk=2048, dtype="fp8", seed=0,
                        heavy_count=round(0.01 * 32768), heavy_factor=3.0, w_div=8.0),
    # batch of 32 decode queries over 131072-token fp8 caches
    "decode_128k": dict(kind="decode", B=32, Lmax=131072, H=64, D=128, topk=2048, seed=0,
                        ragged=False, w_div=8.0),
    # 47-layer reuse schedule at L=65536, correlated layers
    "fs_47": dict(kind="fs", N=47, L=65536, H=64, D=128, topk=2048, dtype="fp8", seed=0,
                  rho=0.9, sigma=0.44, w_div=8.0),
    # one decode step through 47 correlated layers, 32 sequences x 131072 cached tokens
    "fs_decode_47": dict(kind="fs_decode", N=47, B=32, Lmax=131072, H=64, D=128, topk=2048, seed=0,
                         ragged=False, rho=0.9, sigma=0.44, w_div=8.0),
    # L=196608 fp8 prefill, 1% heavy keys at 3x
    "prefill_196k": dict(kind="prefill", L=196608, H=64, D=128, topk=2048, dtype="fp8", seed=0,
                         heavy_count=round(0.01 * 196608), heavy_factor=3.0, w_div=8.0),
}


def ragged_decode_config(base: str = "decode_128k") -> dict:
    c = dict(CONFIGS[base])
    c["ragged"] = True
    return c


FS_PATTERNS = {
    "all_F": "F" * 47,
    "uniform_1_4": "".join("F" if l % 4 == 0 else "S" for l in range(47)),
    "searched_1_4": "FSFSFSSSSFSSSFSSFFSSFSSFSSSSFSSSFSSSSFSSSSSSSSS",
}


def _rows(rows, L):
    if rows is None:
        return np.arange(L, dtype=np.int64)
    return np.asarray(rows, dtype=np.int64)


def prefill_inputs(cfg: dict, rows=None, with_keys: bool = True) -> dict:
    """Host-side prefill inputs.  ``rows`` selects which query rows to build
    (all by default); keys are always built whole when ``with_keys``.

    Returns numpy arrays: ``k`` [L,D] (uint8 e4m3 codes or uint16 bf16 bits),
    ``k_scale`` [L] float32 (fp8 only), ``q`` [R,H,D], ``q_scale`` [R] float32
    (fp8 only; one scale per token shared by all heads), ``w`` [R,H] uint16
    bf16 bits, ``rows`` [R], ``heavy`` positions.
    """
    L, H, D, seed = cfg["L"], cfg["H"], cfg["D"], cfg["seed"]
    rows = _rows(rows, L)
    out = {"rows": rows}
    heavy = heavy_positions(seed, L, cfg.get("heavy_count", 0))
    out["heavy"] = heavy
    if with_keys:
        K = normal_f32(seed, _sid("k"), np.arange(L * D, dtype=np.uint64)).reshape(L, D)
        if cfg["dtype"] == "bf16":
            K = (K / _F32(cfg["qk_div"])).astype(np.float32)
        if len(heavy):
            K[heavy] = (K[heavy] * _F32(cfg["heavy_factor"])).astype(np.float32)
        if cfg["dtype"] == "fp8":
            out["k"], out["k_scale"] = quant_rows_e4m3(K)
        else:
            out["k"], out["k_scale"] = bf16_bits(K), None
    qidx = (rows[:, None].astype(np.uint64) * np.uint64(H * D)
            + np.arange(H * D, dtype=np.uint64)[None, :])
    Q = normal_f32(seed, _sid("q"), qidx).reshape(len(rows), H, D)
    if cfg["dtype"] == "fp8":
        out["q"], out["q_scale"] = quant_rows_e4m3(Q)
    else:
        out["q"], out["q_scale"] = bf16_bits((Q / _F32(cfg["qk_div"])).astype(np.float32)), None
    widx = rows[:, None].astype(np.uint64) * np.uint64(H) + np.arange(H, dtype=np.uint64)[None, :]
    W = normal_f32(seed, _sid("w"), widx) / _F32(cfg["w_div"])
    out["w"] = bf16_bits(W.astype(np.float32))
    return out


def decode_lens(cfg: dict) -> np.ndarray:
    B, Lmax = cfg["B"], cfg["Lmax"]
    if not cfg.get("ragged"):
        return np.full(B, Lmax, dtype=np.int32)
    lo = Lmax // 2
    return uniform_int(cfg["seed"], _sid("lens"), np.arange(B, dtype=np.uint64), lo, Lmax).astype(np.int32)


def decode_inputs(cfg: dict, seqs=None) -> dict:
    """Host-side decode inputs for sequences ``seqs`` (all by default).

    ``cache`` [S,Lmax,D] uint8 e4m3 codes, ``k_scale`` [S,Lmax] float32 (one
    scale per cached token), ``q`` [S,H,D] uint16 bf16 bits, ``w`` [S,H]
    uint16 bf16 bits, ``lens`` [S] int32, ``seqs`` [S].
    """
    B, Lmax, H, D, seed = cfg["B"], cfg["Lmax"], cfg["H"], cfg["D"], cfg["seed"]
    seqs = np.arange(B, dtype=np.int64) if seqs is None else np.asarray(seqs, dtype=np.int64)
    lens = decode_lens(cfg)[seqs]
    S = len(seqs)
    cache = np.empty((S, Lmax, D), dtype=np.uint8)
    kscale = np.empty((S, Lmax), dtype=np.float32)
    for i, b in enumerate(seqs):
        idx = np.uint64(int(b) * Lmax * D) + np.arange(Lmax * D, dtype=np.uint64)
        K = normal_f32(seed, _sid("k"), idx).reshape(Lmax, D)
        cache[i], kscale[i] = quant_rows_e4m3(K)
    qidx = seqs[:, None].astype(np.uint64) * np.uint64(H * D) + np.arange(H * D, dtype=np.uint64)[None, :]
    q = bf16_bits(normal_f32(seed, _sid("q"), qidx)).reshape(S, H, D)
    widx = seqs[:, None].astype(np.uint64) * np.uint64(H) + np.arange(H, dtype=np.uint64)[None, :]
    w = bf16_bits((normal_f32(seed, _sid("w"), widx) / _F32(cfg["w_div"])).astype(np.float32))
    return {"cache": cache, "k_scale": kscale, "q": q, "w": w, "lens": lens, "seqs": seqs}


def fs_noise_rows(cfg: dict, name: str, layer: int, rows, ncols: int) -> np.ndarray:
    """Layer ``layer`` of the correlated recurrence X_0 = N_0,
    X_l = rho*X_{l-1} + sigma*N_l (float32, each product and the sum rounded),
    evaluated for ``rows`` of a [*, ncols] tensor."""
    rows = np.asarray(rows, dtype=np.int64)
    idx = rows[:, None].astype(np.uint64) * np.uint64(ncols) + np.arange(ncols, dtype=np.uint64)[None, :]
    rho, sigma = _F32(cfg["rho"]), _F32(cfg["sigma"])
    X = normal_f32(cfg["seed"], _sid(name, 0), idx)
    for l in range(1, layer + 1):
        N = normal_f32(cfg["seed"], _sid(name, l), idx)
        X = ((rho * X).astype(np.float32) + (sigma * N).astype(np.float32)).astype(np.float32)
    return X


def fs_layer_inputs(cfg: dict, layer: int, rows=None, with_keys: bool = True) -> dict:
    """Host-side inputs of one layer of the layer-reuse workload (fp8 q/k with
    per-token scales, bf16 w; q, k and w all follow the recurrence, no heavy keys)."""
    L, H, D = cfg["L"], cfg["H"], cfg["D"]
    rows = _rows(rows, L)
    out = {"rows": rows}
    if with_keys:
        K = fs_noise_rows(cfg, "k", layer, np.arange(L), D)
        out["k"], out["k_scale"] = quant_rows_e4m3(K)
    Q = fs_noise_rows(cfg, "q", layer, rows, H * D).reshape(len(rows), H, D)
    out["q"], out["q_scale"] = quant_rows_e4m3(Q)
    W = fs_noise_rows(cfg, "w", layer, rows, H) / _F32(cfg["w_div"])
    out["w"] = bf16_bits(W.astype(np.float32))
    return out


def fs_decode_layer_inputs(cfg: dict, layer: int, seqs=None) -> dict:
    """Host-side inputs of one layer of the decode layer-reuse workload, for
    sequences ``seqs`` (all by default): the decode tensors of
    ``decode_inputs`` (e4m3 cache with per-token scales, bf16 q and w), where
    the cache rows (sequence b, token s: row b*Lmax + s), q and w all follow
    the layer recurrence of ``fs_noise_rows``.  ``lens`` is shared by all layers."""
    B, Lmax, H, D = cfg["B"], cfg["Lmax"], cfg["H"], cfg["D"]
    seqs = np.arange(B, dtype=np.int64) if seqs is None else np.asarray(seqs, dtype=np.int64)
    S = len(seqs)
    cache = np.empty((S, Lmax, D), dtype=np.uint8)
    kscale = np.empty((S, Lmax), dtype=np.float32)
    for i, b in enumerate(seqs):
        K = fs_noise_rows(cfg, "k", layer, int(b) * Lmax + np.arange(Lmax, dtype=np.int64), D)
        cache[i], kscale[i] = quant_rows_e4m3(K)
    q = bf16_bits(fs_noise_rows(cfg, "q", layer, seqs, H * D)).reshape(S, H, D)
    w = bf16_bits((fs_noise_rows(cfg, "w", layer, seqs, H) / _F32(cfg["w_div"])).astype(np.float32))
    return {"cache": cache, "k_scale": kscale, "q": q, "w": w, "lens": decode_lens(cfg)[seqs], "seqs": seqs}


def standin_latent(seed: int, which: int, B: int, Lmax: int, seqs=None) -> np.ndarray:
    """Latent cache number ``which`` for the stand-in attention: bf16 bits
    [S, Lmax, 576] of N/4, row b*Lmax + s of stream ("latent", which)."""
    seqs = np.arange(B, dtype=np.int64) if seqs is None else np.asarray(seqs, dtype=np.int64)
    out = np.empty((len(seqs), Lmax, 576), dtype=np.uint16)
    for i, b in enumerate(seqs):
        idx = np.uint64(int(b) * Lmax * 576) + np.arange(Lmax * 576, dtype=np.uint64)
        X = normal_f32(seed, _sid("latent", which), idx) / _F32(4.0)
        out[i] = bf16_bits(X.astype(np.float32)).reshape(Lmax, 576)
    return out


def standin_query(seed: int, layer: int, B: int, seqs=None) -> np.ndarray:
    """Stand-in attention query of layer ``layer``: bf16 bits [S, 576] of N/4."""
    seqs = np.arange(B, dtype=np.int64) if seqs is None else np.asarray(seqs, dtype=np.int64)
    idx = seqs[:, None].astype(np.uint64) * np.uint64(576) + np.arange(576, dtype=np.uint64)[None, :]
    return bf16_bits((normal_f32(seed, _sid("qa", layer), idx) / _F32(4.0)).astype(np.float32))


def fs_keys_by_layer(cfg: dict, last_layer: int):
    """Yields (layer, k codes [L,D] uint8, k_scale [L] float32) for layers
    0..last_layer of the layer-reuse workload, carrying the key recurrence
    forward instead of restarting it for every layer (same values as
    ``fs_layer_inputs(cfg, layer)["k"]``)."""
    L, D = cfg["L"], cfg["D"]
    idx = np.arange(L, dtype=np.uint64)[:, None] * np.uint64(D) + np.arange(D, dtype=np.uint64)[None, :]
    rho, sigma = _F32(cfg["rho"]), _F32(cfg["sigma"])
    X = normal_f32(cfg["seed"], _sid("k", 0), idx)
    for layer in range(last_layer + 1):
        if layer > 0:
            N = normal_f32(cfg["seed"], _sid("k", layer), idx)
            X = ((rho * X).astype(np.float32) + (sigma * N).astype(np.float32)).astype(np.float32)
        codes, scales = quant_rows_e4m3(X)
        yield layer, codes, scales
