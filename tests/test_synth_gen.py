"""Pins of the host-side input generator (formats and generator core)."""
import numpy as np
import pytest
import torch

from synth import gen


def test_splitmix64_reference_outputs():
    # First outputs of SplitMix64 started from state 0 (published reference
    # implementation; widely used test vector).
    z = 0
    outs = []
    for _ in range(3):
        z = (z + gen.GAMMA) & ((1 << 64) - 1)
        outs.append(gen.mix64_int(z))
    assert outs[0] == 0xE220A8397B1DCDAF
    assert outs[1] == 0x6E789E6AA1B965F4
    assert outs[2] == 0x06C45D188009454F


def test_hash_matches_scalar_splitmix():
    base = gen.stream_base(7, 1025)
    idx = np.array([0, 1, 2, 12345, 2**40 + 3], dtype=np.uint64)
    h = gen.hash_u64(7, 1025, idx)
    for i, v in zip(idx.tolist(), h.tolist()):
        assert v == gen.mix64_int(base + (i + 1) * gen.GAMMA)


def test_normal_table_moments_and_symmetry():
    t = gen.NORMAL_TABLE.astype(np.float64)
    assert t.shape == (65536,)
    assert np.all(np.diff(t) > 0)
    assert np.max(np.abs(t + t[::-1])) < 1e-6
    assert abs(t.mean()) < 1e-7
    assert abs(t.var() - 1.0) < 2e-3       # discretised N(0,1), tails cut at +-4.33
    x = gen.normal_f32(0, 1, np.arange(1 << 20, dtype=np.uint64)).astype(np.float64)
    assert abs(x.mean()) < 5e-3 and abs(x.std() - 1.0) < 5e-3


def test_uniform_int_range():
    v = gen.uniform_int(0, 5, np.arange(100000, dtype=np.uint64), 65536, 131072)
    assert v.min() >= 65536 and v.max() <= 131072
    assert abs(v.mean() - (65536 + 131072) / 2) < 500


def _torch_e4m3(x):
    return torch.from_numpy(np.asarray(x, dtype=np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def test_e4m3_encoder_matches_torch_in_range():
    rng = np.random.default_rng(0)
    mags = np.exp2(rng.uniform(-14, 8.8, size=200000)).astype(np.float32)
    x = (mags * rng.choice([-1, 1], size=mags.size)).astype(np.float32)
    x = x[np.abs(x) <= 448]
    # exact e4m3 values and exact midpoints between neighbours (ties to even)
    vals = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).float().numpy()
    vals = np.sort(np.unique(vals[np.isfinite(vals)]))
    mids = ((vals[1:].astype(np.float64) + vals[:-1]) / 2).astype(np.float32)
    x = np.concatenate([x, vals.astype(np.float32), mids])
    np.testing.assert_array_equal(gen.e4m3_bits(x), _torch_e4m3(x))


def test_e4m3_encoder_saturates():
    x = np.array([448.0, 449.0, 464.0, 465.0, 480.0, 1e6, -1e6, -500.0], dtype=np.float32)
    assert gen.e4m3_bits(x).tolist() == [0x7E, 0x7E, 0x7E, 0x7E, 0x7E, 0x7E, 0xFE, 0xFE]


def test_bf16_encoder_matches_torch():
    rng = np.random.default_rng(1)
    x = (rng.standard_normal(100000) * np.exp2(rng.uniform(-30, 30, 100000))).astype(np.float32)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(gen.bf16_bits(x), ref)


def test_quant_rows_scale_and_range():
    rng = np.random.default_rng(2)
    X = rng.standard_normal((16, 256)).astype(np.float32)
    X[3] = 0.0
    codes, scale = gen.quant_rows_e4m3(X)
    assert scale[3] == 1.0 and np.all(codes[3] == 0)
    amax = np.abs(X).max(axis=1)
    np.testing.assert_array_equal(scale[amax > 0], (amax / np.float32(448))[amax > 0])
    dec = torch.from_numpy(codes).view(torch.float8_e4m3fn).float().numpy()
    # the largest element of every nonzero row lands on +-448
    for r in range(16):
        if r != 3:
            assert np.abs(dec[r]).max() == 448.0
    # round-trip error of RNE: at most half a unit in the last place of e4m3
    rel = np.abs(dec * scale[:, None] - X) / np.maximum(np.abs(X), 2.0**-6 * scale[:, None])
    assert rel.max() <= 2.0**-4 + 1e-6


def test_prefill_recipe_shapes_and_heavy_keys():
    cfg = dict(gen.CONFIGS["tiny"])
    inp = gen.prefill_inputs(cfg, rows=[0, 5, 2047])
    assert inp["k"].shape == (2048, 64) and inp["k"].dtype == np.uint16
    assert inp["q"].shape == (3, 8, 64) and inp["w"].shape == (3, 8)
    assert len(inp["heavy"]) == 16 and len(np.unique(inp["heavy"])) == 16
    # heavy keys carry 4x the norm of their unplanted draw
    K = torch.from_numpy(inp["k"].view(np.int16)).view(torch.bfloat16).float().numpy()
    raw = gen.normal_f32(0, gen.STREAM["k"] * 1024, np.arange(2048 * 64, dtype=np.uint64)).reshape(2048, 64) / 8
    h = inp["heavy"][0]
    np.testing.assert_allclose(np.linalg.norm(K[h]), 4 * np.linalg.norm(raw[h]), rtol=1e-2)
    # rebuilding a subset of rows gives the same bytes as the full build
    full = gen.prefill_inputs(cfg, rows=None)
    np.testing.assert_array_equal(full["q"][[0, 5, 2047]], inp["q"])
    np.testing.assert_array_equal(full["w"][[0, 5, 2047]], inp["w"])


def test_fp8_recipe_counts():
    cfg = gen.CONFIGS["prefill_32k"]
    assert cfg["heavy_count"] == 328
    assert gen.CONFIGS["prefill_196k"]["heavy_count"] == 1966
    p = gen.FS_PATTERNS
    assert len(p["searched_1_4"]) == 47 and p["searched_1_4"].count("F") == 12
    assert len(p["uniform_1_4"]) == 47 and p["uniform_1_4"].count("F") == 12


def test_fs_recurrence_rows_consistent():
    cfg = gen.CONFIGS["fs_47"]
    a = gen.fs_noise_rows(cfg, "q", 3, [0, 9], 16)
    b = gen.fs_noise_rows(cfg, "q", 3, [9], 16)
    np.testing.assert_array_equal(a[1], b[0])
    # correlation between consecutive layers close to rho / sqrt(rho^2 + sigma^2)
    x2 = gen.fs_noise_rows(cfg, "k", 2, np.arange(2000), 64).ravel()
    x3 = gen.fs_noise_rows(cfg, "k", 3, np.arange(2000), 64).ravel()
    c = np.corrcoef(x2, x3)[0, 1]
    assert abs(c - 0.9 / np.sqrt(0.81 + 0.44**2)) < 0.01


def test_fs_decode_layer_zero_is_the_decode_recipe():
    """Layer 0 of the decode layer-reuse workload draws the same streams and
    rows as the single-layer decode recipe, so the two agree bit for bit."""
    cfg = dict(gen.CONFIGS["fs_decode_47"], B=3, Lmax=700, ragged=True)
    a = gen.fs_decode_layer_inputs(cfg, 0)
    b = gen.decode_inputs(cfg)
    for key in ("cache", "k_scale", "q", "w", "lens"):
        np.testing.assert_array_equal(a[key], b[key], err_msg=key)
    c = gen.fs_decode_layer_inputs(cfg, 2, seqs=[1])
    d = gen.fs_decode_layer_inputs(cfg, 2)
    for key in ("cache", "k_scale", "q", "w", "lens"):
        np.testing.assert_array_equal(c[key][0], d[key][1], err_msg=key)
