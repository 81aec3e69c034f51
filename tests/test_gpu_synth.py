"""The device input generator reproduces the host generator bit for bit."""
import numpy as np
import pytest

from synth import gen
from tests.gpu_util import host, note

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def g():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from synth.gpu import DeviceGen
    return DeviceGen()


def test_tiny_bf16_tensors_identical(g):
    cfg = gen.CONFIGS["tiny"]
    note("synth tiny")
    d = g.prefill_inputs(cfg)
    h = gen.prefill_inputs(cfg)
    for key in ("q", "k", "w"):
        assert np.array_equal(host(d[key]), h[key]), key
    assert np.array_equal(d["heavy"], h["heavy"])


def test_fp8_prefill_rows_identical(g):
    import torch
    cfg = dict(gen.CONFIGS["prefill_32k"], L=3000, heavy_count=30)
    note("synth fp8 prefill L=3000")
    d = g.prefill_inputs(cfg)
    h = gen.prefill_inputs(cfg)
    for key in ("q", "q_scale", "k", "k_scale", "w"):
        assert np.array_equal(host(d[key]), h[key]), key


def test_fs_layer_recurrence_identical(g):
    cfg = dict(gen.CONFIGS["fs_47"], L=500)
    note("synth fs layers 0, 1, 7")
    for layer in (0, 1, 7):
        d = g.fs_layer_inputs(cfg, layer)
        h = gen.fs_layer_inputs(cfg, layer)
        for key in ("q", "q_scale", "k", "k_scale", "w"):
            assert np.array_equal(host(d[key]), h[key]), (layer, key)


def test_decode_small_identical(g):
    cfg = dict(gen.CONFIGS["decode_128k"], B=3, Lmax=4000, ragged=True)
    note("synth decode B=3")
    d = g.decode_inputs(cfg)
    h = gen.decode_inputs(cfg)
    for key in ("cache", "k_scale", "q", "w", "lens"):
        assert np.array_equal(host(d[key]), h[key]), key


def test_fs_decode_layer_recurrence_identical(g):
    cfg = dict(gen.CONFIGS["fs_decode_47"], B=3, Lmax=1500, ragged=True)
    note("synth fs decode layers 0, 3")
    for layer in (0, 3):
        d = g.fs_decode_layer_inputs(cfg, layer)
        h = gen.fs_decode_layer_inputs(cfg, layer)
        for key in ("cache", "k_scale", "q", "w", "lens"):
            assert np.array_equal(host(d[key]), h[key]), (layer, key)
