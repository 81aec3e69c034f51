"""GPU tests of the lagged (multi-layer indexer) decode schedule and of its
stand-in attention consumer, through the C ABI."""
import numpy as np
import pytest

import oracle
from synth import gen
from tests import parity
from tests.gpu_util import dev, host, note

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dsa():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import sparse_attention_token_02_amd as m
    return m


def _std_sel(rng, B, Lmax, topk):
    sel = np.full((B, topk), -1, dtype=np.int32)
    for b in range(B - 1):
        n = int(rng.integers(1, min(topk, Lmax) + 1))
        sel[b, :n] = np.sort(rng.choice(Lmax, size=n, replace=False))
    return sel   # the last row is all padding


@pytest.mark.parametrize("B,Lmax,topk,scale", [(5, 3000, 256, 1.0), (3, 700, 2048, 0.0417), (2, 130, 100, 4.0)])
def test_standin_attention_matches_oracle(dsa, B, Lmax, topk, scale):
    import torch
    rng = np.random.default_rng(B * 7 + topk)
    lat = gen.standin_latent(1, 0, B, Lmax)
    q = gen.standin_query(1, 0, B)
    sel = _std_sel(rng, B, Lmax, topk)
    sel[0, 0] = Lmax + 3 if sel[0, 0] >= 0 and topk > 1 else sel[0, 0]   # out-of-range entry: skipped
    note(f"standin attention B={B} Lmax={Lmax} k={topk}")
    out = dsa.standin_sparse_attention(dev(q), dev(lat), dev(sel), scale)
    torch.cuda.synchronize()
    want = oracle.standin_attention(q, lat, sel, scale)
    got = host(out).astype(np.float64)
    np.testing.assert_allclose(got, want, rtol=1e-4, atol=2e-6)
    assert np.all(got[-1] == 0.0)


def test_mli_schedule_matches_oracle_and_waits_for_each_selection(dsa):
    """FSFFSFF, B=3: every layer attends the selection the oracle's lagged
    schedule names, byte for byte equal to a standalone decode of that layer
    (itself checked against the oracle), the stand-in attention of every
    layer matches the oracle on it, and slot i ends with the i-th F layer's
    selection.  The side stream is held back by a sleep and the slots start
    as a sentinel, so an attention that did not wait for its indexer would
    be seen."""
    import torch
    cfg = dict(gen.CONFIGS["fs_decode_47"], B=3, Lmax=3000, topk=256, ragged=True)
    pattern = "FSFFSFF"
    N, B, topk = len(pattern), cfg["B"], cfg["topk"]
    note("mli schedule 7 layers B=3 Lmax=3000 k=256")
    hl = [gen.fs_decode_layer_inputs(cfg, l) if pattern[l] == "F" else None for l in range(N)]
    dl = [{key: dev(v) for key, v in h.items() if key != "seqs"} if h else None for h in hl]
    pick = lambda key: [dl[l][key] if dl[l] else None for l in range(N)]
    lens = dl[0]["lens"]
    lat = [dev(gen.standin_latent(2, l % 2, B, cfg["Lmax"])) for l in range(2)]
    qa = [dev(gen.standin_query(2, l, B)) for l in range(N)]
    got_sel = [torch.empty((B, topk), dtype=torch.int32, device="cuda") for _ in range(N)]
    got_out = [torch.empty((B, 512), dtype=torch.float32, device="cuda") for _ in range(N)]
    aws = torch.empty(dsa.standin_sparse_attention_workspace(B, topk), dtype=torch.uint8, device="cuda")
    calls = []

    def attn(layer, src, selection):
        calls.append((layer, src))
        got_sel[layer].copy_(selection)
        dsa.standin_sparse_attention(qa[layer], lat[layer % 2], selection, 0.5, out=got_out[layer], workspace=aws)

    nf = pattern.count("F")
    sel_buf = torch.full((nf, B, topk), -7, dtype=torch.int32, device="cuda")
    side = torch.cuda.Stream()
    torch.cuda.synchronize()
    with torch.cuda.stream(side):
        torch.cuda._sleep(5_000_000)
    sel_buf, asrc = dsa.indexcache_run_decode_layers_mli(pattern, pick("q"), pick("w"), pick("cache"),
                                                         pick("k_scale"), lens, topk, sel_buf=sel_buf, attn=attn,
                                                         side_stream=side)
    torch.cuda.synchronize()
    assert asrc == oracle.mli_resolve(pattern) == [0, 0, 0, 2, 3, 3, 5]
    assert calls == list(enumerate(asrc))
    want, osrc, ncalls = oracle.mli_run(pattern, lambda l: oracle.decode(
        hl[l]["q"], hl[l]["w"], hl[l]["cache"], hl[l]["k_scale"], hl[l]["lens"], topk, return_scores=True))
    assert ncalls == pattern.count("F")
    alone = {}
    for l in range(N):
        if pattern[l] == "F":
            alone[l], _ = dsa.dsa_indexer_topk_decode(dl[l]["q"], dl[l]["w"], dl[l]["cache"], dl[l]["k_scale"],
                                                      lens, topk)
    torch.cuda.synchronize()
    for l in range(N):
        s = asrc[l]
        assert torch.equal(got_sel[l], alone[s]), (l, s)
        g = host(got_sel[l])
        M = parity.decode_query_mag(hl[s]["q"], hl[s]["w"], hl[s]["cache"], hl[s]["k_scale"], hl[s]["lens"])
        for b in range(B):
            assert parity.check_row(g[b], want[l]["o"][b], want[l]["A"][b], topk, fmt="fp8q",
                                    M=M[b]) is None, (l, b)
        ref = oracle.standin_attention(host(qa[l]), host(lat[l % 2]), g, 0.5)
        np.testing.assert_allclose(host(got_out[l]).astype(np.float64), ref, rtol=1e-4, atol=2e-6)
    # lagged: the F layers 2, 3, 5, 6 attend the previous F layer, not themselves
    assert not torch.equal(got_sel[3], alone[3])
    f_layers = [l for l in range(N) if pattern[l] == "F"]
    for i, f in enumerate(f_layers):
        assert torch.equal(sel_buf[i], alone[f]), i


def test_mli_without_attention_and_on_one_stream(dsa):
    """attn may be NULL, and the same stream for both roles gives the same
    selections (serially)."""
    import torch
    cfg = dict(gen.CONFIGS["fs_decode_47"], B=2, Lmax=1500, topk=64, ragged=True)
    pattern = "FFS"
    N = len(pattern)
    note("mli one stream B=2")
    dl = [{key: dev(v) for key, v in gen.fs_decode_layer_inputs(cfg, l).items() if key != "seqs"} if pattern[l] == "F"
          else None for l in range(N)]
    pick = lambda key: [dl[l][key] if dl[l] else None for l in range(N)]
    cur = torch.cuda.current_stream()
    sel_a, _ = dsa.indexcache_run_decode_layers_mli(pattern, pick("q"), pick("w"), pick("cache"), pick("k_scale"),
                                                    dl[0]["lens"], cfg["topk"], side_stream=cur)
    sel_b, _ = dsa.indexcache_run_decode_layers_mli(pattern, pick("q"), pick("w"), pick("cache"), pick("k_scale"),
                                                    dl[0]["lens"], cfg["topk"])
    torch.cuda.synchronize()
    assert torch.equal(sel_a, sel_b)
    one, _ = dsa.dsa_indexer_topk_decode(dl[1]["q"], dl[1]["w"], dl[1]["cache"], dl[1]["k_scale"], dl[1]["lens"],
                                         cfg["topk"])
    torch.cuda.synchronize()
    assert torch.equal(sel_a[1], one)   # the second F layer wrote the second slot
