"""GPU tests of the IndexCache F/S driver and the overlap kernel."""
import numpy as np
import pytest

import oracle
from synth import gen
from tests import parity
from tests.gpu_util import dev, host, note, sample_rows

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dsa():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import sparse_attention_token_02_amd as m
    return m


def _random_sets(N, L, k, seed):
    rng = np.random.default_rng(seed)
    out = np.full((N, L, k), -1, dtype=np.int32)
    for i in range(N):
        for t in range(L):
            n = min(k, t + 1)
            out[i, t, :n] = np.sort(rng.permutation(t + 1)[:n])
    return out


@pytest.mark.parametrize("N,L,k,rows", [(6, 700, 64, None), (47, 1400, 1024, None), (8, 2400, 2048, None), (5, 900, 32, (10, 900, 7)),
                                        (64, 600, 48, None)])
def test_overlap_matches_oracle_exactly(dsa, N, L, k, rows):
    import torch
    sets = _random_sets(N, L, k, seed=N)
    if N > 2:
        sets[2] = sets[1]             # two identical layers
    note(f"overlap N={N} L={L} k={k}")
    idx = [dev(sets[i]) for i in range(N)]
    rb, re_, rs = rows if rows else (k - 1, L, 1)
    counts, ratio = dsa.topk_overlap_matrix(idx, k, row_begin=rb, row_end=re_, row_stride=rs)
    torch.cuda.synchronize()
    C = counts.cpu().numpy().astype(np.uint64)
    R = list(range(rb, re_, rs))
    want = oracle.overlap_counts([sets[i] for i in range(N)], R)
    assert np.array_equal(C, want)
    np.testing.assert_array_equal(ratio, oracle.overlap_ratio(want, k, len(R)))
    if N > 2:
        assert ratio[1, 2] == ratio[1, 1]


@pytest.mark.parametrize("kmax", [131072, 400000])
def test_overlap_of_decode_rows_matches_oracle(dsa, kmax):
    """Decode-shaped rows: one row per sequence, keys far beyond the row
    number (below kmax), short rows padded with -1, one empty row.  Rows of
    up to 16 windows of 8192 keys get their window boundaries up front, longer
    ones (kmax = 400000) one search per window."""
    import torch
    rng = np.random.default_rng(5)
    N, R, k = 7, 40, 512
    sets = np.full((N, R, k), -1, dtype=np.int32)
    for b in range(R - 1):
        n = int(rng.integers(k // 2, kmax))
        base = np.sort(rng.choice(n, size=min(k, n), replace=False))
        for i in range(N):
            keep = base.copy()
            swap = rng.random(len(keep)) < 0.3 * i / N       # layers drift apart
            keep[swap] = rng.choice(n, size=int(swap.sum()), replace=True)
            keep = np.unique(keep)[:k]
            sets[i, b, :len(keep)] = keep
    note(f"overlap decode rows N=7 R=40 k=512 kmax={kmax}")
    counts, ratio = dsa.topk_overlap_matrix([dev(sets[i]) for i in range(N)], k, row_begin=0, row_end=R)
    torch.cuda.synchronize()
    want = oracle.overlap_counts([sets[i] for i in range(N)], range(R))
    assert np.array_equal(counts.cpu().numpy().astype(np.uint64), want)
    assert 0.5 < ratio[0, 1] < 1.0 and ratio[0, N - 1] < ratio[0, 1]


def test_overlap_closed_form(dsa):
    import torch
    L, k = 5000, 128
    suf = np.array([list(range(max(0, t - k + 1), t + 1)) + [-1] * (k - min(k, t + 1)) for t in range(L)],
                   dtype=np.int32)
    pre = np.array([list(range(min(k, t + 1))) + [-1] * (k - min(k, t + 1)) for t in range(L)], dtype=np.int32)
    note("overlap closed form")
    counts, _ = dsa.topk_overlap_matrix([dev(suf), dev(pre)], k, ratio=False)
    torch.cuda.synchronize()
    C = counts.cpu().numpy()
    assert int(C[0, 1]) == sum(max(0, 2 * k - t - 1) for t in range(k - 1, L))
    assert int(C[0, 0]) == k * (L - k + 1)


def test_fs_driver_reuses_cache_in_place(dsa):
    import torch
    cfg = dict(gen.CONFIGS["fs_47"], L=900, topk=64)
    pattern = "FSFSSF"
    N = len(pattern)
    note("fs driver 6 layers L=900")
    layers = []
    for l in range(N):
        inp = gen.fs_layer_inputs(cfg, l)
        layers.append({key: (dev(v) if v is not None and key != "rows" else v) for key, v in inp.items()})
    seen = []

    def hook(layer, src, tcache):
        seen.append((layer, src, tcache.data_ptr(), tcache.clone()))

    q = [layers[l]["q"] if pattern[l] == "F" else None for l in range(N)]
    qs = [layers[l]["q_scale"] if pattern[l] == "F" else None for l in range(N)]
    k = [layers[l]["k"] if pattern[l] == "F" else None for l in range(N)]
    ks = [layers[l]["k_scale"] if pattern[l] == "F" else None for l in range(N)]
    w = [layers[l]["w"] if pattern[l] == "F" else None for l in range(N)]
    tcache, src = dsa.indexcache_run_layers(pattern, q, qs, k, ks, w, cfg["topk"], "fp8", hook=hook)
    torch.cuda.synchronize()
    assert src == oracle.fs_resolve(pattern)
    assert [s[0] for s in seen] == list(range(N)) and [s[1] for s in seen] == src
    assert len(set(s[2] for s in seen)) == 1 and seen[0][2] == tcache.data_ptr()
    for l in range(N):
        if pattern[l] == "S":
            assert torch.equal(seen[l][3], seen[src[l]][3]), l
        else:
            alone, _, _ = dsa.dsa_indexer_topk_prefill(q[l], qs[l], k[l], ks[l], w[l], cfg["topk"], "fp8")
            torch.cuda.synchronize()
            assert torch.equal(alone, seen[l][3]), l
    # each F layer against the oracle on sampled rows
    rows = sample_rows(cfg["L"], cfg["topk"], 16)
    for l in range(N):
        if pattern[l] != "F":
            continue
        hi = gen.fs_layer_inputs(cfg, l, rows=rows)
        res = oracle.prefill(hi["q"], hi["q_scale"], hi["k"], hi["k_scale"], hi["w"], "fp8", cfg["topk"],
                             rows=rows, return_scores=True)
        got = host(seen[l][3])
        for r, t in enumerate(rows):
            assert parity.check_row(got[t], res["o"][r], res["A"][r], cfg["topk"]) is None, (l, t)


def test_fs_decode_driver_matches_oracle(dsa):
    """One decode step through the F/S schedule: every F layer's selection
    equals the oracle's for every sequence, S layers hand on their source's
    buffer unchanged, and an F layer equals a standalone decode call."""
    import torch
    cfg = dict(gen.CONFIGS["fs_decode_47"], B=3, Lmax=3000, topk=256, ragged=True)
    pattern = "FSSFSF"
    N, B, topk = len(pattern), cfg["B"], cfg["topk"]
    note("fs decode driver 6 layers B=3 Lmax=3000 k=256")
    hl = [gen.fs_decode_layer_inputs(cfg, l) if pattern[l] == "F" else None for l in range(N)]
    dl = [{key: dev(v) for key, v in h.items() if key != "seqs"} if h else None for h in hl]
    pick = lambda key: [dl[l][key] if dl[l] else None for l in range(N)]
    lens = dl[0]["lens"]
    seen = []

    def hook(layer, src, tcache):
        seen.append((layer, src, tcache.data_ptr(), tcache.clone()))

    tcache, src = dsa.indexcache_run_decode_layers(pattern, pick("q"), pick("w"), pick("cache"), pick("k_scale"),
                                                   lens, topk, hook=hook)
    torch.cuda.synchronize()
    assert src == oracle.fs_resolve(pattern)
    assert [s[0] for s in seen] == list(range(N)) and [s[1] for s in seen] == src
    assert len(set(s[2] for s in seen)) == 1 and seen[0][2] == tcache.data_ptr()
    want, osrc, calls = oracle.fs_run(pattern, lambda l: oracle.decode(
        hl[l]["q"], hl[l]["w"], hl[l]["cache"], hl[l]["k_scale"], hl[l]["lens"], topk, return_scores=True))
    assert osrc == src and calls == pattern.count("F")
    M = {l: parity.decode_query_mag(hl[l]["q"], hl[l]["w"], hl[l]["cache"], hl[l]["k_scale"], hl[l]["lens"])
         for l in range(N) if hl[l]}
    for l in range(N):
        got = host(seen[l][3])
        for b in range(B):
            assert parity.check_row(got[b], want[l]["o"][b], want[l]["A"][b], topk, fmt="fp8q",
                                    M=M[src[l]][b]) is None, (l, b)
        if pattern[l] == "S":
            assert torch.equal(seen[l][3], seen[src[l]][3]), l
        else:
            alone, _ = dsa.dsa_indexer_topk_decode(dl[l]["q"], dl[l]["w"], dl[l]["cache"], dl[l]["k_scale"], lens,
                                                   topk)
            torch.cuda.synchronize()
            assert torch.equal(alone, seen[l][3]), l
    # the layers differ, so the S layers really did reuse rather than recompute
    assert not torch.equal(seen[0][3], seen[3][3])
    # overlap of the per-layer decode selections (rows are sequences)
    counts, _ = dsa.topk_overlap_matrix([s[3] for s in seen], topk, row_begin=0, row_end=B, ratio=False)
    torch.cuda.synchronize()
    want_c = oracle.overlap_counts([want[l]["idx"] for l in range(N)], range(B))
    assert np.array_equal(counts.cpu().numpy().astype(np.uint64), want_c)
    assert want_c[0, 3] > 0
