"""GPU parity of the decode indexer over a paged key cache: the same bytes as
the contiguous decode on the cache the pages describe, and the fp64 oracle."""
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


def _paginate(cache, k_scale, lens, page, seed, spare=3):
    """Scatter a contiguous [B, Lmax, D] cache into shuffled pages; blocks past
    each sequence's end get -1 in the table, spare pages hold junk."""
    import torch
    B, Lmax, D = cache.shape
    mb = Lmax // page
    g = torch.Generator().manual_seed(seed)
    n_used = B * mb
    perm = torch.randperm(n_used + spare, generator=g)[:n_used].to(cache.device)
    pages = torch.full((n_used + spare, page, D), 0x7E, dtype=torch.uint8, device=cache.device)
    spages = torch.full((n_used + spare, page), 1e30, dtype=torch.float32, device=cache.device)
    pages.index_copy_(0, perm, cache.reshape(n_used, page, D))
    spages.index_copy_(0, perm, k_scale.reshape(n_used, page))
    table = perm.to(torch.int32).reshape(B, mb).clone()
    nblk = (lens.to(torch.int64) + page - 1) // page
    table[torch.arange(mb, device=cache.device)[None, :] >= nblk[:, None]] = -1
    return pages, spages, table


@pytest.mark.parametrize("page,H,D", [(32, 64, 128), (64, 64, 128), (256, 64, 128), (64, 16, 64), (128, 32, 128),
                                      (32, 64, 64), (64, 128, 128)])
def test_paged_equals_contiguous_and_oracle(dsa, page, H, D):
    import torch
    B, Lmax, topk = 5, 4096, 256
    rng = np.random.default_rng(page + H + D)
    cache, ks = gen.quant_rows_e4m3(rng.standard_normal((B * Lmax, D)).astype(np.float32))
    cache, ks = cache.reshape(B, Lmax, D), ks.reshape(B, Lmax)
    q = gen.bf16_bits(rng.standard_normal((B, H, D)).astype(np.float32))
    w = gen.bf16_bits((rng.standard_normal((B, H)) / 8).astype(np.float32))
    lens = np.array([4096, 1, 200, 3001, 2048], dtype=np.int32)
    dc, dk, dq, dw, dl = dev(cache), dev(ks), dev(q), dev(w), dev(lens)
    note(f"decode paged page={page} H={H} D={D}")
    idx_c, sc_c = dsa.dsa_indexer_topk_decode(dq, dw, dc, dk, dl, topk, want_scores=True)
    pages, spages, table = _paginate(dc, dk, dl, page, seed=page)
    idx_p, sc_p = dsa.dsa_indexer_topk_decode_paged(dq, dw, pages, spages, table, dl, topk, want_scores=True)
    torch.cuda.synchronize()
    assert torch.equal(idx_p, idx_c) and torch.equal(sc_p, sc_c)
    res = oracle.decode(q, w, cache, ks, lens, topk, return_scores=True)
    M = parity.decode_query_mag(q, w, cache, ks, lens)
    ih, sh = host(idx_p), host(sc_p)
    for b in range(B):
        assert parity.check_row(ih[b], res["o"][b], res["A"][b], topk, g_score=sh[b], fmt="fp8q",
                                M=M[b]) is None, b


def test_paged_lengths_outside_the_cache(dsa):
    """Lengths of 0, below 0 and above the table's reach are clamped on the
    device exactly as in the contiguous decode: empty rows of -1, and a
    length past the last block reads every block."""
    import torch
    B, Lmax, D, H, topk, page = 4, 4096, 128, 64, 256, 64
    rng = np.random.default_rng(31)
    cache, ks = gen.quant_rows_e4m3(rng.standard_normal((B * Lmax, D)).astype(np.float32))
    cache, ks = cache.reshape(B, Lmax, D), ks.reshape(B, Lmax)
    q = gen.bf16_bits(rng.standard_normal((B, H, D)).astype(np.float32))
    w = gen.bf16_bits((rng.standard_normal((B, H)) / 8).astype(np.float32))
    lens = np.array([0, -5, Lmax + 904, 3000], dtype=np.int32)
    dc, dk, dq, dw, dl = dev(cache), dev(ks), dev(q), dev(w), dev(lens)
    note("decode paged lengths 0, negative and past the table")
    idx_c, sc_c = dsa.dsa_indexer_topk_decode(dq, dw, dc, dk, dl, topk, want_scores=True)
    pages, spages, table = _paginate(dc, dk, dl, page, seed=31)
    idx_p, sc_p = dsa.dsa_indexer_topk_decode_paged(dq, dw, pages, spages, table, dl, topk, want_scores=True)
    torch.cuda.synchronize()
    assert torch.equal(idx_p, idx_c) and torch.equal(sc_p, sc_c)
    ih = host(idx_p)
    assert np.all(ih[0] == -1) and np.all(ih[1] == -1)
    res = oracle.decode(q, w, cache, ks, np.clip(lens, 0, Lmax), topk, return_scores=True)
    M = parity.decode_query_mag(q, w, cache, ks, np.clip(lens, 0, Lmax))
    sh = host(sc_p)
    for b in (2, 3):
        assert parity.check_row(ih[b], res["o"][b], res["A"][b], topk, g_score=sh[b], fmt="fp8q",
                                M=M[b]) is None, b


def test_paged_128k_batch_equals_contiguous(dsa):
    """B=32 x 131072 (the benchmark's decode), 64-token pages in shuffled order."""
    import torch
    from synth.gpu import DeviceGen
    cfg = gen.CONFIGS["decode_128k"]
    topk = cfg["topk"]
    note("decode paged 128k: generate")
    d = DeviceGen().decode_inputs(cfg)
    idx_c, sc_c = dsa.dsa_indexer_topk_decode(d["q"], d["w"], d["cache"], d["k_scale"], d["lens"], topk,
                                              want_scores=True)
    pages, spages, table = _paginate(d["cache"], d["k_scale"], d["lens"], 64, seed=7)
    del d["cache"]
    note("decode paged 128k: kernel")
    idx_p, sc_p = dsa.dsa_indexer_topk_decode_paged(d["q"], d["w"], pages, spages, table, d["lens"], topk,
                                                    want_scores=True)
    torch.cuda.synchronize()
    assert torch.equal(idx_p, idx_c) and torch.equal(sc_p, sc_c)
