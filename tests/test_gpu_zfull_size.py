"""Full-size GPU parity runs of the long-context prefill and of the 47-layer
IndexCache schedule, checked against the fp64 oracle on seeded row samples
and against the schedule's own invariants.  These allocate tens of GB of
device memory and run last."""
import numpy as np
import pytest

import oracle
from synth import gen
from tests import parity
from tests.gpu_util import check_structure_all, host, note, sample_rows

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dsa():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import sparse_attention_token_02_amd as m
    return m


def _oracle_rows_chunked(q, qs, k, ks, w, rows, topk, chunk=8):
    """oracle.prefill on `rows`, a few rows at a time (memory bound on host)."""
    os_, As_ = [], []
    for i in range(0, len(rows), chunk):
        sl = slice(i, i + chunk)
        res = oracle.prefill(q[sl], None if qs is None else qs[sl], k, ks, w[sl], "fp8", topk, rows=rows[sl],
                             return_scores=True)
        os_ += res["o"]
        As_ += res["A"]
    return os_, As_


def test_prefill_196k_sampled_rows(dsa):
    """L=196608 fp8 prefill in the benchmark's launch configuration; oracle on
    a seeded sample of 512 query rows (with the first and last rows)."""
    import torch
    from synth.gpu import DeviceGen
    cfg = gen.CONFIGS["prefill_196k"]
    L, topk = cfg["L"], cfg["topk"]
    note("prefill 196k generate")
    d = DeviceGen().prefill_inputs(cfg)
    note("prefill 196k kernel")
    idx, sc, _ = dsa.dsa_indexer_topk_prefill(d["q"], d["q_scale"], d["k"], d["k_scale"], d["w"], topk, "fp8",
                                              want_scores=True)
    torch.cuda.synchronize()
    check_structure_all(idx, topk)
    rows = sample_rows(L, topk, 512, seed=196)
    hi = gen.prefill_inputs(cfg, rows=rows)
    assert np.array_equal(host(d["k"]), hi["k"])
    sel = torch.from_numpy(rows).cuda()
    idx_h, sc_h = host(idx[sel]), host(sc[sel])
    note("prefill 196k oracle (512 rows)")
    o, A = _oracle_rows_chunked(hi["q"], hi["q_scale"], hi["k"], hi["k_scale"], hi["w"], rows, topk)
    bad = [(int(t), e) for r, t in enumerate(rows)
           if (e := parity.check_row(idx_h[r], o[r], A[r], topk, g_score=sc_h[r]))]
    assert not bad, f"{len(bad)} rows differ, first: {bad[:3]}"


def _fs47_check_rows(job):
    """Worker thread: the oracle on a few sampled rows of one layer, checked
    against those rows of every run that computed the layer.  Returns the
    failures (rows and floor-decided rows are counted in parity.STATS)."""
    layer, hi, kc, ks, rows, sl, topk, got_by_run = job
    o, A = _oracle_rows_chunked(hi["q"][sl], hi["q_scale"][sl], kc, ks, hi["w"][sl], rows[sl], topk)
    errs = []
    for run, got in got_by_run.items():
        for r, t in enumerate(rows[sl]):
            e = parity.check_row(got[sl][r], o[r], A[r], topk, row_id=(run, layer, int(t)))
            if e:
                errs.append((run, layer, int(t), e))
    return errs


@pytest.fixture(scope="module")
def fs47(dsa):
    """The 47-layer schedule at L=65536 under all three patterns: every
    layer's indices of the all-F run (kept on the device), and the F layers of
    the other two runs, with the S-layer identities checked as they run."""
    import torch
    from synth.gpu import DeviceGen
    cfg = gen.CONFIGS["fs_47"]
    N, L, topk = cfg["N"], cfg["L"], cfg["topk"]
    g = DeviceGen()
    note("fs47 generate 47 layers")
    layers = [g.fs_layer_inputs(cfg, l) for l in range(N)]
    runs = {}
    for pname, pat in gen.FS_PATTERNS.items():
        src = dsa.indexcache_resolve(pat)
        for l in range(N):
            assert src[l] == (l if pat[l] == "F" else max(j for j in range(l) if pat[j] == "F"))
        keep = [None] * N
        seen = []

        def hook(layer, s, tc, keep=keep, seen=seen, pat=pat):
            seen.append((layer, s, tc.data_ptr()))
            if pat[layer] == "F":
                keep[layer] = tc.clone()
            else:   # an S layer sees its source layer's bytes, in place
                assert torch.equal(tc, keep[s]), (pat, layer)

        note(f"fs47 run {pname}")
        tcache = torch.empty((L, topk), dtype=torch.int32, device="cuda")
        dsa.indexcache_run_layers(pat, [x["q"] for x in layers], [x["q_scale"] for x in layers],
                                  [x["k"] for x in layers], [x["k_scale"] for x in layers],
                                  [x["w"] for x in layers], topk, "fp8", tcache=tcache, hook=hook)
        torch.cuda.synchronize()
        assert [x[0] for x in seen] == list(range(N))
        assert all(p == tcache.data_ptr() for _, _, p in seen)       # one buffer, overwritten in place
        runs[pname] = keep
    del layers
    return cfg, runs


def test_fs47_full_size_layers_against_oracle(dsa, fs47):
    """Every layer of the all-F run, and every F layer of the two 12-F
    patterns, against the oracle on 64 seeded rows plus the edge rows; the F
    layers of the 12-F runs are byte-identical to the same layers of the
    all-F run."""
    import os
    import torch
    from concurrent.futures import ThreadPoolExecutor
    from threadpoolctl import threadpool_limits
    cfg, runs = fs47
    N, L, topk = cfg["N"], cfg["L"], cfg["topk"]
    for pname, pat in gen.FS_PATTERNS.items():
        for l in range(N):
            if pat[l] == "F":
                assert torch.equal(runs[pname][l], runs["all_F"][l]), (pname, l)
    check_structure_all(runs["all_F"][N - 1], topk)
    rows = sample_rows(L, topk, 64, seed=47)
    sel = torch.from_numpy(rows).cuda()
    note(f"fs47 oracle: {N} layers x {len(rows)} rows")
    # numpy releases the GIL inside BLAS: worker threads with one BLAS thread
    # each (a process pool would fork a process that holds the GPU)
    workers = max(1, min(16, os.cpu_count() or 1))
    futs = []
    with threadpool_limits(1), ThreadPoolExecutor(max_workers=workers) as ex:
        for layer, kc, ks in gen.fs_keys_by_layer(cfg, N - 1):
            hi = gen.fs_layer_inputs(cfg, layer, rows=rows, with_keys=False)
            got = {p: host(runs[p][layer][sel]) for p, pat in gen.FS_PATTERNS.items() if pat[layer] == "F"}
            for i in range(0, len(rows), 8):
                futs.append(ex.submit(_fs47_check_rows, (layer, hi, kc, ks, rows, slice(i, i + 8), topk, got)))
        errs = [e for f in futs for e in f.result()]
    assert parity.STATS["rows"] >= N * 64
    assert not errs, f"{len(errs)} rows differ, first: {errs[:3]}"


def test_fs47_full_size_overlap_against_oracle(dsa, fs47):
    """The 47x47 overlap counts of the all-F run against the oracle on a
    strided row sample; symmetric, with k * rows on the diagonal."""
    import torch
    cfg, runs = fs47
    N, L, topk = cfg["N"], cfg["L"], cfg["topk"]
    keep = runs["all_F"]
    rb, re_, rs = topk - 1, L, 1021
    note("fs47 overlap")
    counts, ratio = dsa.topk_overlap_matrix(keep, topk, row_begin=rb, row_end=re_, row_stride=rs)
    torch.cuda.synchronize()
    R = list(range(rb, re_, rs))
    selr = torch.tensor(R, device="cuda")
    sets = [host(keep[l][selr]) for l in range(N)]
    # the oracle reads idx_layers[i][t]; only the sampled rows are needed
    rows_of = [{t: sets[l][r] for r, t in enumerate(R)} for l in range(N)]
    want = oracle.overlap_counts(rows_of, R)
    C = counts.cpu().numpy().astype(np.uint64)
    assert np.array_equal(C, want)
    assert np.array_equal(C, C.T)
    for l in range(N):
        assert C[l, l] == len(R) * topk
    assert np.allclose(ratio, want.astype(np.float64) / (topk * len(R)))
