"""GPU parity of the chunked prefill (a block of query rows at an offset into
the sequence) against the whole-sequence prefill and the fp64 oracle."""
import numpy as np
import pytest

import oracle
from synth import gen
from tests import parity
from tests.gpu_util import check_structure_all, dev, host, note

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dsa():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import sparse_attention_token_02_amd as m
    return m


def _whole(dsa, d, topk, dt):
    import torch
    idx, sc, _ = dsa.dsa_indexer_topk_prefill(d["q"], d["q_scale"], d["k"], d["k_scale"], d["w"], topk, dt,
                                              want_scores=True)
    torch.cuda.synchronize()
    return idx, sc


def _chunk(dsa, d, q0, lq, topk, dt):
    import torch
    qs = d["q_scale"][q0:q0 + lq] if d["q_scale"] is not None else None
    ks = d["k_scale"][:q0 + lq] if d["k_scale"] is not None else None
    idx, sc = dsa.dsa_indexer_topk_prefill_chunk(d["q"][q0:q0 + lq], qs, d["k"][:q0 + lq], ks, d["w"][q0:q0 + lq],
                                                 q0, topk, dt, want_scores=True)
    torch.cuda.synchronize()
    return idx, sc


@pytest.mark.parametrize("cfg_name,L,topk", [("prefill_32k", 5000, 256), ("tiny", 2048, 128)])
def test_chunks_equal_whole_sequence_rows(dsa, cfg_name, L, topk):
    """Chunks at ragged offsets (below k, inside an item, single rows, the
    tail) return exactly the whole-sequence rows, indices and scores."""
    import torch
    cfg = dict(gen.CONFIGS[cfg_name], L=L, topk=topk, heavy_count=max(1, L // 100))
    inp = gen.prefill_inputs(cfg)
    d = {key: (dev(inp[key]) if inp.get(key) is not None else None) for key in ("q", "q_scale", "k", "k_scale", "w")}
    dt = cfg["dtype"]
    note(f"prefill chunks {cfg_name} L={L} k={topk}: whole")
    idx_w, sc_w = _whole(dsa, d, topk, dt)
    cuts = [(0, 100), (100, 1), (101, topk), (101 + topk, 333), (700, 1), (701, 1200), (1901, L - 1901)]
    for q0, lq in cuts:
        note(f"prefill chunk q0={q0} Lq={lq}")
        idx_c, sc_c = _chunk(dsa, d, q0, lq, topk, dt)
        assert torch.equal(idx_c, idx_w[q0:q0 + lq]), (q0, lq)
        assert torch.equal(sc_c, sc_w[q0:q0 + lq]), (q0, lq)
    # one chunk against the oracle, every row
    q0 = 1901
    lq = min(150, L - q0)
    idx_c, sc_c = _chunk(dsa, d, q0, lq, topk, dt)
    rows = np.arange(q0, q0 + lq)
    qs = inp["q_scale"][rows] if inp.get("q_scale") is not None else None
    res = oracle.prefill(inp["q"][rows], qs, inp["k"], inp.get("k_scale"), inp["w"][rows], dt, topk, rows=rows,
                         return_scores=True)
    ih, sh = host(idx_c), host(sc_c)
    for r, t in enumerate(rows):
        assert parity.check_row(ih[r], res["o"][r], res["A"][r], topk, g_score=sh[r]) is None, t


def test_chunk_32k_tail_equals_whole_run(dsa):
    """The last 8192 rows of the L=32768 benchmark sequence as one chunk, and
    the same rows as four chunks of 2048: identical to the whole run."""
    import torch
    from synth.gpu import DeviceGen
    cfg = gen.CONFIGS["prefill_32k"]
    L, topk = cfg["L"], cfg["topk"]
    note("prefill 32k chunk: generate")
    d = DeviceGen().prefill_inputs(cfg)
    note("prefill 32k chunk: whole")
    idx_w, sc_w = _whole(dsa, d, topk, "fp8")
    note("prefill 32k chunk: tail")
    idx_c, sc_c = _chunk(dsa, d, L - 8192, 8192, topk, "fp8")
    check_structure_all(idx_c, topk, row0=L - 8192)
    assert torch.equal(idx_c, idx_w[L - 8192:]) and torch.equal(sc_c, sc_w[L - 8192:])
    for j in range(4):
        q0 = L - 8192 + 2048 * j
        idx_j, _ = _chunk(dsa, d, q0, 2048, topk, "fp8")
        assert torch.equal(idx_j, idx_w[q0:q0 + 2048]), j


def test_varlen_batch_equals_per_sequence_calls(dsa):
    """A packed ragged batch: whole sequences, chunks at the end of longer key
    ranges, a one-token sequence and an empty query range; each sequence's
    rows equal its own call byte for byte, and the oracle on sampled rows."""
    import torch
    base = gen.CONFIGS["prefill_32k"]
    topk = 128
    seqs = [(3000, 3000), (1200, 5003), (1, 1), (0, 700), (257, 257), (64, 2500)]   # (Lq, Lk)
    parts = []
    for i, (lq, lk) in enumerate(seqs):
        cfg = dict(base, L=lk, topk=topk, heavy_count=max(1, lk // 100), seed=10 + i)
        parts.append(gen.prefill_inputs(cfg))
    rows_of = [np.arange(lk - lq, lk) for lq, lk in seqs]
    cat = lambda key, sl: np.concatenate([p[key][sl(i)] for i, p in enumerate(parts)])
    q = cat("q", lambda i: rows_of[i])
    qs = cat("q_scale", lambda i: rows_of[i])
    w = cat("w", lambda i: rows_of[i])
    k = cat("k", lambda i: slice(None))
    ks = cat("k_scale", lambda i: slice(None))
    cu_q = np.concatenate([[0], np.cumsum([lq for lq, _ in seqs])]).tolist()
    cu_k = np.concatenate([[0], np.cumsum([lk for _, lk in seqs])]).tolist()
    note("prefill varlen 6 sequences")
    idx, sc = dsa.dsa_indexer_topk_prefill_varlen(dev(q), dev(qs), dev(k), dev(ks), dev(w), cu_q, cu_k, topk, "fp8",
                                                  want_scores=True)
    torch.cuda.synchronize()
    for i, (lq, lk) in enumerate(seqs):
        if lq == 0:
            continue
        p = parts[i]
        r = rows_of[i]
        one, one_sc = dsa.dsa_indexer_topk_prefill_chunk(dev(p["q"][r]), dev(p["q_scale"][r]), dev(p["k"]),
                                                         dev(p["k_scale"]), dev(p["w"][r]), lk - lq, topk, "fp8",
                                                         want_scores=True)
        torch.cuda.synchronize()
        assert torch.equal(idx[cu_q[i]:cu_q[i + 1]], one), i
        assert torch.equal(sc[cu_q[i]:cu_q[i + 1]], one_sc), i
        pick = np.unique(np.linspace(0, lq - 1, 6).astype(int))
        res = oracle.prefill(p["q"][r][pick], p["q_scale"][r][pick], p["k"], p["k_scale"], p["w"][r][pick], "fp8",
                             topk, rows=r[pick], return_scores=True)
        ih = host(idx[cu_q[i]:cu_q[i + 1]])
        for j, t in enumerate(pick):
            assert parity.check_row(ih[t], res["o"][j], res["A"][j], topk) is None, (i, t)
