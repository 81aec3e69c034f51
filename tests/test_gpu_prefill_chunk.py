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
    """A packed ragged batch in one launch: whole sequences, chunks at the end
    of longer key ranges, a one-token sequence, an empty query range and one
    invalid sequence (more queries than keys, skipped: its rows keep their
    bytes); each valid sequence's rows equal its own call byte for byte, and
    the oracle on sampled rows."""
    import torch
    base = gen.CONFIGS["prefill_32k"]
    topk = 128
    seqs = [(3000, 3000), (1200, 5003), (1, 1), (0, 700), (257, 257), (64, 2500), (40, 20)]   # (Lq, Lk)
    parts = []
    for i, (lq, lk) in enumerate(seqs):
        cfg = dict(base, L=max(lq, lk), topk=topk, heavy_count=max(1, lk // 100), seed=10 + i)
        parts.append(gen.prefill_inputs(cfg))
    rows_of = [np.arange(max(lk - lq, 0), max(lk - lq, 0) + lq) for lq, lk in seqs]
    cat = lambda key, sl: np.concatenate([p[key][sl(i)] for i, p in enumerate(parts)])
    q = cat("q", lambda i: rows_of[i])
    qs = cat("q_scale", lambda i: rows_of[i])
    w = cat("w", lambda i: rows_of[i])
    k = cat("k", lambda i: slice(0, seqs[i][1]))
    ks = cat("k_scale", lambda i: slice(0, seqs[i][1]))
    cu_q = np.concatenate([[0], np.cumsum([lq for lq, _ in seqs])]).astype(np.int32)
    cu_k = np.concatenate([[0], np.cumsum([lk for _, lk in seqs])]).astype(np.int32)
    note("prefill varlen 7 sequences, one launch")
    idx = torch.full((len(q), topk), -7, dtype=torch.int32, device="cuda")
    idx, sc = dsa.dsa_indexer_topk_prefill_varlen(dev(q), dev(qs), dev(k), dev(ks), dev(w), dev(cu_q), dev(cu_k),
                                                  topk, "fp8", out_idx=idx, want_scores=True)
    torch.cuda.synchronize()
    # without scores (items of rows with t + 1 <= topk are then not scored): the same indices
    plain = torch.full((len(q), topk), -7, dtype=torch.int32, device="cuda")
    plain, _ = dsa.dsa_indexer_topk_prefill_varlen(dev(q), dev(qs), dev(k), dev(ks), dev(w), dev(cu_q), dev(cu_k),
                                                   topk, "fp8", out_idx=plain)
    torch.cuda.synchronize()
    assert torch.equal(plain, idx)
    for i, (lq, lk) in enumerate(seqs):
        if lq == 0:
            continue
        if lq > lk:
            assert bool(torch.all(idx[cu_q[i]:cu_q[i + 1]] == -7)), i
            continue
        p = parts[i]
        r = rows_of[i]
        one, one_sc = dsa.dsa_indexer_topk_prefill_chunk(dev(p["q"][r]), dev(p["q_scale"][r]), dev(p["k"][:lk]),
                                                         dev(p["k_scale"][:lk]), dev(p["w"][r]), lk - lq, topk,
                                                         "fp8", want_scores=True)
        torch.cuda.synchronize()
        assert torch.equal(idx[cu_q[i]:cu_q[i + 1]], one), i
        assert torch.equal(sc[cu_q[i]:cu_q[i + 1]], one_sc), i
        pick = np.unique(np.linspace(0, lq - 1, 6).astype(int))
        res = oracle.prefill(p["q"][r][pick], p["q_scale"][r][pick], p["k"][:lk], p["k_scale"][:lk],
                             p["w"][r][pick], "fp8", topk, rows=r[pick], return_scores=True)
        ih = host(idx[cu_q[i]:cu_q[i + 1]])
        for j, t in enumerate(pick):
            assert parity.check_row(ih[t], res["o"][j], res["A"][j], topk) is None, (i, t)


def test_varlen_many_short_sequences_against_oracle(dsa):
    """1100 sequences (more than the 1024 the table builder sorts), each of
    1-40 keys with its last 1-3 rows as queries: every row against the oracle."""
    import torch
    rng = np.random.default_rng(42)
    topk, H, D = 16, 64, 128
    n = 1100
    lk = rng.integers(1, 41, size=n)
    lq = np.minimum(lk, rng.integers(1, 4, size=n))
    cu_q = np.concatenate([[0], np.cumsum(lq)]).astype(np.int32)
    cu_k = np.concatenate([[0], np.cumsum(lk)]).astype(np.int32)
    K, kscale = gen.quant_rows_e4m3(rng.standard_normal((int(cu_k[-1]), D)).astype(np.float32))
    Q, qscale = gen.quant_rows_e4m3(rng.standard_normal((int(cu_q[-1]), H * D)).astype(np.float32))
    Q = Q.reshape(-1, H, D)
    W = gen.bf16_bits((rng.standard_normal((int(cu_q[-1]), H)) / 8).astype(np.float32))
    note("prefill varlen 1100 short sequences")
    idx, sc = dsa.dsa_indexer_topk_prefill_varlen(dev(Q), dev(qscale), dev(K), dev(kscale), dev(W), dev(cu_q),
                                                  dev(cu_k), topk, "fp8", want_scores=True)
    torch.cuda.synchronize()
    ih, sh = host(idx), host(sc)
    for i in range(n):
        q0 = int(lk[i] - lq[i])
        rows = np.arange(q0, int(lk[i]))
        sl = slice(int(cu_q[i]), int(cu_q[i + 1]))
        res = oracle.prefill(Q[sl], qscale[sl], K[cu_k[i]:cu_k[i + 1]], kscale[cu_k[i]:cu_k[i + 1]], W[sl], "fp8",
                             topk, rows=rows, return_scores=True)
        for j in range(len(rows)):
            g = int(cu_q[i]) + j
            assert parity.check_row(ih[g], res["o"][j], res["A"][j], topk, g_score=sh[g]) is None, (i, j)


@pytest.mark.parametrize("dt,H,D", [("bf16", 16, 64), ("fp8", 8, 128), ("bf16", 32, 128), ("fp8", 128, 128),
                                     ("bf16", 64, 128)])
def test_varlen_other_shapes_equal_per_sequence_calls(dsa, dt, H, D):
    """The ragged batch for other built (dtype, H, D): per-head scales for fp8,
    none for bf16; every sequence equals its own chunk call."""
    import torch
    rng = np.random.default_rng(H * D)
    topk = 64
    seqs = [(900, 900), (300, 1400), (1, 70), (65, 65)]
    qs_all, ks_all = None, None
    tq, tk = sum(a for a, _ in seqs), sum(b for _, b in seqs)
    if dt == "bf16":
        q = gen.bf16_bits((rng.standard_normal((tq, H, D)) / 8).astype(np.float32))
        k = gen.bf16_bits((rng.standard_normal((tk, D)) / 8).astype(np.float32))
    else:
        q, qs_all = gen.quant_rows_e4m3(rng.standard_normal((tq * H, D)).astype(np.float32))
        q, qs_all = q.reshape(tq, H, D), qs_all.reshape(tq, H)       # one scale per (token, head)
        k, ks_all = gen.quant_rows_e4m3(rng.standard_normal((tk, D)).astype(np.float32))
    w = gen.bf16_bits((rng.standard_normal((tq, H)) / 8).astype(np.float32))
    cu_q = np.concatenate([[0], np.cumsum([a for a, _ in seqs])]).astype(np.int32)
    cu_k = np.concatenate([[0], np.cumsum([b for _, b in seqs])]).astype(np.int32)
    stride = 1 if dt == "fp8" else 0
    dq, dk, dw = dev(q), dev(k), dev(w)
    dqs = dev(qs_all) if qs_all is not None else None
    dks = dev(ks_all) if ks_all is not None else None
    note(f"prefill varlen {dt} H={H} D={D}")
    idx, sc = dsa.dsa_indexer_topk_prefill_varlen(dq, dqs, dk, dks, dw, dev(cu_q), dev(cu_k), topk, dt,
                                                  q_scale_head_stride=stride, want_scores=True)
    torch.cuda.synchronize()
    for i, (lq, lk) in enumerate(seqs):
        a, b, c, d = int(cu_q[i]), int(cu_q[i + 1]), int(cu_k[i]), int(cu_k[i + 1])
        one, one_sc = dsa.dsa_indexer_topk_prefill_chunk(dq[a:b], dqs[a:b] if dqs is not None else None, dk[c:d],
                                                         dks[c:d] if dks is not None else None, dw[a:b], lk - lq,
                                                         topk, dt, q_scale_head_stride=stride, want_scores=True)
        torch.cuda.synchronize()
        assert torch.equal(idx[a:b], one) and torch.equal(sc[a:b], one_sc), i
        rows = np.arange(lk - lq, lk)
        res = oracle.prefill(q[a:b], qs_all[a:b] if qs_all is not None else None, k[c:d],
                             ks_all[c:d] if ks_all is not None else None, w[a:b], dt, topk, rows=rows,
                             return_scores=True)
        ih, sh = host(one), host(one_sc)
        for j in range(0, lq, max(1, lq // 7)):
            assert parity.check_row(ih[j], res["o"][j], res["A"][j], topk, g_score=sh[j]) is None, (i, j)


def test_prefill_and_ragged_graph_replays(dsa):
    """The whole-sequence and the ragged-batch prefill captured in HIP graphs
    (the work counter and the item table are written by kernels, no memset)
    and replayed several times, with eager calls on other inputs between the
    replays sharing the same workspace: every replay equals the eager result."""
    import torch
    base = gen.CONFIGS["prefill_32k"]
    topk = 256
    ca = dict(base, L=3000, topk=topk, heavy_count=30, seed=31)
    cb = dict(base, L=2500, topk=topk, heavy_count=25, seed=32)
    ia, ib = gen.prefill_inputs(ca), gen.prefill_inputs(cb)
    da = {key: dev(ia[key]) for key in ("q", "q_scale", "k", "k_scale", "w")}
    db = {key: dev(ib[key]) for key in ("q", "q_scale", "k", "k_scale", "w")}
    ws = torch.full((dsa.dsa_indexer_topk_prefill_workspace(3000, 64, 128, topk, "fp8"),), 0x5A, dtype=torch.uint8,
                    device="cuda")
    note("prefill graph: eager references")
    want_a, _, _ = dsa.dsa_indexer_topk_prefill(da["q"], da["q_scale"], da["k"], da["k_scale"], da["w"], topk, "fp8")
    want_b, _, _ = dsa.dsa_indexer_topk_prefill(db["q"], db["q_scale"], db["k"], db["k_scale"], db["w"], topk, "fp8")
    # ragged batch of the two sequences, the second one as its last 700 rows
    q = torch.cat([da["q"], db["q"][-700:]])
    qs = torch.cat([da["q_scale"], db["q_scale"][-700:]])
    w = torch.cat([da["w"], db["w"][-700:]])
    k = torch.cat([da["k"], db["k"]])
    ks = torch.cat([da["k_scale"], db["k_scale"]])
    cu_q = torch.tensor([0, 3000, 3700], dtype=torch.int32, device="cuda")
    cu_k = torch.tensor([0, 3000, 5500], dtype=torch.int32, device="cuda")
    wsr = torch.full((dsa.dsa_indexer_topk_prefill_varlen_workspace(2, 3700, 64, 128, topk, "fp8"),), 0xFF,
                     dtype=torch.uint8, device="cuda")
    oa = torch.empty((3000, topk), dtype=torch.int32, device="cuda")
    orr = torch.empty((3700, topk), dtype=torch.int32, device="cuda")

    def whole():
        dsa.dsa_indexer_topk_prefill(da["q"], da["q_scale"], da["k"], da["k_scale"], da["w"], topk, "fp8",
                                     out_idx=oa, workspace=ws)

    def ragged():
        dsa.dsa_indexer_topk_prefill_varlen(q, qs, k, ks, w, cu_q, cu_k, topk, "fp8", out_idx=orr, workspace=wsr)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):   # warm-up on the capture stream
        whole()
        ragged()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g1, g2 = torch.cuda.CUDAGraph(), torch.cuda.CUDAGraph()
    with torch.cuda.graph(g1):
        whole()
    with torch.cuda.graph(g2):
        ragged()
    for rep in range(3):
        note(f"prefill graph replay {rep}")
        oa.fill_(-7)
        orr.fill_(-7)
        g1.replay()
        g2.replay()
        torch.cuda.synchronize()
        assert torch.equal(oa, want_a), rep
        assert torch.equal(orr[:3000], want_a) and torch.equal(orr[3000:], want_b[-700:]), rep
        other, _, _ = dsa.dsa_indexer_topk_prefill(db["q"], db["q_scale"], db["k"], db["k_scale"], db["w"], topk,
                                                   "fp8", workspace=ws)
        torch.cuda.synchronize()
        assert torch.equal(other, want_b), rep
