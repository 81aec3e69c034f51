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
