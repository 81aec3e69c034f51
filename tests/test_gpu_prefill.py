"""GPU parity of the fused prefill indexer + top-k against the fp64 oracle."""
import numpy as np
import pytest

import oracle
from synth import gen
from tests import parity
from tests.gpu_util import check_structure_all, dev, host, note, sample_rows

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dsa():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import sparse_attention_token_02_amd as m
    return m


def _run(dsa, inp, cfg, **kw):
    import torch
    q = dev(inp["q"])
    k = dev(inp["k"])
    w = dev(inp["w"])
    qs = dev(inp["q_scale"]) if inp.get("q_scale") is not None else None
    ks = dev(inp["k_scale"]) if inp.get("k_scale") is not None else None
    out = dsa.dsa_indexer_topk_prefill(q, qs, k, ks, w, cfg["topk"], cfg["dtype"], **kw)
    torch.cuda.synchronize()
    return out


def _oracle_rows(inp, cfg, rows):
    qs = inp["q_scale"][rows] if inp.get("q_scale") is not None else None
    return oracle.prefill(inp["q"][rows], qs, inp["k"], inp.get("k_scale"), inp["w"][rows], cfg["dtype"],
                          cfg["topk"], rows=rows, return_scores=True)


def _compare(idx, sc, res, rows, topk, fmt="fp8"):
    bad = []
    for r, t in enumerate(rows):
        err = parity.check_row(idx[t], res["o"][r], res["A"][r], topk,
                               g_score=None if sc is None else sc[t], fmt=fmt)
        if err:
            bad.append((int(t), err))
    assert not bad, f"{len(bad)} rows differ, first: {bad[:3]}"


def test_tiny_bf16_every_row_and_dense_scores(dsa):
    cfg = gen.CONFIGS["tiny"]
    note("prefill tiny bf16 L=2048 H=8 D=64 k=128")
    inp = gen.prefill_inputs(cfg)
    idx, sc, dense = _run(dsa, inp, cfg, want_scores=True, want_dense=True)
    idx, sc, dense = host(idx), host(sc), host(dense)
    rows = np.arange(cfg["L"])
    res = _oracle_rows(inp, cfg, rows)
    _compare(idx, sc, res, rows, cfg["topk"], fmt="bf16")
    worst_a = worst_o = 0.0
    for t in rows:
        assert parity.check_dense(dense[t], res["o"][t], res["A"][t]) is None, t
        ea, eo = parity.max_rel_err(dense[t][: t + 1], res["o"][t], res["A"][t])
        worst_a, worst_o = max(worst_a, ea), max(worst_o, eo)
    print(f"tiny dense scores: max |err|/A {worst_a:.3g}, max |err|/|o| (|o| >= 0.1 A) {worst_o:.3g}")
    assert worst_o <= parity.SCORE_RTOL
    assert worst_a <= parity.SCORE_RTOL * parity.SCORE_FLOOR_A


@pytest.mark.parametrize("L,topk", [(1000, 100), (777, 64)])
def test_fp8_small_every_row(dsa, L, topk):
    cfg = dict(gen.CONFIGS["prefill_32k"], L=L, topk=topk, heavy_count=L // 100)
    note(f"prefill fp8 small L={L} k={topk}")
    inp = gen.prefill_inputs(cfg)
    idx, sc, _ = _run(dsa, inp, cfg, want_scores=True)
    idx, sc = host(idx), host(sc)
    rows = np.arange(L)
    _compare(idx, sc, _oracle_rows(inp, cfg, rows), rows, topk)


def test_fp8_per_head_scales(dsa):
    import torch
    cfg = dict(gen.CONFIGS["prefill_32k"], L=600, topk=50, heavy_count=6)
    note("prefill fp8 per-head q scales L=600")
    inp = gen.prefill_inputs(cfg)
    rng = np.random.default_rng(1)
    qs2 = (inp["q_scale"][:, None] * np.exp2(rng.integers(-2, 3, size=(600, 64)))).astype(np.float32)
    out = dsa.dsa_indexer_topk_prefill(dev(inp["q"]), dev(qs2), dev(inp["k"]), dev(inp["k_scale"]),
                                       dev(inp["w"]), 50, "fp8", q_scale_head_stride=1, want_scores=True)
    torch.cuda.synchronize()
    idx, sc = host(out[0]), host(out[1])
    rows = np.arange(600)
    res = oracle.prefill(inp["q"], qs2, inp["k"], inp["k_scale"], inp["w"], "fp8", 50, rows=rows,
                         return_scores=True)
    _compare(idx, sc, res, rows, 50)


def _ramp_inputs(L, H, D, sign, zero_q=False):
    """k = e_0 for every key with k_scale[s] = s + 1 and q = e_0 for every head:
    score(t, s) = (sum_h w[t,h]) * (s + 1) exactly; strictly monotone in s."""
    q = np.zeros((L, H, D), dtype=np.uint8)
    if not zero_q:
        q[:, :, 0] = 0x38                      # e4m3 1.0
    k = np.zeros((L, D), dtype=np.uint8)
    k[:, 0] = 0x38
    ks = np.arange(1, L + 1, dtype=np.float32)
    qs = np.ones(L, dtype=np.float32)
    rng = np.random.default_rng(2)
    w = gen.bf16_bits((rng.uniform(0.1, 1.0, size=(L, H)) * sign).astype(np.float32))
    return {"q": q, "q_scale": qs, "k": k, "k_scale": ks, "w": w}


@pytest.mark.parametrize("case", ["increasing", "decreasing", "all_zero"])
def test_closed_form_orders_stress_the_streaming_select(dsa, case):
    """Increasing scores make every key beat the running threshold, so the
    candidate lists overflow and are compacted many times per row; all-zero
    scores are one giant tie that must resolve to the lowest indices."""
    L, H, D, topk = 3000, 64, 128, 64
    sign = -1.0 if case == "decreasing" else 1.0
    inp = _ramp_inputs(L, H, D, sign, zero_q=(case == "all_zero"))
    cfg = {"topk": topk, "dtype": "fp8"}
    note(f"prefill closed form {case} L={L} k={topk}")
    idx, sc, _ = _run(dsa, inp, cfg, want_scores=True)
    idx = host(idx)
    for t in range(L):
        n = min(topk, t + 1)
        want = list(range(t - n + 1, t + 1)) if case == "increasing" else list(range(n))
        assert idx[t].tolist() == want + [-1] * (topk - n), t
    rows = sample_rows(L, topk, 24)
    _compare(idx, host(sc), _oracle_rows(inp, cfg, rows), rows, topk)


def test_deterministic_bytes(dsa):
    import torch
    cfg = dict(gen.CONFIGS["prefill_32k"], L=2500, topk=256, heavy_count=25)
    note("prefill determinism L=2500")
    inp = gen.prefill_inputs(cfg)
    ws_bytes = dsa.dsa_indexer_topk_prefill_workspace(2500, 64, 128, 256, "fp8")
    ws = torch.full((ws_bytes,), 0x5A, dtype=torch.uint8, device="cuda")
    a = _run(dsa, inp, cfg, want_scores=True, workspace=ws)
    ws.fill_(0xC3)
    b = _run(dsa, inp, cfg, want_scores=True, workspace=ws)
    assert torch.equal(a[0], b[0])
    assert torch.equal(a[1].view(torch.int32), b[1].view(torch.int32))


def test_prefill_32k_full_size_sampled_rows(dsa):
    """The L=32768 fp8 workload at full size, in the launch configuration the
    benchmark times; oracle on a seeded row sample (with the edge rows)."""
    import torch
    from synth.gpu import DeviceGen
    cfg = gen.CONFIGS["prefill_32k"]
    L, topk = cfg["L"], cfg["topk"]
    note("prefill 32k generate on device")
    g = DeviceGen()
    d = g.prefill_inputs(cfg)
    rows = sample_rows(L, topk, 40, seed=3)
    host_inp = gen.prefill_inputs(cfg, rows=rows)
    # the device generator produced the same bytes as the host one
    assert np.array_equal(host(d["k"]), host_inp["k"])
    assert np.array_equal(host(d["k_scale"]), host_inp["k_scale"])
    assert np.array_equal(host(d["q"][torch.from_numpy(rows).cuda()]), host_inp["q"])
    assert np.array_equal(host(d["w"][torch.from_numpy(rows).cuda()]), host_inp["w"])
    note("prefill 32k kernel")
    idx, sc, _ = dsa.dsa_indexer_topk_prefill(d["q"], d["q_scale"], d["k"], d["k_scale"], d["w"], topk, "fp8",
                                              want_scores=True)
    torch.cuda.synchronize()
    check_structure_all(idx, topk)
    idx_h, sc_h = host(idx), host(sc)
    res = oracle.prefill(host_inp["q"], host_inp["q_scale"], host_inp["k"], host_inp["k_scale"], host_inp["w"],
                         "fp8", topk, rows=rows, return_scores=True)
    _compare(idx_h, sc_h, res, rows, topk)


# Every (dtype, H, D) the library builds: the H >= 32 split-head layout, the
# H = 16 and H = 8 layouts (one and two queries per lane half), and both tile
# sizes.  Ragged L (not a multiple of the 8- to 32-row work item or of a tile).
BUILT = [("fp8", 64, 128), ("fp8", 64, 64), ("fp8", 32, 128), ("fp8", 32, 64), ("fp8", 16, 128),
         ("fp8", 16, 64), ("fp8", 8, 128), ("fp8", 8, 64), ("bf16", 64, 64), ("bf16", 32, 128),
         ("bf16", 32, 64), ("bf16", 16, 128), ("bf16", 16, 64), ("bf16", 8, 128), ("bf16", 8, 64),
         # one wave per SIMD (4 rows per work item)
         ("fp8", 128, 128), ("fp8", 128, 64), ("bf16", 128, 128), ("bf16", 128, 64), ("bf16", 64, 128)]


@pytest.mark.parametrize("dt,H,D", BUILT)
def test_every_built_configuration(dsa, dt, H, D):
    L, topk = 1109, 96
    cfg = dict(kind="prefill", L=L, H=H, D=D, topk=topk, dtype=dt, seed=H + D + (dt == "bf16"),
               heavy_count=11, heavy_factor=3.0, qk_div=8.0, w_div=8.0)
    note(f"prefill configuration {dt} H={H} D={D} L={L} k={topk}")
    inp = gen.prefill_inputs(cfg)
    idx, sc, _ = _run(dsa, inp, cfg, want_scores=True)
    check_structure_all(idx, topk)
    rows = sample_rows(L, topk, 48, seed=H * D)
    _compare(host(idx), host(sc), _oracle_rows(inp, cfg, rows), rows, topk, fmt=dt)


@pytest.mark.parametrize("dt,H,D", [("fp8", 24, 128), ("fp8", 40, 64), ("fp8", 56, 128), ("bf16", 24, 64),
                                     ("bf16", 48, 64), ("fp8", 96, 128), ("bf16", 72, 64)])
def test_head_counts_between_the_built_widths(dsa, dt, H, D):
    """H a multiple of 8 that no kernel is built for runs on the next
    built width with zero heads appended; the caller's [L, H, D] layout is
    read as it is."""
    L, topk = 1109, 96
    cfg = dict(kind="prefill", L=L, H=H, D=D, topk=topk, dtype=dt, seed=5 * H + D + (dt == "bf16"),
               heavy_count=11, heavy_factor=3.0, qk_div=8.0, w_div=8.0)
    note(f"prefill padded head count {dt} H={H} D={D} L={L} k={topk}")
    inp = gen.prefill_inputs(cfg)
    idx, sc, _ = _run(dsa, inp, cfg, want_scores=True)
    check_structure_all(idx, topk)
    rows = sample_rows(L, topk, 48, seed=H * D + 1)
    _compare(host(idx), host(sc), _oracle_rows(inp, cfg, rows), rows, topk, fmt=dt)


@pytest.mark.parametrize("dt,H,D", BUILT)
def test_every_built_configuration_with_key_sample(dsa, dt, H, D):
    """L=5003, k=64: work items from position 2048 (128-key tiles) or 4096
    (256-key tiles) on score a key sample first and filter with its
    threshold, so this covers the sample path of every layout (the query
    slots of H <= 16 included), not only the benchmark's."""
    L, topk = 5003, 64
    cfg = dict(kind="prefill", L=L, H=H, D=D, topk=topk, dtype=dt, seed=3 * H + D + (dt == "bf16"),
               heavy_count=L // 100, heavy_factor=3.0, qk_div=8.0, w_div=8.0)
    note(f"prefill configuration with key sample {dt} H={H} D={D} L={L} k={topk}")
    inp = gen.prefill_inputs(cfg)
    idx, sc, _ = _run(dsa, inp, cfg, want_scores=True)
    check_structure_all(idx, topk)
    around = {2047, 2048, 2049, 2055, 2056, 4095, 4096, 4097, 4103, 4104}
    rows = np.array(sorted(set(sample_rows(L, topk, 20, seed=H + D).tolist()) | around), dtype=np.int64)
    _compare(host(idx), host(sc), _oracle_rows(inp, cfg, rows), rows, topk, fmt=dt)


@pytest.mark.parametrize("dt,H,D,L,topk", [("fp8", 64, 128, 5003, 2048), ("bf16", 16, 64, 1109, 256),
                                          ("fp8", 8, 128, 700, 100)])
def test_without_scores_equals_with_scores(dsa, dt, H, D, L, topk):
    """Without requested scores, a work item whose rows all have t + 1 <= topk
    is answered without scoring: each row keeps every key 0..t.  With finite
    scores that is the selection the scoring path makes, so every row of the
    call equals the call that also returns scores."""
    cfg = dict(kind="prefill", L=L, H=H, D=D, topk=topk, dtype=dt, seed=7 * H + D + (dt == "bf16"),
               heavy_count=L // 100, heavy_factor=3.0, qk_div=8.0, w_div=8.0)
    note(f"prefill without scores {dt} H={H} D={D} L={L} k={topk}")
    inp = gen.prefill_inputs(cfg)
    plain, _, _ = _run(dsa, inp, cfg)
    with_sc, _, _ = _run(dsa, inp, cfg, want_scores=True)
    plain, with_sc = host(plain), host(with_sc)
    assert np.array_equal(plain, with_sc)
    for t in range(min(L, topk)):
        assert plain[t, :t + 1].tolist() == list(range(t + 1)) and np.all(plain[t, t + 1:] == -1), t


@pytest.mark.parametrize("L,topk", [(700, 1), (5003, 4096)])
def test_topk_limits(dsa, L, topk):
    """The smallest k and the largest the library accepts."""
    cfg = dict(gen.CONFIGS["prefill_32k"], L=L, topk=topk, heavy_count=L // 100)
    note(f"prefill topk limit L={L} k={topk}")
    inp = gen.prefill_inputs(cfg)
    idx, sc, _ = _run(dsa, inp, cfg, want_scores=True)
    check_structure_all(idx, topk)
    rows = sample_rows(L, topk, 24, seed=topk)
    _compare(host(idx), host(sc), _oracle_rows(inp, cfg, rows), rows, topk)


@pytest.mark.parametrize("L", [1, 2, 3])
def test_shortest_sequences_select_every_key(dsa, L):
    """L <= k: every row keeps all of its keys 0..t, in order, -1 padded."""
    topk = 2048
    cfg = dict(gen.CONFIGS["prefill_32k"], L=L, topk=topk, heavy_count=0)
    note(f"prefill L={L}")
    inp = gen.prefill_inputs(cfg)
    idx, sc, _ = _run(dsa, inp, cfg, want_scores=True)
    idx, sc = host(idx), host(sc)
    for t in range(L):
        assert idx[t].tolist() == list(range(t + 1)) + [-1] * (topk - t - 1), t
    rows = np.arange(L)
    _compare(idx, sc, _oracle_rows(inp, cfg, rows), rows, topk)


def test_overflowing_scores_still_write_every_row(dsa):
    """Finite but extreme head weights on some rows overflow their scores to
    inf and NaN (mixed signs).  A NaN or -inf score is never selected, so
    such a row may hold fewer than min(k, t+1) keys, but every row is still
    written in full (the sentinel the output starts with is gone, -1 padded),
    and the rows with ordinary weights still match the oracle."""
    import torch
    L, topk = 3000, 64
    cfg = dict(gen.CONFIGS["prefill_32k"], L=L, topk=topk, heavy_count=30)
    note(f"prefill overflowing weights L={L} k={topk}")
    inp = gen.prefill_inputs(cfg)
    w = inp["w"].copy()
    hot = np.arange(1000, 1100)
    big = gen.bf16_bits(np.float32(3.0e38))
    w[hot, 0::2] = big
    w[hot, 1::2] = big | np.uint16(0x8000)       # the same magnitude, negative
    inp = dict(inp, w=w)
    out = torch.full((L, topk), 0x7FFFFFFF, dtype=torch.int32, device="cuda")
    idx, sc, _ = _run(dsa, inp, cfg, want_scores=True, out_idx=out)
    idx = host(idx)
    assert not np.any(idx == 0x7FFFFFFF), "a row was left unwritten"
    for t in hot:
        v = idx[t][idx[t] >= 0]
        m = len(v)
        assert m <= min(topk, t + 1)
        assert np.all(idx[t][m:] == -1) and np.all(v <= t) and np.all(np.diff(v) > 0), t
    rows = np.array(sorted(set(sample_rows(L, topk, 24).tolist()) - set(hot.tolist())), dtype=np.int64)
    _compare(idx, host(sc), _oracle_rows(inp, cfg, rows), rows, topk)
