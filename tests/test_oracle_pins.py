"""Pins of the fp64 oracle against things other than itself.

Each test checks the oracle against a fact fixed by the pages or by the
mathematics, not by retyping its own formula: the storage formats against
torch's float8/bfloat16, a hand-worked 4-token example, closed-form selection
families, brute-force ranking, and algebraic identities of the score that a
dropped ReLU, a wrong sign, a swapped head/key index or a transposed operand
would break.
"""
import json
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
from synth import gen

HERE = os.path.dirname(os.path.abspath(__file__))


# ----------------------------------------------------------------------------
# formats
# ----------------------------------------------------------------------------

def test_e4m3_decoder_all_codes_vs_torch():
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], dtype=np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).float().numpy().astype(np.float64)
    got = oracle.dec_e4m3(codes)
    np.testing.assert_array_equal(got, ref)
    assert np.array_equal(np.signbit(got), np.signbit(ref))


def test_e4m3_decoder_spec_points_and_nan():
    d = oracle.dec_e4m3
    assert d([0x7E])[0] == 448.0 and d([0xFE])[0] == -448.0
    assert d([0x01])[0] == 2.0**-9 and d([0x07])[0] == 7 * 2.0**-9
    assert d([0x08])[0] == 2.0**-6 and d([0x38])[0] == 1.0
    for c in (0x7F, 0xFF):
        with pytest.raises(ValueError):
            d([c])


def test_bf16_decoder_vs_torch():
    rng = np.random.default_rng(0)
    bits = rng.integers(0, 2**16, 50000).astype(np.uint16)
    bits = bits[((bits >> 7) & 0xFF) != 0xFF]          # finite only
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).double().numpy()
    np.testing.assert_array_equal(oracle.dec_bf16(bits), ref)


# ----------------------------------------------------------------------------
# hand-worked example
# ----------------------------------------------------------------------------

def _hand():
    with open(os.path.join(HERE, "golden", "hand_4token.json")) as f:
        return json.load(f)


@pytest.mark.parametrize("fmt", ["bf16", "fp8"])
def test_hand_example_scores_and_sets(fmt):
    g = _hand()
    q = np.array(g["q"], dtype=np.float32)
    w = np.array(g["w"], dtype=np.float32)
    enc = gen.bf16_bits if fmt == "bf16" else gen.e4m3_bits
    for layer in g["layers"]:
        k = np.array(layer["k"], dtype=np.float32)
        ones = np.ones(4, dtype=np.float32) if fmt == "fp8" else None
        res = oracle.prefill(enc(q), ones, enc(k), ones, gen.bf16_bits(w), fmt, g["topk"],
                             rows=range(4), return_scores=True)
        for t in range(4):
            np.testing.assert_array_equal(res["o"][t], np.array(layer["scores"][t], dtype=np.float64))
        np.testing.assert_array_equal(res["idx"], np.array(layer["idx"]))


def test_hand_example_fs_and_overlap():
    g = _hand()
    q = gen.bf16_bits(np.array(g["q"], dtype=np.float32))
    w = gen.bf16_bits(np.array(g["w"], dtype=np.float32))
    per_layer = [oracle.prefill(q, None, gen.bf16_bits(np.array(L["k"], dtype=np.float32)), None, w,
                                "bf16", g["topk"], rows=range(4))["idx"] for L in g["layers"]]
    outs, src, calls = oracle.fs_run(g["fs_pattern"], lambda l: per_layer[l])
    assert src == g["fs_src"] and calls == 2
    assert outs[1] is outs[0]
    np.testing.assert_array_equal(outs[2], np.array(g["layers"][2]["idx"]))
    C = oracle.overlap_counts(per_layer, g["overlap_rows"])
    np.testing.assert_array_equal(C, np.array(g["overlap_counts"], dtype=np.uint64))
    R = oracle.overlap_ratio(C, g["topk"], len(g["overlap_rows"]))
    assert np.all(np.diag(R) == 1.0)


# ----------------------------------------------------------------------------
# selection: closed forms and brute force
# ----------------------------------------------------------------------------

def _ramp_problem(L, H, w_sign, zero_q=False):
    """q[t,h] = e_0 for every head, k[s] = (s+1) e_0, so score(t,s) = (sum_h w[t,h]) * (s+1)."""
    D = 8
    q = np.zeros((L, H, D), dtype=np.float32)
    if not zero_q:
        q[:, :, 0] = 1.0
    k = np.zeros((L, D), dtype=np.float32)
    k[:, 0] = np.arange(1, L + 1)
    rng = np.random.default_rng(3)
    w = rng.uniform(0.1, 1.0, size=(L, H)).astype(np.float32) * w_sign
    return gen.bf16_bits(q), gen.bf16_bits(k), gen.bf16_bits(w)


@pytest.mark.parametrize("topk", [1, 5, 16, 40])
def test_selection_closed_forms(topk):
    L, H = 48, 4
    for w_sign, zero_q, expect in [
        (+1, False, lambda t: list(range(max(0, t - topk + 1), t + 1))),   # increasing scores: last k
        (-1, False, lambda t: list(range(0, min(topk, t + 1)))),           # decreasing scores: first k
        (+1, True, lambda t: list(range(0, min(topk, t + 1)))),            # all zero: ties -> lowest
    ]:
        q, k, w = _ramp_problem(L, H, w_sign, zero_q)
        res = oracle.prefill(q, None, k, None, w, "bf16", topk, rows=range(L))
        for t in range(L):
            e = expect(t)
            assert res["idx"][t].tolist() == e + [-1] * (topk - len(e))


def _brute_select(o, k):
    """s is chosen iff fewer than k keys beat it (higher score, or equal score and lower index)."""
    n = len(o)
    chosen = []
    for s in range(n):
        better = sum(1 for u in range(n) if o[u] > o[s] or (o[u] == o[s] and u < s))
        if better < k:
            chosen.append(s)
    return chosen


def test_selection_brute_force_all_k():
    rng = np.random.default_rng(4)
    for n in [1, 2, 3, 7, 20, 33]:
        for trial in range(3):
            o = rng.integers(-3, 4, size=n).astype(np.float64)   # many ties
            if trial == 2:
                o = rng.standard_normal(n)
            for k in range(1, n + 3):
                idx, sc = oracle.select_topk(o, k)
                want = _brute_select(list(o), k)
                assert idx.tolist() == want + [-1] * (k - len(want))
                np.testing.assert_array_equal(sc[:len(want)], o[want])
                assert np.all(np.isneginf(sc[len(want):]))


def test_selection_negative_zero_ties_positive_zero():
    o = np.array([0.0, -0.0, 0.0, -1.0])
    idx, _ = oracle.select_topk(o, 2)
    assert idx.tolist() == [0, 1]


# ----------------------------------------------------------------------------
# score identities
# ----------------------------------------------------------------------------

def _rand_fp8_problem(L=40, H=6, D=16, seed=5):
    rng = np.random.default_rng(seed)
    Q = rng.standard_normal((L, H, D)).astype(np.float32)
    K = rng.standard_normal((L, D)).astype(np.float32)
    q, qs = gen.quant_rows_e4m3(Q)
    k, ks = gen.quant_rows_e4m3(K)
    w = gen.bf16_bits(rng.standard_normal((L, H)).astype(np.float32))
    return q, qs, k, ks, w


def _scores(q, qs, k, ks, w, rows, fmt="fp8"):
    """Scores of token rows ``rows``; q, q-scale and w are given for all tokens."""
    rows = list(rows)
    res = oracle.prefill(q[rows], None if qs is None else qs[rows], k, ks, w[rows], fmt, 4,
                         rows=rows, return_scores=True)
    return res["o"], res["A"]


def test_relu_identity_linear_part():
    """o(q) - o(-q) = sum_h w_h (q_h . k), because ReLU(x) - ReLU(-x) = x.
    The right side is evaluated with exact rationals, one term at a time."""
    q, qs, k, ks, w = _rand_fp8_problem()
    neg = q ^ np.uint8(0x80)                       # flip the sign bit of every code
    rows = [0, 7, 39]
    o_pos, _ = _scores(q, qs, k, ks, w, rows)
    o_neg, _ = _scores(neg, qs, k, ks, w, rows)
    qd = oracle.dec_e4m3(q)
    kd = oracle.dec_e4m3(k)
    wd = oracle.dec_bf16(w)
    for r, t in enumerate(rows):
        for s in range(t + 1):
            lin = Fraction(0)
            for h in range(q.shape[1]):
                dot = sum(Fraction(float(qd[t, h, i])) * Fraction(float(kd[s, i])) for i in range(q.shape[2]))
                lin += Fraction(float(wd[t, h])) * dot
            lin *= Fraction(float(qs[t])) * Fraction(float(ks[s]))
            assert abs(o_pos[r][s] - o_neg[r][s] - float(lin)) <= 1e-12 * (1 + abs(float(lin)))


def test_relu_gate_nonnegative_with_nonnegative_weights():
    q, qs, k, ks, _ = _rand_fp8_problem()
    w = gen.bf16_bits(np.abs(np.random.default_rng(6).standard_normal((40, 6))).astype(np.float32))
    o, _ = _scores(q, qs, k, ks, w, range(40))
    assert all(np.all(x >= 0) for x in o)
    # and some scores are strictly positive while some head dots are negative
    assert sum(np.count_nonzero(x) for x in o) > 100


def test_single_head_unit_weight_is_relu_gemv():
    """H=1, w=1: the score is max(q.k_s, 0), a ReLU of a matrix-vector product."""
    rng = np.random.default_rng(7)
    Q = rng.standard_normal((30, 1, 12)).astype(np.float32)
    K = rng.standard_normal((30, 12)).astype(np.float32)
    q, k = gen.bf16_bits(Q), gen.bf16_bits(K)
    w = gen.bf16_bits(np.ones((30, 1), dtype=np.float32))
    o, _ = _scores(q, None, k, None, w, range(30), fmt="bf16")
    Kt = torch.from_numpy(k.view(np.int16)).view(torch.bfloat16).double()
    Qt = torch.from_numpy(q.view(np.int16)).view(torch.bfloat16).double()
    for t in range(30):
        ref = torch.relu(torch.mv(Kt[: t + 1], Qt[t, 0])).numpy()
        np.testing.assert_allclose(o[t], ref, rtol=0, atol=1e-12)


def test_head_permutation_invariance():
    q, qs, k, ks, w = _rand_fp8_problem()
    perm = np.random.default_rng(8).permutation(q.shape[1])
    o1, _ = _scores(q, qs, k, ks, w, range(40))
    o2, _ = _scores(q[:, perm], qs, k, ks, w[:, perm], range(40))
    for a, b in zip(o1, o2):
        np.testing.assert_allclose(a, b, rtol=1e-13, atol=1e-13)


def test_key_order_not_head_order():
    """Permuting the keys permutes the scores (key index and head index are not mixed up)."""
    q, qs, k, ks, w = _rand_fp8_problem(L=24)
    t = 23
    perm = np.random.default_rng(9).permutation(24)
    o1, _ = _scores(q, qs, k, ks, w, [t])
    o2, _ = _scores(q, qs, k[perm], ks[perm], w, [t])
    np.testing.assert_allclose(o2[0], o1[0][perm], rtol=1e-13, atol=1e-13)


def test_positive_scaling_equivariance():
    q, qs, k, ks, w = _rand_fp8_problem()
    o1, A1 = _scores(q, qs, k, ks, w, range(40))
    o2, _ = _scores(q, qs * np.float32(4), k, ks, w, range(40))
    o3, _ = _scores(q, qs, k, ks * np.float32(0.5), w, range(40))
    w2 = gen.bf16_bits(oracle.dec_bf16(w).astype(np.float32) * np.float32(2))
    o4, _ = _scores(q, qs, k, ks, w2, range(40))
    for a, b, c, d, m in zip(o1, o2, o3, o4, A1):
        np.testing.assert_allclose(b, 4 * a, rtol=1e-13, atol=1e-13)
        np.testing.assert_allclose(c, 0.5 * a, rtol=1e-13, atol=1e-13)
        np.testing.assert_allclose(d, 2 * a, rtol=1e-13, atol=1e-13)
        assert np.all(np.abs(a) <= m * (1 + 1e-12))


def test_per_head_scale_equals_per_token_scale():
    q, qs, k, ks, w = _rand_fp8_problem()
    qs2 = np.repeat(qs[:, None], q.shape[1], axis=1)
    o1, _ = _scores(q, qs, k, ks, w, range(40))
    o2, _ = _scores(q, qs2, k, ks, w, range(40))
    for a, b in zip(o1, o2):
        np.testing.assert_array_equal(a, b)


def test_causal_prefix_only():
    q, qs, k, ks, w = _rand_fp8_problem()
    res = oracle.prefill(q, qs, k, ks, w, "fp8", 8, rows=range(40))
    for t in range(40):
        row = res["idx"][t]
        valid = row[row >= 0]
        assert len(valid) == min(8, t + 1)
        assert np.all(valid <= t) and np.all(np.diff(valid) > 0)
        assert np.all(row[len(valid):] == -1)


def test_decode_equals_prefill_last_row():
    rng = np.random.default_rng(10)
    B, Lmax, H, D = 3, 50, 4, 16
    cache, ks = gen.quant_rows_e4m3(rng.standard_normal((B * Lmax, D)).astype(np.float32))
    cache = cache.reshape(B, Lmax, D)
    ks = ks.reshape(B, Lmax)
    q = gen.bf16_bits(rng.standard_normal((B, H, D)).astype(np.float32))
    w = gen.bf16_bits(rng.standard_normal((B, H)).astype(np.float32))
    lens = np.array([50, 17, 1])
    dec = oracle.decode(q, w, cache, ks, lens, 6)
    for b in range(B):
        n = lens[b]
        # a prefill whose row n-1 carries the decode query sees the same keys
        pre = oracle.prefill(q[b][None], None, cache[b, :n], ks[b, :n], w[b][None], "bf16", 6,
                             rows=[n - 1], k_fmt="fp8")
        np.testing.assert_array_equal(dec["idx"][b], pre["idx"][0])
        np.testing.assert_array_equal(dec["score"][b], pre["score"][0])


# ----------------------------------------------------------------------------
# layer-reuse schedule
# ----------------------------------------------------------------------------

def test_fs_resolve_tables():
    p = gen.FS_PATTERNS
    assert oracle.fs_resolve(p["all_F"], 47) == list(range(47))
    assert oracle.fs_resolve(p["uniform_1_4"], 47) == [4 * (l // 4) for l in range(47)]
    src = oracle.fs_resolve(p["searched_1_4"], 47)
    fl = [0, 2, 4, 9, 13, 16, 17, 20, 23, 28, 32, 37]
    assert [l for l in range(47) if src[l] == l] == fl
    runs = [fl[i + 1] - fl[i] - 1 for i in range(len(fl) - 1)] + [46 - fl[-1]]
    assert [r for r in runs if r] == [1, 1, 4, 3, 2, 2, 2, 4, 3, 4, 9]
    for l in range(47):
        assert src[l] == max(j for j in range(l + 1) if p["searched_1_4"][j] == "F")


@pytest.mark.parametrize("bad", ["SFF", "FXF", "", "FF"])
def test_fs_resolve_rejects(bad):
    with pytest.raises(ValueError):
        oracle.fs_resolve(bad, 3)


def test_fs_run_reuses_source_output():
    seen = []
    outs, src, calls = oracle.fs_run("FSSFS", lambda l: (seen.append(l), np.full((2, 2), l))[1])
    assert seen == [0, 3] and calls == 2 and src == [0, 0, 0, 3, 3]
    assert outs[1] is outs[0] and outs[2] is outs[0] and outs[4] is outs[3]


def test_greedy_search_additive_loss_closed_form():
    """With loss = sum of a fixed cost per S layer, the greedy search turns
    layers into S in increasing cost order (the first layer never)."""
    rng = np.random.default_rng(8)
    N = 12
    cost = rng.permutation(N).astype(float) + 0.5
    loss = lambda p: sum(cost[l] for l, c in enumerate(p) if c == "S")
    pat, trace, flipped = oracle.fs_greedy_search(N, N - 1, loss)
    order = [int(l) for l in np.argsort(cost) if l != 0]
    assert flipped == order and pat == "F" + "S" * (N - 1)
    assert trace == [0.0] + list(np.cumsum([cost[l] for l in order]))
    pat9, _, _ = oracle.fs_greedy_search(N, 9, loss)
    assert pat9.count("F") == 3 and pat9[0] == "F"


def test_greedy_search_evaluation_count_matches_report():
    """A full run (N-1 steps) evaluates N(N-1)/2 trial patterns, the count the
    deep-dive report gives for the full greedy search, plus the all-F start."""
    for N in (2, 5, 47):
        seen = []
        oracle.fs_greedy_search(N, N - 1, lambda p: (seen.append(p), 0.0)[1])
        assert len(seen) == 1 + N * (N - 1) // 2
        assert seen[0] == "F" * N and all(p[0] == "F" for p in seen)


def test_greedy_search_ties_and_hand_traced_interaction():
    # a constant loss: every tie goes to the lowest layer
    assert oracle.fs_greedy_search(6, 4, lambda p: 1.0)[2] == [1, 2, 3, 4]
    # a hand-made table where the greedy first step blocks the best pair:
    # FSFF is the best single flip, but FFSS is the best pair
    table = {"FFFF": 0.0, "FSFF": 1.0, "FFSF": 2.0, "FFFS": 2.0, "FSSF": 5.0, "FSFS": 5.0, "FFSS": 1.5,
             "FSSS": 9.0}
    pat, trace, flipped = oracle.fs_greedy_search(4, 2, lambda p: table[p])
    assert (pat, trace, flipped) == ("FSSF", [0.0, 1.0, 5.0], [1, 2])
    with pytest.raises(ValueError):
        oracle.fs_greedy_search(4, 4, lambda p: 0.0)


def test_overlap_proxy_closed_form():
    R = np.array([[1.0, 0.8, 0.5, 0.4], [0.8, 1.0, 0.7, 0.6], [0.5, 0.7, 1.0, 0.9], [0.4, 0.6, 0.9, 1.0]])
    assert oracle.overlap_proxy_loss("FFFF", R) == 0.0
    # FSFS: layer 1 reuses 0 (lost 0.2), layer 3 reuses 2 (lost 0.1)
    assert abs(oracle.overlap_proxy_loss("FSFS", R) - 0.3 / 4) < 1e-15
    # FSSS: layers 1, 2, 3 all reuse 0: lost 0.2 + 0.5 + 0.6
    assert abs(oracle.overlap_proxy_loss("FSSS", R) - 1.3 / 4) < 1e-15


def test_mli_resolve_tables():
    """Lagged schedule, written out by hand from its rule: an F layer attends
    the previous F layer's selection, an S layer the nearest earlier F layer's,
    the first layer its own."""
    assert oracle.mli_resolve("F") == [0]
    assert oracle.mli_resolve("FSFFS") == [0, 0, 0, 2, 3]
    assert oracle.mli_resolve("FFSSF") == [0, 0, 1, 1, 1]
    p = gen.FS_PATTERNS
    assert oracle.mli_resolve(p["all_F"]) == [0] + list(range(46))
    assert oracle.mli_resolve(p["uniform_1_4"]) == [0] + [4 * ((l - 1) // 4) for l in range(1, 47)]
    fl = [0, 2, 4, 9, 13, 16, 17, 20, 23, 28, 32, 37]
    src = oracle.mli_resolve(p["searched_1_4"])
    assert [src[f] for f in fl] == [0] + fl[:-1]                 # each F layer lags one F layer
    fs = oracle.fs_resolve(p["searched_1_4"])
    assert all(src[l] == fs[l] for l in range(47) if l not in fl)  # S layers as in IndexCache
    for bad in ["SFF", "FXF", ""]:
        with pytest.raises(ValueError):
            oracle.mli_resolve(bad)


def test_mli_run_lags_f_layers():
    seen = []
    outs, asrc, calls = oracle.mli_run("FSFFS", lambda l: (seen.append(l), np.full((2, 2), l))[1])
    assert seen == [0, 2, 3] and calls == 3 and asrc == [0, 0, 0, 2, 3]
    assert outs[0] is outs[1] and outs[2] is outs[0] and int(outs[3][0, 0]) == 2 and int(outs[4][0, 0]) == 3


def test_hand_example_lagged_schedule():
    """FSF on the hand example: layer 2 attends layer 0's sets (its own, L2's,
    differ at t = 3) and layer 0 attends its own."""
    g = _hand()
    q = gen.bf16_bits(np.array(g["q"], dtype=np.float32))
    w = gen.bf16_bits(np.array(g["w"], dtype=np.float32))
    per_layer = [oracle.prefill(q, None, gen.bf16_bits(np.array(L["k"], dtype=np.float32)), None, w,
                                "bf16", g["topk"], rows=range(4))["idx"] for L in g["layers"]]
    outs, asrc, calls = oracle.mli_run(g["fs_pattern"], lambda l: per_layer[l])
    assert asrc == [0, 0, 0] and calls == 2
    np.testing.assert_array_equal(outs[2], np.array(g["layers"][0]["idx"]))
    assert not np.array_equal(outs[2], np.array(g["layers"][2]["idx"]))


# ----------------------------------------------------------------------------
# stand-in attention
# ----------------------------------------------------------------------------

def _latent(rng, B, Lmax):
    return gen.bf16_bits((rng.standard_normal((B, Lmax, 576)) / 4).astype(np.float32))


def test_standin_attention_zero_query_is_mean_of_values():
    rng = np.random.default_rng(3)
    lat = _latent(rng, 2, 50)
    sel = np.array([[3, 7, 11, -1], [0, 49, -1, -1]])
    out = oracle.standin_attention(np.zeros((2, 576), dtype=np.uint16), lat, sel, 0.7)
    for b in range(2):
        rows = [s for s in sel[b] if s >= 0]
        want = sum(oracle.dec_bf16(lat[b, s, :512]) for s in rows) / len(rows)
        np.testing.assert_allclose(out[b], want, rtol=0, atol=1e-15)


def test_standin_attention_two_rows_weights_three_to_one():
    """Scores differing by ln 3 weight the rows 3/4 and 1/4."""
    rng = np.random.default_rng(4)
    lat = _latent(rng, 1, 4)
    lat[0, :, 0] = gen.bf16_bits(np.array([1.0, 0.0, 0.5, 0.5], dtype=np.float32))
    q = np.zeros((1, 576), dtype=np.uint16)
    q[0, 0] = gen.bf16_bits(np.array([1.0], dtype=np.float32))[0]
    out = oracle.standin_attention(q, lat, np.array([[0, 1]]), float(np.log(3.0)))
    v = oracle.dec_bf16(lat[0, :2, :512])
    np.testing.assert_allclose(out[0], 0.75 * v[0] + 0.25 * v[1], rtol=0, atol=1e-14)


def test_standin_attention_invariances_and_limits():
    rng = np.random.default_rng(5)
    B, Lmax = 3, 64
    lat = _latent(rng, B, Lmax)
    q = gen.bf16_bits((rng.standard_normal((B, 576)) / 4).astype(np.float32))
    sel = np.stack([np.sort(rng.choice(Lmax, 8, replace=False)) for _ in range(B)])
    base = oracle.standin_attention(q, lat, sel, 0.3)
    # order of the selection does not matter; padding and out-of-range entries are skipped
    perm = sel[:, ::-1].copy()
    np.testing.assert_allclose(oracle.standin_attention(q, lat, perm, 0.3), base, rtol=1e-13, atol=1e-15)
    padded = np.concatenate([sel, np.full((B, 3), -1), np.full((B, 1), Lmax + 5)], axis=1)
    np.testing.assert_allclose(oracle.standin_attention(q, lat, padded, 0.3), base, rtol=1e-13, atol=1e-15)
    assert np.all(oracle.standin_attention(q, lat, np.full((B, 4), -1), 0.3) == 0.0)
    # a dimension on which every latent row agrees shifts all scores equally
    lat2, q2 = lat.copy(), q.copy()
    lat2[:, :, 575] = gen.bf16_bits(np.array([2.0], dtype=np.float32))[0]
    q2[:, 575] = gen.bf16_bits(np.array([3.0], dtype=np.float32))[0]
    lat_ref = lat.copy()
    lat_ref[:, :, 575] = 0
    np.testing.assert_allclose(oracle.standin_attention(q2, lat2, sel, 0.3),
                               oracle.standin_attention(q, lat_ref, sel, 0.3), rtol=1e-12, atol=1e-14)
    # a very large scale picks the value of the highest-scoring row
    hard = oracle.standin_attention(q, lat, sel, 1e4)
    for b in range(B):
        d = [float(oracle.dec_bf16(lat[b, s]) @ oracle.dec_bf16(q[b])) for s in sel[b]]
        np.testing.assert_allclose(hard[b], oracle.dec_bf16(lat[b, sel[b][int(np.argmax(d))], :512]), atol=1e-12)


# ----------------------------------------------------------------------------
# overlap
# ----------------------------------------------------------------------------

def test_overlap_closed_form_suffix_vs_prefix():
    """Last-k sets against first-k sets overlap in max(0, 2k - t - 1) keys at row t."""
    L, k = 40, 8
    suf = np.array([list(range(max(0, t - k + 1), t + 1)) + [-1] * (k - min(k, t + 1)) for t in range(L)])
    pre = np.array([list(range(min(k, t + 1))) + [-1] * (k - min(k, t + 1)) for t in range(L)])
    rows = range(k - 1, L)
    C = oracle.overlap_counts([suf, pre], rows)
    assert C[0, 1] == C[1, 0] == sum(max(0, 2 * k - t - 1) for t in rows)
    assert C[0, 0] == C[1, 1] == k * len(rows)


def test_overlap_random_sets_brute_force():
    rng = np.random.default_rng(11)
    N, L, k = 5, 30, 6
    layers = []
    for _ in range(N):
        rowsets = []
        for t in range(L):
            n = min(k, t + 1)
            s = np.sort(rng.choice(t + 1, size=n, replace=False))
            rowsets.append(list(s) + [-1] * (k - n))
        layers.append(np.array(rowsets))
    rows = list(range(k - 1, L))
    C = oracle.overlap_counts(layers, rows)
    for i in range(N):
        for j in range(N):
            want = sum(len(set(layers[i][t][layers[i][t] >= 0]) & set(layers[j][t][layers[j][t] >= 0])) for t in rows)
            assert C[i, j] == want
    assert np.array_equal(C, C.T)
    R = oracle.overlap_ratio(C, k, len(rows))
    assert np.all(np.diag(R) == 1.0)
    Cs = oracle.overlap_counts([layers[0]] * 3, rows)
    assert np.all(oracle.overlap_ratio(Cs, k, len(rows)) == 1.0)
