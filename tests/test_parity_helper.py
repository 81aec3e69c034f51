"""The parity contract itself, exercised with mistakes planted in oracle outputs."""
import numpy as np
import pytest

import oracle
from synth import gen
from tests import parity


def _row():
    inp = gen.prefill_inputs(gen.CONFIGS["tiny"], rows=[1500])
    res = oracle.prefill(inp["q"], None, inp["k"], None, inp["w"], "bf16", 128, rows=[1500],
                         return_scores=True)
    return res["idx"][0], res["score"][0], res["o"][0], res["A"][0]


def _kth(o, k):
    order = np.lexsort((np.arange(len(o)), -o))
    return order, order[k - 1], order[k]


def test_exact_copy_passes():
    idx, sc, o, A = _row()
    assert parity.check_row(idx, o, A, 128, g_score=sc.astype(np.float32)) is None


def test_swap_outside_band_fails():
    idx, sc, o, A = _row()
    chosen = set(idx.tolist())
    worst = min((s for s in range(len(o)) if s not in chosen), key=lambda s: o[s])
    bad = np.array(sorted((chosen - {int(idx[0])}) | {worst}))
    assert parity.check_row(bad, o, A, 128) is not None


def _swapped(o, k, rel):
    """A selection that trades the k-th key for the runner-up, with the
    runner-up's score set to tau * (1 - rel)."""
    order, kth, nxt = _kth(o, k)
    o2 = o.copy()
    o2[nxt] = o2[kth] * (1 - rel) if o2[kth] > 0 else o2[kth] * (1 + rel)
    alt = np.array(sorted((set(np.sort(order[:k]).tolist()) - {int(kth)}) | {int(nxt)}))
    return alt, o2


def test_swap_inside_strict_band_passes_without_floor():
    idx, sc, o, A = _row()
    alt, o2 = _swapped(o, 128, 5e-4)
    parity.reset_stats()
    # A small enough that the rounding floor is far below the band
    assert parity.check_row(alt, o2, np.full_like(A, 1e-6), 128, fmt="bf16") is None
    assert parity.STATS["floor_rows"] == 0


def test_swap_just_outside_strict_band_fails_when_rounding_cannot_explain_it():
    idx, sc, o, A = _row()
    alt, o2 = _swapped(o, 128, 2e-3)
    assert parity.check_row(alt, o2, np.full_like(A, 1e-6), 128, fmt="bf16") is not None


def test_swap_explained_by_rounding_is_floor_decided_and_counted():
    idx, sc, o, A = _row()
    order, kth, _ = _kth(o, 128)
    tau = abs(o[kth])
    alt, o2 = _swapped(o, 128, 2e-3)
    # a magnitude whose rounding bound covers a 2e-3 relative gap on each side
    bigA = np.full_like(A, 2e-3 * tau / parity.fp32_error_bound(1.0, fmt="bf16"))
    parity.reset_stats()
    assert parity.check_row(alt, o2, bigA, 128, row_id=7, fmt="bf16") is None
    assert parity.STATS["floor_rows"] == 1
    assert parity.take_floor_rows()[0][0] == 7


def test_error_bound_value():
    # bf16: (D + H + 4) u with the 1% margin; fp8 adds the matrix-core group loss 7 * 2^-13
    assert np.isclose(parity.fp32_error_bound(1.0, fmt="bf16"), 1.01 * 196 * 2.0 ** -24)
    assert np.isclose(parity.fp32_error_bound(1.0, terms=72, fmt="bf16"), 1.01 * 76 * 2.0 ** -24)
    assert np.isclose(parity.fp32_error_bound(1.0), 7 * 2.0 ** -13 + 1.01 * 196 * 2.0 ** -24)


def test_structure_errors():
    idx, sc, o, A = _row()
    assert parity.check_row(idx[::-1], o, A, 128) is not None       # not ascending
    short = np.array(list(range(10)) + [-1] * 118)
    assert parity.check_row(short, o[:10], A[:10], 128) is None
    assert parity.check_row(np.array([0, 1, 2, -1, 4] + [-1] * 123), o[:10], A[:10], 128) is not None


def test_score_tolerance_relative_to_the_score():
    idx, sc, o, A = _row()
    og, Ag = o[idx], A[idx]
    j = int(np.argmax(np.abs(og) / Ag))          # a key with |o| well above 0.1 A
    assert abs(og[j]) >= 0.1 * Ag[j]
    s2 = sc.copy()
    s2[j] = og[j] * (1 + 2.5e-3)
    assert parity.check_row(idx, o, A, 128, g_score=s2) is not None
    s3 = sc.copy()
    s3[j] = og[j] * (1 + 1.5e-3)
    assert parity.check_row(idx, o, A, 128, g_score=s3) is None


def test_score_tolerance_near_zero_scores():
    idx, sc, o, A = _row()
    # a short row (every key selected), one key's exact score cancelling to 0
    n = 10
    o2, A2 = o[:n].copy(), A[:n]
    o2[3] = 0.0
    g = np.array(list(range(n)) + [-1] * 118)
    s2 = np.concatenate([o2, np.full(118, -np.inf)])
    s2[3] = 1.5e-4 * A2[3]                         # inside 2e-3 * 0.1 A
    assert parity.check_row(g, o2, A2, 128, g_score=s2) is None
    s2[3] = 2.5e-4 * A2[3]
    assert parity.check_row(g, o2, A2, 128, g_score=s2) is not None


def test_dense_check_uses_the_same_score_rule():
    idx, sc, o, A = _row()
    n = len(o)
    row = np.concatenate([o, np.full(4, -np.inf)])
    assert parity.check_dense(row, o, A) is None
    j = int(np.argmax(np.abs(o) / A))
    bad = row.copy()
    bad[j] = o[j] * (1 + 2.5e-3)
    assert parity.check_dense(bad, o, A) is not None
    bad = row.copy()
    bad[n] = 0.0                                   # a masked key must stay -inf
    assert parity.check_dense(bad, o, A) is not None


def _e4m3_round(v):
    """Nearest OCP e4m3 value of v (|v| <= 448), ties to even, in float64:
    a grid of 2^-9 below 2^-6, else 3 mantissa bits at v's exponent."""
    a = np.abs(v)
    ulp = np.where(a < 2.0 ** -6, 2.0 ** -9, np.exp2(np.floor(np.log2(np.maximum(a, 2.0 ** -6))) - 3))
    return np.sign(v) * np.round(a / ulp) * ulp


def _limb(v):
    """One limb of a block (rows of v): e4m3 values on the grid 2^e set by the
    block maximum m (m 2^-e in (224, 448]); blocks with m < 2^-100 give 0."""
    m = np.max(np.abs(v), axis=1, keepdims=True)
    E = np.floor(np.log2(np.maximum(m, 2.0 ** -100)))
    e = np.where(m / np.exp2(E) <= 1.75, E - 8, E - 7)
    out = _e4m3_round(v * np.exp2(-e)) * np.exp2(e)
    return np.where(m >= 2.0 ** -100, out, 0.0)


def test_fp8q_query_split_limits():
    """The two-limb split of a bf16 query block that the fp8q bound assumes:
    loss <= 2^-22 of the block maximum, none when the block spans <= 2^14,
    and limb magnitudes <= 1.125 |q| + 2^-16 max |q|."""
    rng = np.random.default_rng(3)
    n = 6000
    spread = np.concatenate([np.zeros(n // 3), rng.uniform(1, 14, n // 3), rng.uniform(14, 40, n - 2 * (n // 3))])
    x = rng.standard_normal((n, 32)) * np.exp2(rng.uniform(0, 1, (n, 32)) * spread[:, None] - spread[:, None] / 2)
    x *= np.exp2(rng.integers(-60, 60, (n, 1)).astype(np.float64))
    u = x.astype(np.float32).view(np.uint32)
    q = ((u + 0x7FFF + ((u >> 16) & 1)) & 0xFFFF0000).astype(np.uint32).view(np.float32).astype(np.float64)
    l0 = _limb(q)
    l1 = _limb(q - l0)
    m = np.max(np.abs(q), axis=1, keepdims=True)
    err = np.abs(l0 + l1 - q)
    assert np.all(err <= 2.0 ** -22 * m)
    nz = np.where(q != 0, np.abs(q), np.inf)
    narrow = (m[:, 0] <= 2.0 ** 14 * np.min(nz, axis=1))
    assert narrow.sum() > n // 3 and np.all(err[narrow] == 0)
    assert np.all(np.abs(l0) + np.abs(l1) <= 1.125 * np.abs(q) + 2.0 ** -16 * m)
    assert np.max(err / m) > 2.0 ** -30          # the wide blocks do lose bits


def test_fp8q_bound_terms():
    assert np.isclose(parity.fp32_error_bound(1.0, fmt="fp8q", M=0.0),
                      1.125 * (7 * 2.0 ** -13 + 1.01 * 196 * 2.0 ** -24))
    assert np.isclose(parity.fp32_error_bound(0.0, fmt="fp8q", M=1.0), 2.0 ** -21)
    with pytest.raises(ValueError):
        parity.fp32_error_bound(1.0, fmt="fp8q")
