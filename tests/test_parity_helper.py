"""The parity contract itself, exercised with mistakes planted in oracle outputs."""
import numpy as np

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
