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


def test_exact_copy_passes():
    idx, sc, o, A = _row()
    assert parity.check_row(idx, o, A, 128, g_score=sc.astype(np.float32)) is None


def test_swap_outside_band_fails():
    idx, sc, o, A = _row()
    chosen = set(idx.tolist())
    worst = min((s for s in range(len(o)) if s not in chosen), key=lambda s: o[s])
    bad = np.array(sorted((chosen - {int(idx[0])}) | {worst}))
    assert parity.check_row(bad, o, A, 128) is not None


def test_swap_inside_band_passes():
    idx, sc, o, A = _row()
    n = len(o)
    order = np.lexsort((np.arange(n), -o))
    kth, nxt = order[127], order[128]
    o2 = o.copy()
    o2[nxt] = o2[kth] * (1 - 1e-5)          # make the runner-up a near tie
    alt = np.array(sorted((set(np.sort(order[:128]).tolist()) - {int(kth)}) | {int(nxt)}))
    assert parity.check_row(alt, o2, A, 128) is None


def test_structure_errors():
    idx, sc, o, A = _row()
    assert parity.check_row(idx[::-1], o, A, 128) is not None       # not ascending
    short = np.array(list(range(10)) + [-1] * 118)
    assert parity.check_row(short, o[:10], A[:10], 128) is None
    assert parity.check_row(np.array([0, 1, 2, -1, 4] + [-1] * 123), o[:10], A[:10], 128) is not None


def test_score_tolerance():
    idx, sc, o, A = _row()
    s2 = sc.copy()
    s2[5] += 3e-3 * A[idx[5]]
    assert parity.check_row(idx, o, A, 128, g_score=s2) is not None
    s3 = sc.copy()
    s3[5] += 1e-3 * A[idx[5]]
    assert parity.check_row(idx, o, A, 128, g_score=s3) is None
