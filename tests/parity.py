"""Comparison of device results with the fp64 oracle.

Contract
--------
* Scores: |g - o| <= 2e-3 * A(t, s), where A = sum_h |w_h| sum_i |q_h,i k_s,i| is
  the magnitude that bounds the rounding error of any evaluation order (a bare
  |o| denominator is ill-conditioned where heads cancel and o is near 0).
* Top-k sets: with tau the oracle's k-th score of the row, the band
  B = {s : |o(s) - tau| <= max(1e-3 |tau|, 1e-4 A(s))} holds the keys whose
  order fp32 rounding may legitimately change.  A row passes when both sets
  have min(k, n) members and they agree outside B.
* Structure: ascending, distinct, causal (< n), -1 only in the tail.
"""
from __future__ import annotations

import numpy as np

SCORE_RTOL = 2e-3
BAND_REL = 1e-3
BAND_ABS_A = 1e-4


def check_structure(g_idx: np.ndarray, n: int, k: int) -> str | None:
    g = np.asarray(g_idx)
    m = min(k, n)
    if g.shape[0] != k:
        return f"row length {g.shape[0]} != {k}"
    if not np.all(g[m:] == -1):
        return "padding is not -1"
    v = g[:m]
    if np.any(v < 0) or np.any(v >= n):
        return "index out of the causal range"
    if m > 1 and not np.all(np.diff(v) > 0):
        return "indices not strictly ascending"
    return None


def check_row(g_idx, o, A, k, g_score=None) -> str | None:
    """Returns None when the device row matches the oracle row, else a reason."""
    o = np.asarray(o, dtype=np.float64)
    A = np.asarray(A, dtype=np.float64)
    n = len(o)
    err = check_structure(g_idx, n, k)
    if err:
        return err
    m = min(k, n)
    g = np.asarray(g_idx[:m], dtype=np.int64)
    order = np.lexsort((np.arange(n), -o))
    O = np.sort(order[:m])
    if m == n:
        if not np.array_equal(g, O):
            return "short row must select every key"
    else:
        tau = o[order[m - 1]]
        band = np.abs(o - tau) <= np.maximum(BAND_REL * abs(tau), BAND_ABS_A * A)
        gs = set(g.tolist())
        os_ = set(O.tolist())
        diff = gs.symmetric_difference(os_)
        bad = [s for s in diff if not band[s]]
        if bad:
            s = bad[0]
            return (f"index {s} differs outside the tie band (o={o[s]:.6g}, tau={tau:.6g}, "
                    f"A={A[s]:.3g}, {len(bad)} such)")
    if g_score is not None:
        gsc = np.asarray(g_score[:m], dtype=np.float64)
        e = np.abs(gsc - o[g])
        lim = SCORE_RTOL * A[g]
        if np.any(e > lim):
            j = int(np.argmax(e - lim))
            return f"score of key {g[j]} off: got {gsc[j]:.7g}, oracle {o[g[j]]:.7g}, A {A[g[j]]:.3g}"
        if np.any(np.asarray(g_score[m:]) != -np.inf):
            return "padded scores must be -inf"
    return None


def check_dense(g_row, o, A) -> str | None:
    """A dense score row: s <= t within tolerance, s > t must be -inf."""
    g = np.asarray(g_row, dtype=np.float64)
    n = len(o)
    e = np.abs(g[:n] - o)
    lim = SCORE_RTOL * np.asarray(A)
    if np.any(e > lim):
        j = int(np.argmax(e - lim))
        return f"dense score {j} off: {g[j]:.7g} vs {o[j]:.7g} (A {A[j]:.3g})"
    if not np.all(np.isneginf(g[n:])):
        return "masked dense scores must be -inf"
    return None


def max_rel_err(g, o, A) -> tuple[float, float]:
    """(max |g-o|/A, max |g-o|/|o| over entries with |o| >= 0.1 A)."""
    g = np.asarray(g, dtype=np.float64)
    o = np.asarray(o, dtype=np.float64)
    A = np.asarray(A, dtype=np.float64)
    e = np.abs(g - o)
    r1 = float(np.max(e / np.maximum(A, 1e-300))) if len(e) else 0.0
    big = np.abs(o) >= 0.1 * A
    r2 = float(np.max(e[big] / np.abs(o[big]))) if np.any(big) else 0.0
    return r1, r2
