"""Comparison of device results with the fp64 oracle.

Contract
--------
* Scores: |g - o| <= 2e-3 * max(|o|, 0.1 A(t, s)), where
  A = sum_h |w_h| sum_i |q_h,i k_s,i| (dequantised values).  That is 2e-3
  relative to the score wherever |o| >= 0.1 A, and 2e-4 A below that, where
  heads or dimensions cancel and a bare |o| denominator is ill-conditioned
  (o can be exactly 0 while every term is not).
* Top-k sets: with tau the oracle's k-th score of the row, a key may differ
  between the device set and the oracle set only if |o(s) - tau| <= 1e-3 |tau|
  (the strict band).  Beyond it, a difference is accepted only when fp32
  rounding can explain it: every swap exchanges a key s that the device ranks
  too high with a key s' that it ranks too low, which needs
  |o(s) - o(s')| <= E(s) + E(s'), with E the rounding bound below, so each
  swapped key lies within E(s) + max E over the swapped keys of tau.  Such
  rows are "floor-decided"; they are counted in STATS and reported per test.
* Rounding bound of a device score, by input format:
  - bf16 (bf16 inputs on the bf16 matrix cores):
    the dot product's D exact products take at most D - 1 fp32 roundings
    (gamma_D), the weighted head sum at most H (gamma_H), and the folded
    weight w * q_scale, the ReLU product and k_scale one each:
    E(s) = 1.01 (D + H + 4) 2^-24 A(s).
  - fp8 (e4m3 x e4m3 on the matrix cores): measured on gfx950, the fp8
    matrix-core instruction is not fp32-exact.  It adds each group of 8
    consecutive products in a fixed-point window that keeps bits down to
    2^-13 of the group's largest product (a product of 448 next to 63
    products of 2^-6 loses exactly its 7 group-mates; random codes err by up
    to 1.1e-4 of the sum of |products|).  Each of the other 7 products of a
    group can lose < 2^-13 of the group's largest, so
    E(s) = (7 * 2^-13 + 1.01 (D + H + 4) 2^-24) A(s).
  - fp8q (the decode path: fp8 keys against a bf16 query split into
    two e4m3 limbs with e8m0 scales per block of 32 dimensions, both limbs
    on the fp8 matrix cores).  The split loses at most 2^-22 of the block's
    largest |q| per element (it is exact when a block spans at most 2^14 in
    magnitude), and the limbs' magnitudes add up to at most 1.125 |q_i| +
    2^-16 max|q| per element, which scales the fp8 term above.  With
    M(s) = k_scale(s) sum_h |w_h| max_i |q_h,i| sum_i |k_s,i|:
    E(s) = 1.125 (7 * 2^-13 + 1.01 (D + H + 4) 2^-24) A(s) + 2^-21 M(s).
    tests/test_parity_helper.py checks both limits on an emulation of the
    split.
  `terms` = D + H (192 at H=64, D=128, the largest built shape).  The bound
  is a worst case: the measured worst errors are about 1e-6 A (fp8) and
  1e-8 A (bf16), and the per-test report shows how many rows needed the
  floor at all.
* Structure: ascending, distinct, causal (< n), -1 only in the tail.
"""
from __future__ import annotations

import threading

import numpy as np

SCORE_RTOL = 2e-3
SCORE_FLOOR_A = 0.1
BAND_REL = 1e-3
U32 = 2.0 ** -24
DEFAULT_TERMS = 192

# Accumulated over a session: rows compared, rows whose set difference needed
# the rounding floor, and the worst relative score errors seen.
STATS = {"rows": 0, "floor_rows": 0, "max_err_rel_o": 0.0, "max_err_rel_A": 0.0}
# floor-decided rows since the last take_floor_rows(): (t or row id, worst |o-tau|/|tau|)
_FLOOR_LOG: list = []
_LOCK = threading.Lock()   # the full-size checks call check_row from worker threads


def reset_stats() -> None:
    STATS.update(rows=0, floor_rows=0, max_err_rel_o=0.0, max_err_rel_A=0.0)
    _FLOOR_LOG.clear()


def take_floor_rows() -> list:
    out = list(_FLOOR_LOG)
    _FLOOR_LOG.clear()
    return out


FP8_GROUP_LOSS = 7 * 2.0 ** -13   # fp8 matrix-core groups of 8 products (see module doc)
QLIMB_MAG = 1.125                 # limb magnitudes against |q| (fp8q)
QLIMB_LOSS = 2.0 ** -21           # split loss and limb magnitude slack against M (fp8q)


def fp32_error_bound(A, terms: int = DEFAULT_TERMS, fmt: str = "fp8", M=None):
    """Bound on |device score - exact score| for magnitude A (and, for fmt
    "fp8q", the query-block magnitude M; see module doc)."""
    A = np.asarray(A, dtype=np.float64)
    if fmt == "fp8q":
        if M is None:
            raise ValueError("fmt='fp8q' needs M")
        rel = QLIMB_MAG * (1.01 * (terms + 4) * U32 + FP8_GROUP_LOSS)
        return rel * A + QLIMB_LOSS * np.asarray(M, dtype=np.float64)
    if fmt not in ("fp8", "bf16"):
        raise ValueError(f"unknown format {fmt!r}")
    rel = 1.01 * (terms + 4) * U32 + (FP8_GROUP_LOSS if fmt == "fp8" else 0.0)
    return rel * A


def decode_query_mag(q, w, cache, k_scale, lens) -> list:
    """M for every sequence of a decode batch: per sequence b, the array over
    s < lens[b] of k_scale[b, s] * sum_h |w[b, h]| max_i |q[b, h, i]| *
    sum_i |k[b, s, i]| (dequantised inputs)."""
    import oracle
    out = []
    for b in range(len(lens)):
        n = int(lens[b])
        g = float(np.sum(np.abs(oracle.dec_bf16(w[b])) * np.max(np.abs(oracle.dec_bf16(q[b])), axis=1)))
        out.append(g * np.sum(np.abs(oracle.dequant(cache[b, :n], k_scale[b, :n], "fp8")), axis=1))
    return out


def score_limit(o, A):
    o = np.asarray(o, dtype=np.float64)
    A = np.asarray(A, dtype=np.float64)
    return SCORE_RTOL * np.maximum(np.abs(o), SCORE_FLOOR_A * A)


def _note_score_errors(g, o, A) -> None:
    e = np.abs(np.asarray(g, dtype=np.float64) - o)
    if not len(e):
        return
    ra = float(np.max(e / np.maximum(A, 1e-300)))
    big = np.abs(o) >= SCORE_FLOOR_A * A
    ro = float(np.max(e[big] / np.abs(o[big]))) if np.any(big) else 0.0
    with _LOCK:
        STATS["max_err_rel_A"] = max(STATS["max_err_rel_A"], ra)
        STATS["max_err_rel_o"] = max(STATS["max_err_rel_o"], ro)


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


def check_row(g_idx, o, A, k, g_score=None, terms: int = DEFAULT_TERMS, row_id=None,
              fmt: str = "fp8", M=None) -> str | None:
    """Returns None when the device row matches the oracle row, else a reason."""
    o = np.asarray(o, dtype=np.float64)
    A = np.asarray(A, dtype=np.float64)
    n = len(o)
    err = check_structure(g_idx, n, k)
    if err:
        return err
    with _LOCK:
        STATS["rows"] += 1
    m = min(k, n)
    g = np.asarray(g_idx[:m], dtype=np.int64)
    order = np.lexsort((np.arange(n), -o))
    O = np.sort(order[:m])
    if m == n:
        if not np.array_equal(g, O):
            return "short row must select every key"
    else:
        tau = o[order[m - 1]]
        diff = np.array(sorted(set(g.tolist()).symmetric_difference(O.tolist())), dtype=np.int64)
        if diff.size:
            dist = np.abs(o[diff] - tau)
            strict = dist <= BAND_REL * abs(tau)
            E = fp32_error_bound(A[diff], terms, fmt, None if M is None else np.asarray(M)[diff])
            floor = E + E.max()
            ok = strict | (dist <= floor)
            if not np.all(ok):
                s = int(diff[~ok][0])
                return (f"index {s} differs outside the tie band (o={o[s]:.6g}, tau={tau:.6g}, "
                        f"|o-tau|/|tau|={abs(o[s] - tau) / max(abs(tau), 1e-300):.3g}, A={A[s]:.3g}, "
                        f"{int(np.sum(~ok))} such)")
            if not np.all(strict):
                with _LOCK:
                    STATS["floor_rows"] += 1
                    _FLOOR_LOG.append((row_id, float(np.max(dist) / max(abs(tau), 1e-300))))
    if g_score is not None:
        gsc = np.asarray(g_score[:m], dtype=np.float64)
        og, Ag = o[g], A[g]
        e = np.abs(gsc - og)
        lim = score_limit(og, Ag)
        if np.any(e > lim):
            j = int(np.argmax(e - lim))
            return (f"score of key {g[j]} off: got {gsc[j]:.7g}, oracle {og[j]:.7g}, "
                    f"|err|/|o|={e[j] / max(abs(og[j]), 1e-300):.3g}, A {Ag[j]:.3g}")
        _note_score_errors(gsc, og, Ag)
        if np.any(np.asarray(g_score[m:]) != -np.inf):
            return "padded scores must be -inf"
    return None


def check_dense(g_row, o, A) -> str | None:
    """A dense score row: s <= t within tolerance, s > t must be -inf."""
    g = np.asarray(g_row, dtype=np.float64)
    o = np.asarray(o, dtype=np.float64)
    A = np.asarray(A, dtype=np.float64)
    n = len(o)
    e = np.abs(g[:n] - o)
    lim = score_limit(o, A)
    if np.any(e > lim):
        j = int(np.argmax(e - lim))
        return f"dense score {j} off: {g[j]:.7g} vs {o[j]:.7g} (A {A[j]:.3g})"
    _note_score_errors(g[:n], o, A)
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
    big = np.abs(o) >= SCORE_FLOOR_A * A
    r2 = float(np.max(e[big] / np.abs(o[big]))) if np.any(big) else 0.0
    return r1, r2
