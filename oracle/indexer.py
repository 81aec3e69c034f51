"""Plain, slow, fp64 statement of what the lightning-indexer path computes.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Sources (the pages are cited by title and section):

* "IndexCache deep-dive report" (zako-mio.github.io, IndexShare 03), abstract
  and section 1.1: DSA's lightning indexer is a multi-head, ReLU-gated dot
  product run in FP8 that scores every earlier token and keeps the k = 2048
  best (top-k).  The pages print no equation; the scoring rule used here is
  score(t, s) = sum_h w[t,h] * ReLU(q[t,h] . k[s]) over the causal prefix
  s <= t, one key vector per token shared by all heads.
* Same report, section 1.2: the cross-layer overlap statistic |T_i ∩ T_j| / k.
* Same report, section 2.1, and "Index Share logic" (foosynaptic.github.io,
  tech note 06) section 4.2: Full (F) layers run the indexer and overwrite the
  cached index tensor, Shared (S) layers skip it and use the indices of the
  nearest earlier F layer, f(l) = max{j < l : c_j = F}; the first layer is
  always F.
* Same report, section 3.1: the training-free route chooses the pattern
  greedily -- from all F, each step tries turning every remaining F layer
  into S, evaluates a calibration loss for each trial and commits the best,
  for K steps; section 5.2: a full run costs N(N-1)/2 evaluations and
  similarity proxies do not predict the loss.
* Multi-layer Indexer abstract (equalang.com): at decode the indexer scores
  the whole cache of the sequence and keeps the k = 2048 highest.  Adjacent
  layers select nearly the same tokens, so in the lagged schedule a layer
  attends the selection of the previous indexer layer instead of its own,
  which lets its own indexer run beside its attention; with IndexCache, S
  layers keep attending the nearest earlier F layer's selection.  Each layer
  attends only its k selected tokens.

Readings where the pages are silent: the diagonal s = t is part of the
prefix; ties are broken towards the lower key index (a total order: score
descending, then index ascending); selected
indices are returned in ascending order and padded with -1 when fewer than k
keys exist; FP8 is OCP e4m3fn with one fp32 scale per token, applied by
dequantising before scoring; the decode query sits at position len-1 and its
own key is already in the cache; in the lagged schedule the first layer,
having no earlier indexer layer, attends its own selection.

Parity status: every function here is pinned by tests in ``tests/`` that do
not reuse its code (closed forms, invariants, brute force, a hand-worked
4-token example, and the format decoders against torch's float8/bfloat16).
"""
from __future__ import annotations

import numpy as np

__all__ = [
    "dec_e4m3", "dec_bf16", "dequant", "indexer_scores", "select_topk",
    "prefill", "decode", "fs_resolve", "fs_run", "fs_greedy_search", "overlap_proxy_loss",
    "mli_resolve", "mli_run", "standin_attention",
    "overlap_counts", "overlap_ratio",
]


# ----------------------------------------------------------------------------
# Storage formats
# ----------------------------------------------------------------------------

def dec_e4m3(codes) -> np.ndarray:
    """OCP e4m3fn code -> float64: sign bit, 4 exponent bits (bias 7), 3
    mantissa bits; exponent field 0 is subnormal (m * 2**-9); S.1111.111 is
    NaN, which is an error here (inputs must be finite)."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    s = (c >> 7) & 1
    e = (c >> 3) & 0xF
    m = c & 7
    if np.any((e == 15) & (m == 7)):
        raise ValueError("e4m3 NaN code in input")
    mag = np.where(e == 0, m * 2.0 ** -9, (1.0 + m / 8.0) * np.exp2(e - 7.0))
    return np.where(s == 1, -mag, mag)


def dec_bf16(bits) -> np.ndarray:
    """bf16 bit pattern -> float64 (the pattern is the top half of a float32)."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    v = b.view(np.float32).astype(np.float64)
    if not np.all(np.isfinite(v)):
        raise ValueError("non-finite bf16 input")
    return v


def dequant(codes, scale, fmt: str) -> np.ndarray:
    """Decode a stored tensor and multiply row r by scale[r] (scale may be None)."""
    v = dec_e4m3(codes) if fmt == "fp8" else dec_bf16(codes)
    if scale is not None:
        sc = np.asarray(scale, dtype=np.float32).astype(np.float64)
        v = v * sc.reshape(sc.shape + (1,) * (v.ndim - sc.ndim))
    return v


# ----------------------------------------------------------------------------
# Indexer score and top-k
# ----------------------------------------------------------------------------

def indexer_scores(qh: np.ndarray, w: np.ndarray, kh: np.ndarray):
    """Scores of one query against keys ``kh``.

    qh [H, D] dequantised query heads, w [H] head weights, kh [n, D]
    dequantised keys.  Returns (o [n], A [n]) with
      o[s] = sum_h w[h] * max(q_h . k_s, 0)
      A[s] = sum_h |w[h]| * sum_i |q_h,i * k_s,i|   (the magnitude that
             bounds rounding error in any evaluation order of o).
    """
    qh = np.asarray(qh, dtype=np.float64)
    w = np.asarray(w, dtype=np.float64)
    kh = np.asarray(kh, dtype=np.float64)
    x = kh @ qh.T                    # [n, H]: per-head dot products
    o = np.maximum(x, 0.0) @ w       # ReLU gate, then head-weighted sum
    A = (np.abs(kh) @ np.abs(qh).T) @ np.abs(w)
    return o, A


def select_topk(o: np.ndarray, k: int):
    """The min(k, n) best keys under (score descending, index ascending).

    Returns (idx [k] int64 ascending, -1 padded; score [k] float64 aligned with
    idx, -inf in the padding)."""
    o = np.asarray(o, dtype=np.float64)
    n = o.shape[0]
    s = np.arange(n)
    order = np.lexsort((s, -o))      # primary key -o (so score descending), then s
    chosen = np.sort(order[:min(k, n)])
    idx = np.full(k, -1, dtype=np.int64)
    sc = np.full(k, -np.inf, dtype=np.float64)
    idx[:len(chosen)] = chosen
    sc[:len(chosen)] = o[chosen]
    return idx, sc


def prefill(q, q_scale, k, k_scale, w, fmt: str, topk: int, rows,
            return_scores: bool = False, k_fmt: str | None = None):
    """Single-sequence causal prefill, evaluated for query rows ``rows``.

    q [R, H, D] codes of the rows listed in ``rows`` (row r is token rows[r]);
    q_scale [R] or [R, H] fp32 or None; k [L, D] codes of all keys; k_scale [L]
    or None; w [R, H] bf16 bits.  Row t scores keys s = 0..t.  ``fmt`` is the
    storage format of q ("fp8" or "bf16"); ``k_fmt`` that of k (default: fmt).

    Returns dict with ``idx`` [R, topk], ``score`` [R, topk] and, if asked,
    per-row lists ``o`` and ``A`` (length t+1)."""
    rows = np.asarray(rows, dtype=np.int64)
    kh_all = dequant(k, k_scale, fmt if k_fmt is None else k_fmt)
    q = np.asarray(q)
    qs = None if q_scale is None else np.asarray(q_scale, dtype=np.float32)
    R = len(rows)
    out_idx = np.empty((R, topk), dtype=np.int64)
    out_sc = np.empty((R, topk), dtype=np.float64)
    os_, As_ = [], []
    for r, t in enumerate(rows):
        if qs is None:
            qh = dequant(q[r], None, fmt)
        elif qs.ndim == 1:
            qh = dequant(q[r], None, fmt) * np.float64(qs[r])
        else:
            qh = dequant(q[r], qs[r], fmt)
        wr = dec_bf16(w[r])
        o, A = indexer_scores(qh, wr, kh_all[: t + 1])
        out_idx[r], out_sc[r] = select_topk(o, topk)
        if return_scores:
            os_.append(o)
            As_.append(A)
    res = {"idx": out_idx, "score": out_sc}
    if return_scores:
        res["o"], res["A"] = os_, As_
    return res


def decode(q, w, cache, k_scale, lens, topk: int, return_scores: bool = False):
    """Decode: sequence b has one bf16 query q[b] [H, D] at position
    lens[b]-1 and scores its whole cache cache[b, :lens[b]] (e4m3 codes with
    one fp32 scale per cached token)."""
    B = len(lens)
    out_idx = np.empty((B, topk), dtype=np.int64)
    out_sc = np.empty((B, topk), dtype=np.float64)
    os_, As_ = [], []
    for b in range(B):
        n = int(lens[b])
        qh = dec_bf16(q[b])
        kh = dequant(cache[b, :n], k_scale[b, :n], "fp8")
        o, A = indexer_scores(qh, dec_bf16(w[b]), kh)
        out_idx[b], out_sc[b] = select_topk(o, topk)
        if return_scores:
            os_.append(o)
            As_.append(A)
    res = {"idx": out_idx, "score": out_sc}
    if return_scores:
        res["o"], res["A"] = os_, As_
    return res


# ----------------------------------------------------------------------------
# Layer-reuse (F/S) schedule
# ----------------------------------------------------------------------------

def fs_resolve(pattern: str, N: int | None = None) -> list[int]:
    """Source layer of every layer: src[l] = l for an F layer, and for an S
    layer the nearest earlier F layer.  A pattern that starts with S, has a
    character other than F/S, or whose length is not N is an error."""
    if N is not None and len(pattern) != N:
        raise ValueError("pattern length does not match the layer count")
    if len(pattern) == 0:
        raise ValueError("empty pattern")
    if any(c not in "FS" for c in pattern):
        raise ValueError("pattern characters must be F or S")
    if pattern[0] != "F":
        raise ValueError("the first layer must be F")
    src = []
    last_f = None
    for l, c in enumerate(pattern):
        if c == "F":
            last_f = l
        src.append(last_f)
    return src


def fs_run(pattern: str, layer_topk):
    """Run the schedule: ``layer_topk(l)`` gives layer l's own indices and is
    called for F layers only; an S layer's output is its source's output (the
    same object).  Returns (outputs per layer, src, number of indexer calls)."""
    src = fs_resolve(pattern)
    cache = None
    outs = []
    calls = 0
    for l, c in enumerate(pattern):
        if c == "F":
            cache = layer_topk(l)
            calls += 1
        outs.append(cache)
    return outs, src, calls


def fs_greedy_search(N: int, steps: int, loss):
    """Greedy pattern search: start from all F; at every step turn into S the
    F layer (never the first) whose trial pattern has the lowest
    ``loss(pattern)``, the lowest layer winning ties.  Returns (pattern, the
    all-F loss then the committed loss per step, the layer flipped per step)."""
    if not (0 <= steps <= N - 1):
        raise ValueError("steps must be in [0, N-1]")
    pat = ["F"] * N
    trace = [float(loss("".join(pat)))]
    flipped = []
    for _ in range(steps):
        trials = []
        for l in range(1, N):
            if pat[l] == "F":
                trial = pat.copy()
                trial[l] = "S"
                trials.append((float(loss("".join(trial))), l))
        best = min(trials)          # lowest loss, then lowest layer
        pat[best[1]] = "S"
        trace.append(best[0])
        flipped.append(best[1])
    return "".join(pat), trace, flipped


def overlap_proxy_loss(pattern: str, ratio) -> float:
    """Similarity proxy (a baseline the report says fails): the lost overlap
    1 - ratio[l, src(l)] summed over the S layers, divided by the layer count."""
    src = fs_resolve(pattern)
    r = np.asarray(ratio, dtype=np.float64)
    return sum(1.0 - r[l, src[l]] for l, c in enumerate(pattern) if c == "S") / len(pattern)


def mli_resolve(pattern: str) -> list[int]:
    """Lagged (multi-layer indexer) schedule: the layer whose selection layer l
    attends -- the last F layer strictly before l, or l itself when no F layer
    precedes it (the first layer).  Pattern rules as in ``fs_resolve``."""
    fs_resolve(pattern)   # validates
    src = []
    prev_f = None
    for l, c in enumerate(pattern):
        src.append(l if prev_f is None else prev_f)
        if c == "F":
            prev_f = l
    return src


def mli_run(pattern: str, layer_topk):
    """Run the lagged schedule: ``layer_topk(l)`` gives layer l's own indices
    (F layers only).  Returns (the selection each layer attends, attn_src,
    number of indexer calls)."""
    asrc = mli_resolve(pattern)
    own = {}
    for l, c in enumerate(pattern):
        if c == "F":
            own[l] = layer_topk(l)
    return [own[asrc[l]] for l in range(len(pattern))], asrc, len(own)


# ----------------------------------------------------------------------------
# Stand-in consumer: one head of sparse softmax attention
# ----------------------------------------------------------------------------

def standin_attention(q, latent, sel, scale: float) -> np.ndarray:
    """Per sequence b: softmax over the selected rows j (entries 0 <= T_j <
    Lmax of sel[b]) of scale * q[b] . latent[b, T_j, :576], applied to the
    value part latent[b, T_j, :512].  q [B,576] and latent [B,Lmax,576] are
    bf16 bits; returns float64 [B,512] (zeros for a row with no entry)."""
    q = np.asarray(q)
    latent = np.asarray(latent)
    sel = np.asarray(sel)
    B, Lmax = latent.shape[0], latent.shape[1]
    out = np.zeros((B, 512), dtype=np.float64)
    for b in range(B):
        rows = sel[b][(sel[b] >= 0) & (sel[b] < Lmax)]
        if len(rows) == 0:
            continue
        X = dec_bf16(latent[b, rows])                 # [n, 576]
        s = float(scale) * (X @ dec_bf16(q[b]))       # [n]
        p = np.exp(s - s.max())
        out[b] = (p / p.sum()) @ X[:, :512]
    return out


# ----------------------------------------------------------------------------
# Cross-layer overlap
# ----------------------------------------------------------------------------

def overlap_counts(idx_layers, rows) -> np.ndarray:
    """C[i, j] = sum over ``rows`` of |T_i(t) ∩ T_j(t)|, where T_i(t) is the
    set of non-negative entries of idx_layers[i][t].  uint64 [N, N]."""
    N = len(idx_layers)
    C = np.zeros((N, N), dtype=np.uint64)
    for t in rows:
        sets = [np.asarray(idx_layers[i][t]) for i in range(N)]
        sets = [s[s >= 0] for s in sets]
        top = max([int(s.max()) + 1 if len(s) else 0 for s in sets] + [1])
        M = np.zeros((N, top), dtype=np.int64)
        for i, s in enumerate(sets):
            M[i, s] = 1
        C += (M @ M.T).astype(np.uint64)   # |T_i ∩ T_j| = sum_s [s in T_i][s in T_j]
    return C


def overlap_ratio(C: np.ndarray, topk: int, nrows: int) -> np.ndarray:
    """|T_i ∩ T_j| / k averaged over rows: C / (k * nrows), one fp64 division."""
    return np.asarray(C, dtype=np.float64) / (float(topk) * float(nrows))
