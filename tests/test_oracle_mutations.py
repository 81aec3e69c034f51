"""Planted mistakes in the oracle must be caught by the pins.

Each mutant replaces one oracle function with a plausible wrong variant (a
dropped ReLU, a wrong head index, an off-by-one causal prefix, a reversed
tie rule, a schedule without the lag, ...).  For every mutant at least one pin of
``test_oracle_pins`` has to fail; a mutant that passes all pins would mean
the pins cannot tell that mistake from the right answer.
"""
import numpy as np
import pytest

import oracle
import oracle.indexer as oi
from tests import test_oracle_pins as pins

_orig_scores = oi.indexer_scores
_orig_select = oi.select_topk
_orig_dequant = oi.dequant


def _scores_with(fn):
    def f(qh, w, kh):
        qh = np.asarray(qh, dtype=np.float64)
        w = np.asarray(w, dtype=np.float64)
        kh = np.asarray(kh, dtype=np.float64)
        x = kh @ qh.T
        A = (np.abs(kh) @ np.abs(qh).T) @ np.abs(w)
        return fn(x, w), A
    return f


def _select_with(order_fn):
    def f(o, k):
        o = np.asarray(o, dtype=np.float64)
        n = o.shape[0]
        order = order_fn(o, np.arange(n))
        chosen = np.sort(order[:min(k, n)])
        idx = np.full(k, -1, dtype=np.int64)
        sc = np.full(k, -np.inf)
        idx[:len(chosen)] = chosen
        sc[:len(chosen)] = o[chosen]
        return idx, sc
    return f


def _prefix_short(qh, w, kh):
    # drops the diagonal key: scores only s < t (the last key is lost)
    kh = np.asarray(kh)
    o, A = _orig_scores(qh, w, kh)
    if len(o) > 1:
        o = o.copy()
        o[-1] = -1e30
    return o, A


def _no_scale_dequant(codes, scale, fmt):
    return _orig_dequant(codes, None, fmt)


_orig_fs_resolve = oi.fs_resolve
_orig_greedy = oi.fs_greedy_search


def _greedy_ties_high(N, steps, loss):
    # a tie goes to the highest layer: search the layers in reverse order
    return _orig_greedy(N, steps, lambda p: loss(p) - 1e-12 * p.rfind("S"))


def _proxy_counts_f_layers(pattern, ratio):
    src = oi.fs_resolve(pattern)
    r = np.asarray(ratio, dtype=np.float64)
    return sum(1.0 - r[l, src[l] - 1 if l else 0] for l in range(len(pattern))) / len(pattern)


def _mli_attends_own(pattern):
    # F layers attend their own selection (IndexCache without the lag)
    return _orig_fs_resolve(pattern)


def _standin_with(values=slice(0, 512), use_scale=True, drop_padding=True):
    def f(q, latent, sel, scale):
        q, latent, sel = np.asarray(q), np.asarray(latent), np.asarray(sel)
        B, Lmax = latent.shape[0], latent.shape[1]
        out = np.zeros((B, 512))
        for b in range(B):
            keep = (sel[b] >= 0) & (sel[b] < Lmax) if drop_padding else (sel[b] < Lmax)
            rows = sel[b][keep]
            if len(rows) == 0:
                continue
            X = oi.dec_bf16(latent[b, rows])
            sc = (float(scale) if use_scale else 1.0) * (X @ oi.dec_bf16(q[b]))
            pr = np.exp(sc - sc.max())
            out[b] = (pr / pr.sum()) @ X[:, values]
        return out
    return f


MUTANTS = {
    "no_relu": ("indexer_scores", _scores_with(lambda x, w: x @ w)),
    "abs_instead_of_relu": ("indexer_scores", _scores_with(lambda x, w: np.abs(x) @ w)),
    "relu_after_weight": ("indexer_scores", _scores_with(lambda x, w: np.maximum(x * w, 0).sum(1))),
    "heads_reversed_in_w": ("indexer_scores", _scores_with(lambda x, w: np.maximum(x, 0) @ w[::-1])),
    "min_instead_of_max": ("indexer_scores", _scores_with(lambda x, w: np.minimum(x, 0) @ w)),
    "diagonal_dropped": ("indexer_scores", _prefix_short),
    "ties_to_higher_index": ("select_topk", _select_with(lambda o, s: np.lexsort((-s, -o)))),
    "keeps_smallest": ("select_topk", _select_with(lambda o, s: np.lexsort((s, o)))),
    "scales_ignored": ("dequant", _no_scale_dequant),
    "mli_f_layers_attend_own": ("mli_resolve", _mli_attends_own),
    "greedy_ties_to_highest_layer": ("fs_greedy_search", _greedy_ties_high),
    "proxy_wrong_source": ("overlap_proxy_loss", _proxy_counts_f_layers),
    "standin_scale_ignored": ("standin_attention", _standin_with(use_scale=False)),
    "standin_values_from_tail": ("standin_attention", _standin_with(values=slice(64, 576))),
    "standin_padding_read": ("standin_attention", _standin_with(drop_padding=False)),
}

PINS = [
    lambda: pins.test_hand_example_scores_and_sets("bf16"),
    lambda: pins.test_hand_example_scores_and_sets("fp8"),
    pins.test_hand_example_fs_and_overlap,
    lambda: pins.test_selection_closed_forms(5),
    pins.test_selection_brute_force_all_k,
    pins.test_relu_identity_linear_part,
    pins.test_relu_gate_nonnegative_with_nonnegative_weights,
    pins.test_single_head_unit_weight_is_relu_gemv,
    pins.test_head_permutation_invariance,
    pins.test_positive_scaling_equivariance,
    pins.test_greedy_search_additive_loss_closed_form,
    pins.test_greedy_search_ties_and_hand_traced_interaction,
    pins.test_overlap_proxy_closed_form,
    pins.test_mli_resolve_tables,
    pins.test_mli_run_lags_f_layers,
    pins.test_hand_example_lagged_schedule,
    pins.test_standin_attention_zero_query_is_mean_of_values,
    pins.test_standin_attention_two_rows_weights_three_to_one,
    pins.test_standin_attention_invariances_and_limits,
]


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name, monkeypatch):
    attr, fn = MUTANTS[name]
    monkeypatch.setattr(oi, attr, fn)
    if hasattr(oracle, attr):           # the package re-exports the module's functions
        monkeypatch.setattr(oracle, attr, fn)
    caught = 0
    for pin in PINS:
        try:
            pin()
        except (AssertionError, ValueError):
            caught += 1
    assert caught > 0, f"no pin detects mutant {name}"
