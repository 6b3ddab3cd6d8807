"""Plant plausible mistakes in the oracle (on the CPU) and check that the pins catch each.

Each mutant replaces one oracle function with a subtly wrong variant; at least
one of the listed pin tests must then fail.  This is how the pins are shown to
constrain every step (dropped term, wrong sign, swapped operand, wrong tie
rule, renormalised gates, ignored bias, unstable grouping)."""
import numpy as np
import pytest

import oracle
import oracle.moe_oracle as om
from tests import test_oracle_layer as L
from tests import test_oracle_router as R


def _silu_wrong_sign(z):
    z = np.asarray(z, dtype=np.float64)
    with np.errstate(over="ignore"):
        return z / (1.0 + np.exp(z))


def _swiglu_swapped(x, w1, w3, w2):
    x = np.asarray(x, dtype=np.float64)
    return (om.silu(x @ np.asarray(w3, dtype=np.float64).T) * (x @ np.asarray(w1, dtype=np.float64).T)) @ np.asarray(w2, dtype=np.float64).T


def _combine_no_shared(y_rows, y_shared, topk_w, token_row):
    return _orig["combine"](y_rows, None, topk_w, token_row)


def _combine_shared_halved(y_rows, y_shared, topk_w, token_row):
    return _orig["combine"](y_rows, None if y_shared is None else 0.5 * np.asarray(y_shared), topk_w, token_row)


def _route_renormalised(u, w_router, k, bias=None):
    idx, g, l, n = _orig["route"](u, w_router, k, bias)
    return idx, g / g.sum(axis=1, keepdims=True), l, n


def _route_ties_high(u, w_router, k, bias=None):
    idx, g, l, n = _orig["route"](u, w_router, k, bias)
    E = np.asarray(w_router).shape[0]
    lr = l[:, ::-1]
    idx2 = np.stack([E - 1 - np.lexsort((np.arange(E), -row))[:k] for row in lr]).astype(np.int32)
    return idx2, np.take_along_axis(oracle.softmax(l), idx2.astype(int), 1), l, n


def _route_ignores_bias(u, w_router, k, bias=None):
    return _orig["route"](u, w_router, k, None)


def _permute_wrong_rank(topk_idx, n_routed):
    counts, offsets, row_token, token_row = _orig["permute"](topk_idx, n_routed)
    return counts, offsets, row_token[::-1].copy(), token_row


def _router_logits_no_bound(u, w_router, bias=None):
    l, beta = _orig["router_logits"](u, w_router, bias)
    return l, 0.0 * beta


_orig = {n: getattr(om, n) for n in ("silu", "swiglu", "combine", "route", "permute", "router_logits")}

MUTANTS = [
    ("silu", _silu_wrong_sign, [L.test_silu_closed_forms, L.test_swiglu_hand_values_fix_branch_roles]),
    ("swiglu", _swiglu_swapped, [L.test_swiglu_hand_values_fix_branch_roles, L.test_swiglu_nonsquare_layout]),
    ("combine", _combine_no_shared, [L.test_shared_term_is_independent_of_the_router_and_never_gated,
                                     L.test_zero_routed_down_leaves_exactly_the_shared_output]),
    ("combine", _combine_shared_halved, [L.test_zero_routed_down_leaves_exactly_the_shared_output]),
    ("route", _route_renormalised, [R.test_gates_are_full_softmax_not_renormalised]),
    ("route", _route_ties_high, [R.test_topk_exact_ties_go_to_lower_index]),
    ("route", _route_ignores_bias, [L.test_sparse_equals_dense_bruteforce_with_bias]),
    ("permute", _permute_wrong_rank, [L.test_permute_matches_stable_argsort_and_invariants]),
    ("router_logits", _router_logits_no_bound, [lambda: R.test_logit_bound_holds_against_exact("f32")]),
]


@pytest.mark.parametrize("name,mutant,pins", MUTANTS, ids=[f"{m[0]}:{m[1].__name__}" for m in MUTANTS])
def test_pins_catch_planted_mistake(monkeypatch, name, mutant, pins):
    monkeypatch.setattr(om, name, mutant)
    monkeypatch.setattr(oracle, name, mutant)
    caught = 0
    for pin in pins:
        try:
            pin()
        except Exception:
            caught += 1
    assert caught >= 1, "no pin caught the planted mistake"
