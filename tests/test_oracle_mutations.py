"""Plant plausible mistakes in the oracle (on the CPU) and check that the pins catch each.

Each mutant replaces one oracle function with a subtly wrong variant; at least
one of the listed pin tests must then fail.  This is how the pins are shown to
constrain every step (dropped term, wrong sign, swapped operand, wrong tie
rule, renormalised gates, ignored bias, unstable grouping)."""
import numpy as np
import pytest

import oracle
import oracle.block as ob
import oracle.moe_oracle as om
from tests import test_oracle_block as B
from tests import test_oracle_groups as GR
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


def _bf16_scaled(x, how):
    x = np.asarray(x, dtype=np.float64)
    out = x.copy()
    fin = np.isfinite(x) & (x != 0.0)
    _, e = np.frexp(x[fin])
    q = np.maximum(e - 8, -133)
    out[fin] = np.ldexp(how(np.ldexp(x[fin], -q)), q)
    return out


def _bf16_ties_away(x):
    return _bf16_scaled(x, lambda v: np.sign(v) * np.floor(np.abs(v) + 0.5))


def _bf16_truncate(x):
    return _bf16_scaled(x, np.trunc)


def _rms_sum_not_mean(x, gamma, eps):
    x = np.asarray(x, dtype=np.float64)
    return x / np.sqrt(np.sum(x * x, axis=1, keepdims=True) + eps) * np.asarray(gamma)[None, :]


def _rms_eps_outside(x, gamma, eps):
    x = np.asarray(x, dtype=np.float64)
    return x / (np.sqrt(np.mean(x * x, axis=1, keepdims=True)) + eps) * np.asarray(gamma)[None, :]


def _block_raw_input(x, gamma, eps, dtype, w_router=None, w1=None, w3=None, w2=None, k=0, bias=None, w1s=None,
                     w3s=None, w2s=None, capacity=None):
    # the FFN reads the raw stream instead of its RMSNorm
    u = ob.store(x, dtype)
    if k == 0:
        r = {"ffn": ob.dense_ffn(u, w1s, w3s, w2s)}
    else:
        r = om.forward(u, w_router, w1, w3, w2, k, bias, w1s, w3s, w2s, capacity)
        r["ffn"] = r["out"]
    r["u"] = u
    r["out"] = np.asarray(x, dtype=np.float64) + r["ffn"]
    return r


def _block_no_residual(x, gamma, eps, dtype, *a, **kw):
    y = _orig_b["block_forward"](x, gamma, eps, dtype, *a, **kw)
    y["out"] = y["ffn"]
    return y


def _block_adds_normalised(x, gamma, eps, dtype, *a, **kw):
    y = _orig_b["block_forward"](x, gamma, eps, dtype, *a, **kw)
    y["out"] = y["u"] + y["ffn"]
    return y


def _permute_keeps_last(topk_idx, n_routed, capacity=None):
    if capacity is None:
        return _orig["permute"](topk_idx, n_routed)
    T = np.asarray(topk_idx).shape[0]
    c, o, rt, tr = _orig["permute"](np.asarray(topk_idx)[::-1], n_routed, capacity)
    return c, o, (T - 1 - rt).astype(np.int32), tr[::-1].copy()


def _permute_one_seat_more(topk_idx, n_routed, capacity=None):
    return _orig["permute"](topk_idx, n_routed, None if capacity is None else capacity + 1)


def _seats_floor(cf, T, k, n_routed):
    from fractions import Fraction
    return int(Fraction(cf) * T * k / n_routed)


def _combine_wraps_dropped(y_rows, y_shared, topk_w, token_row):
    y_rows = np.asarray(y_rows, dtype=np.float64)
    g = np.asarray(topk_w, dtype=np.float64)
    out = np.zeros((g.shape[0], y_rows.shape[1])) if y_shared is None else np.asarray(y_shared, dtype=np.float64).copy()
    for j in range(g.shape[1]):
        out += g[:, j, None] * y_rows[np.asarray(token_row)[:, j]]
    return out


def _groups_by_sum(l_t, lo_t, hi_t, n_group, topk_group, exact_of):
    gs = l_t.reshape(n_group, -1).sum(axis=1)
    return sorted(int(g) for g in np.lexsort((np.arange(n_group), -gs))[:topk_group]), False


def _groups_ties_high(l_t, lo_t, hi_t, n_group, topk_group, exact_of):
    gl = l_t.reshape(n_group, -1).max(axis=1)
    return sorted(int(g) for g in np.lexsort((-np.arange(n_group), -gl))[:topk_group]), False


def _groups_fp64_only(l_t, lo_t, hi_t, n_group, topk_group, exact_of):
    gl = l_t.reshape(n_group, -1).max(axis=1)
    return sorted(int(g) for g in np.lexsort((np.arange(n_group), -gl))[:topk_group]), False


def _groups_ignored(l_t, lo_t, hi_t, n_group, topk_group, exact_of):
    return list(range(n_group)), False


_orig = {n: getattr(om, n) for n in ("silu", "swiglu", "combine", "route", "permute", "router_logits",
                                     "capacity_seats", "_kept_groups")}
_orig_b = {n: getattr(ob, n) for n in ("round_to_bf16", "rms_norm", "block_forward")}

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
    ("permute", _permute_keeps_last, [lambda: B.test_capacity_keeps_first_seats_in_token_order(3)]),
    ("permute", _permute_one_seat_more, [lambda: B.test_capacity_keeps_first_seats_in_token_order(3),
                                         B.test_capacity_zero_leaves_exactly_the_shared_output]),
    ("capacity_seats", _seats_floor, [lambda: B.test_capacity_seats_hand_values(1.1, 16384, 8, 256, 564)]),
    ("combine", _combine_wraps_dropped, [B.test_capacity_drops_contribute_nothing,
                                         B.test_capacity_zero_leaves_exactly_the_shared_output]),
    ("_kept_groups", _groups_by_sum, [GR.test_group_score_is_the_best_expert_not_the_sum]),
    ("_kept_groups", _groups_ties_high, [GR.test_equal_group_scores_go_to_the_lower_group]),
    ("_kept_groups", _groups_fp64_only, [GR.test_group_scores_a_sub_ulp_apart_are_decided_exactly]),
    ("_kept_groups", _groups_ignored, [GR.test_group_limit_changes_the_choice_hand_example]),
]

MUTANTS_BLOCK = [
    ("round_to_bf16", _bf16_ties_away, [B.test_bf16_ties_go_to_even]),
    ("round_to_bf16", _bf16_truncate, [B.test_bf16_nearest_by_brute_force]),
    ("rms_norm", _rms_sum_not_mean, [B.test_rmsnorm_hand_values]),
    ("rms_norm", _rms_eps_outside, [B.test_rmsnorm_hand_values]),
    ("block_forward", _block_raw_input, [B.test_block_ffn_sees_the_normalised_input]),
    ("block_forward", _block_no_residual, [B.test_block_zero_gain_returns_the_raw_input]),
    ("block_forward", _block_adds_normalised, [B.test_block_zero_gain_returns_the_raw_input,
                                               B.test_dense_block_is_residual_plus_swiglu]),
]


@pytest.mark.parametrize("name,mutant,pins", MUTANTS, ids=[f"{m[0]}:{m[1].__name__}" for m in MUTANTS])
def test_pins_catch_planted_mistake(monkeypatch, name, mutant, pins):
    monkeypatch.setattr(om, name, mutant)
    if hasattr(oracle, name):
        monkeypatch.setattr(oracle, name, mutant)
    caught = 0
    for pin in pins:
        try:
            pin()
        except Exception:
            caught += 1
    assert caught >= 1, "no pin caught the planted mistake"


@pytest.mark.parametrize("name,mutant,pins", MUTANTS_BLOCK, ids=[f"{m[0]}:{m[1].__name__}" for m in MUTANTS_BLOCK])
def test_block_pins_catch_planted_mistake(monkeypatch, name, mutant, pins):
    monkeypatch.setattr(ob, name, mutant)
    monkeypatch.setattr(oracle, name, mutant)
    caught = 0
    for pin in pins:
        try:
            pin()
        except Exception:
            caught += 1
    assert caught >= 1, "no pin caught the planted mistake"
