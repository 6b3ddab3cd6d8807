"""Pins of the oracle's group-limited top-k (node-limited routing with n_group groups,
topk_group of them kept; reading: a group scores its best expert's logit)."""
from fractions import Fraction

import numpy as np
import pytest

import oracle


def _basis_case(logits):
    """One token whose logits are exactly `logits`: u = e_0, router column 0 = logits."""
    E = len(logits)
    u = np.zeros((1, 4))
    u[0, 0] = 1.0
    w = np.zeros((E, 4))
    w[:, 0] = logits
    return u, w


def test_group_limit_changes_the_choice_hand_example():
    # groups of 2: g0 = {0: 10, 1: 1}, g1 = {2: 9, 3: 2}, g2 = {4: 8, 5: 7.5}, g3 = {6: 3, 7: 0}
    u, w = _basis_case([10, 1, 9, 2, 8, 7.5, 3, 0])
    plain = oracle.route(u, w, 3)[0][0].tolist()
    grouped = oracle.route(u, w, 3, n_group=4, topk_group=2)[0][0].tolist()
    assert plain == [0, 2, 4]
    assert grouped == [0, 2, 3]  # g2's experts are out although expert 4 beats expert 3
    assert oracle.route(u, w, 3, n_group=4, topk_group=3)[0][0].tolist() == [0, 2, 4]


def test_group_score_is_the_best_expert_not_the_sum():
    # g0 = {0: 6, 1: 5.9} sums to 11.9, g1 = {2: 7, 3: -9} sums to -2: the best expert ranks g1 first
    u, w = _basis_case([6, 5.9, 7, -9])
    assert oracle.route(u, w, 2, n_group=2, topk_group=1)[0][0].tolist() == [2, 3]


def test_equal_group_scores_go_to_the_lower_group():
    # experts 0 and 2 tie at 5: g0 = {0: 5, 1: 0} is kept over g1 = {2: 5, 3: 4}
    u, w = _basis_case([5, 0, 5, 4])
    assert oracle.route(u, w, 2, n_group=2, topk_group=1)[0][0].tolist() == [0, 1]


def test_group_scores_a_sub_ulp_apart_are_decided_exactly():
    # logits 1 (expert 0, g0) and 1 + 2^-60 (expert 2, g1) are both 1.0 in fp64
    u = np.array([[1.0, 2.0 ** -60]])
    w = np.array([[1.0, 0.0], [0.0, 0.0], [1.0, 1.0], [-1.0, 0.0]])
    idx, _, _, n_exact = oracle.route(u, w, 2, n_group=2, topk_group=1)
    assert idx[0].tolist() == [2, 3] and n_exact == 1


@pytest.mark.parametrize("n_group,topk_group", [(1, 1), (4, 4)])
def test_no_limit_cases_equal_plain_routing(n_group, topk_group):
    rng = np.random.default_rng(1)
    u, w = rng.standard_normal((50, 16)), rng.standard_normal((8, 16))
    a = oracle.route(u, w, 3)
    b = oracle.route(u, w, 3, n_group=n_group, topk_group=topk_group)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


def _definition(u_row, w, bias, k, n_group, topk_group):
    """The reading written out over exact keys of every expert."""
    E = w.shape[0]
    G = E // n_group
    key = [oracle.exact_logit(u_row, w[e], None if bias is None else bias[e]) for e in range(E)]
    score = [max(key[g * G:(g + 1) * G]) for g in range(n_group)]
    kept = sorted(range(n_group), key=lambda g: (-score[g], g))[:topk_group]
    pool = [e for e in range(E) if e // G in kept]
    return sorted(pool, key=lambda e: (-key[e], e))[:k]


@pytest.mark.parametrize("E,n_group,topk_group,k", [(12, 4, 2, 3), (16, 8, 3, 5), (8, 2, 1, 4)])
def test_grouped_route_matches_the_definition_by_brute_force(E, n_group, topk_group, k):
    rng = np.random.default_rng(E + k)
    # small integer weights and a coarse bias make exact ties between experts and groups common
    u = rng.integers(-2, 3, size=(60, 6)).astype(np.float64)
    w = rng.integers(-2, 3, size=(E, 6)).astype(np.float64)
    bias = rng.integers(-1, 2, size=E).astype(np.float64) * 0.5
    idx = oracle.route(u, w, k, bias, n_group=n_group, topk_group=topk_group)[0]
    for t in range(u.shape[0]):
        assert idx[t].tolist() == _definition(u[t], w, bias, k, n_group, topk_group), t
        groups = {int(e) // (E // n_group) for e in idx[t]}
        assert len(groups) <= topk_group
    assert idx[:, 0].tolist() == oracle.route(u, w, k, bias)[0][:, 0].tolist()  # the best expert is always kept


def test_grouped_route_rejects_too_few_kept_experts():
    u, w = _basis_case([1, 2, 3, 4])
    with pytest.raises(ValueError):
        oracle.route(u, w, 3, n_group=2, topk_group=1)  # 1 group of 2 experts cannot hold 3
