"""Pins of the oracle's router: closed forms, exact ties, sub-ulp near-ties,
brute force over all expert subsets, softmax invariants."""
import itertools
from fractions import Fraction

import numpy as np
import pytest

import oracle
import workloads


def _bf16(x):
    import torch
    return torch.tensor(x, dtype=torch.float32).to(torch.bfloat16).to(torch.float64).numpy()


def test_logits_closed_form_basis_vectors():
    # u = sqrt(d) e_i has RMS 1 and picks out column i of the router matrix exactly
    rng = np.random.default_rng(1)
    d, E = 16, 5
    w = rng.standard_normal((E, d)).astype(np.float32).astype(np.float64)
    u = np.sqrt(d) * np.eye(d)
    l, beta = oracle.router_logits(u, w)
    assert np.array_equal(l, np.sqrt(d) * w.T)
    assert np.all(beta >= 0)


def test_logits_use_rows_as_centroids_nonsquare():
    # a transposed operand would not even have the right shape / values
    u = np.array([[1.0, 2.0, 3.0]])
    w = np.array([[1.0, 0.0, 0.0], [0.0, 0.0, 1.0]])
    l, _ = oracle.router_logits(u, w, bias=np.array([0.5, -0.25]))
    assert l.tolist() == [[1.5, 2.75]]


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_logit_bound_holds_against_exact(dtype):
    # fp32 inputs make the fp64 sums inexact (48-bit products), bf16 ones mostly exact
    rng = np.random.default_rng(2)
    cast = _bf16 if dtype == "bf16" else (lambda x: np.asarray(x, np.float32).astype(np.float64))
    u = cast(rng.standard_normal((6, 64)))
    w = cast(0.02 * rng.standard_normal((9, 64)))
    b = rng.standard_normal(9).astype(np.float32).astype(np.float64)
    l, beta = oracle.router_logits(u, w, b)
    inexact = 0
    for t in range(6):
        for e in range(9):
            ex = oracle.exact_logit(u[t], w[e], b[e])
            assert abs(Fraction(l[t, e]) - ex) <= Fraction(beta[t, e])
            inexact += Fraction(l[t, e]) != ex
    if dtype == "f32":
        assert inexact > 0


def test_exact_logit_small_values():
    assert oracle.exact_logit([0.5, 2.0 ** -60], [3.0, 1.0], 0.25) == Fraction(7, 4) + Fraction(1, 2 ** 60)


def test_topk_exact_ties_go_to_lower_index():
    # experts 1 and 3 have identical centroids: exact tie, the lower index wins the earlier slot
    w = np.array([[0.0, 1.0], [1.0, 0.0], [0.5, 0.5], [1.0, 0.0], [-1.0, 0.0]])
    u = np.array([[1.0, 0.0]])
    idx, g, _, n_exact = oracle.route(u, w, 2)
    assert idx.tolist() == [[1, 3]]
    assert n_exact == 1
    idx, _, _, _ = oracle.route(u, w, 1)
    assert idx.tolist() == [[1]]
    # all-zero router: every logit ties, the k lowest indices win in order, gates uniform
    idx, g, _, _ = oracle.route(np.ones((3, 2)), np.zeros((6, 2)), 4)
    assert idx.tolist() == [[0, 1, 2, 3]] * 3
    assert np.allclose(g, 1.0 / 6)


def test_topk_sub_ulp_near_tie_decided_exactly():
    # l0 = 1 and l1 = 1 + 2^-60: equal in fp64, different in exact arithmetic
    u = np.array([[1.0, 2.0 ** -60]])
    w = np.array([[1.0, 0.0], [1.0, 1.0], [0.0, 0.0]])
    l, _ = oracle.router_logits(u, w)
    assert l[0, 0] == l[0, 1]
    idx, _, _, n_exact = oracle.route(u, w, 1)
    assert idx.tolist() == [[1]] and n_exact == 1
    idx, _, _, _ = oracle.route(u, w, 2)
    assert idx.tolist() == [[1, 0]]
    # the same through the bias: b1 makes expert 1 larger by 2^-70 only
    u2 = np.array([[1.0, 0.0]])
    w2 = np.array([[1.0, 0.0], [1.0, 0.0]])
    idx, _, _, _ = oracle.route(u2, w2, 1, bias=np.array([0.0, 2.0 ** -70]))
    assert idx.tolist() == [[1]]


def test_topk_fp64_rounding_order_trap():
    # naive fp64 summation drops the 2^-60 terms and ties; exact sums differ
    u = np.array([[1.0, 2.0 ** -60, 2.0 ** -60, -1.0]])
    w = np.array([[1.0, 1.0, 0.0, 1.0], [1.0, 0.0, 0.0, 1.0], [1.0, 1.0, 1.0, 1.0]])
    idx, _, _, _ = oracle.route(u, w, 3)
    assert idx.tolist() == [[2, 0, 1]]


@pytest.mark.parametrize("E,k", [(8, 2), (16, 2), (8, 3)])
def test_topk_brute_force_over_all_subsets(E, k):
    # the selected set maximises the sum of logits over all C(E, k) subsets
    rng = np.random.default_rng(E * 10 + k)
    d, T = 32, 40
    u = _bf16(rng.standard_normal((T, d)))
    w = _bf16(0.02 * rng.standard_normal((E, d)))
    idx, g, l, _ = oracle.route(u, w, k)
    for t in range(T):
        best = max(itertools.combinations(range(E), k), key=lambda s: sum(oracle.exact_logit(u[t], w[e]) for e in s))
        assert set(idx[t].tolist()) == set(best)
        keys = [oracle.exact_logit(u[t], w[e]) for e in idx[t]]
        assert all(keys[j] > keys[j + 1] for j in range(k - 1))  # slots in descending order
    assert len({tuple(sorted(r)) for r in idx.tolist()}) > 1


def test_softmax_invariants():
    rng = np.random.default_rng(3)
    l = rng.standard_normal((7, 11)) * 3
    p = oracle.softmax(l)
    assert np.allclose(p.sum(axis=1), 1.0, atol=1e-15)
    assert np.all(p > 0)
    assert np.allclose(oracle.softmax(l + 123.25), p, rtol=1e-12, atol=0)
    assert np.array_equal(oracle.softmax(np.array([[4.2]])), np.array([[1.0]]))
    # two experts: p0 = sigmoid(l0 - l1)
    two = oracle.softmax(np.array([[0.7, -0.4]]))
    assert abs(two[0, 0] - 1.0 / (1.0 + np.exp(-1.1))) < 1e-15


def test_gates_are_full_softmax_not_renormalised():
    rng = np.random.default_rng(4)
    u = _bf16(rng.standard_normal((20, 32)))
    w = _bf16(0.2 * rng.standard_normal((10, 32)))
    idx, g, l, _ = oracle.route(u, w, 3)
    p = oracle.softmax(l)
    assert np.allclose(g, np.take_along_axis(p, idx.astype(int), 1), rtol=0, atol=0)
    assert np.all(g.sum(axis=1) < 1.0)
    # k = N_r keeps every expert and the gates add up to 1
    _, g_all, _, _ = oracle.route(u, w, 10)
    assert np.allclose(g_all.sum(axis=1), 1.0, atol=1e-14)


def test_single_expert_gate_is_one():
    u = np.array([[0.3, -1.2], [2.0, 0.5]])
    idx, g, _, _ = oracle.route(u, np.array([[0.1, 0.2]]), 1)
    assert idx.tolist() == [[0], [0]] and g.tolist() == [[1.0], [1.0]]


def test_route_on_workload_inputs_agrees_with_exact_ranking():
    wl = workloads.get("eqbudget_fine").with_T(96)
    inp = workloads.make_inputs(wl, seed=5)
    u, w = workloads.to_f64(inp["u"]), workloads.to_f64(inp["w_router"])
    idx, _, _, _ = oracle.route(u, w, wl.top_k)
    for t in range(0, 96, 7):
        keys = [oracle.exact_logit(u[t], w[e]) for e in range(wl.n_routed)]
        assert idx[t].tolist() == sorted(range(wl.n_routed), key=lambda e: (-keys[e], e))[:wl.top_k]
