"""Pins of the oracle's permutation, SwiGLU experts, shared expert and whole layer."""
import numpy as np
import pytest

import oracle
import workloads


def _small(name, T, seed=0):
    wl = workloads.get(name).with_T(T)
    inp = workloads.make_inputs(wl, seed=seed)
    f = {k: workloads.to_f64(v) for k, v in inp.items()}
    return wl, f


def _fwd(wl, f, **over):
    a = dict(u=f["u"], w_router=f["w_router"], w1=f["w1"], w3=f["w3"], w2=f["w2"], k=wl.top_k,
             bias=f["router_bias"], w1s=f["w1s"], w3s=f["w3s"], w2s=f["w2s"])
    a.update(over)
    return oracle.forward(**a)


# ----------------------------------------------------------------------- permutation
def test_permute_matches_stable_argsort_and_invariants():
    rng = np.random.default_rng(0)
    T, k, E = 300, 4, 13
    idx = np.stack([rng.choice(E, size=k, replace=False) for _ in range(T)])
    counts, offsets, row_token, token_row = oracle.permute(idx, E)
    assert counts.sum() == T * k and offsets[0] == 0 and offsets[-1] == T * k
    assert np.array_equal(np.diff(offsets), counts)
    # brute force: walk the experts, and inside each the tokens in order
    rows = [t for e in range(E) for t in range(T) if e in idx[t]]
    assert row_token.tolist() == rows
    for t in range(T):
        for j in range(k):
            r = token_row[t, j]
            assert row_token[r] == t and offsets[idx[t, j]] <= r < offsets[idx[t, j] + 1]
    assert sorted(token_row.ravel().tolist()) == list(range(T * k))


def test_permute_empty_and_single_expert_groups():
    counts, offsets, row_token, token_row = oracle.permute(np.zeros((0, 2), dtype=np.int32), 5)
    assert counts.tolist() == [0] * 5 and offsets.tolist() == [0] * 6 and row_token.size == 0
    idx = np.array([[3], [3], [3]])
    counts, offsets, row_token, token_row = oracle.permute(idx, 4)
    assert counts.tolist() == [0, 0, 0, 3] and offsets.tolist() == [0, 0, 0, 0, 3]
    assert row_token.tolist() == [0, 1, 2] and token_row.ravel().tolist() == [0, 1, 2]


# -------------------------------------------------------------------------- SwiGLU
def test_silu_closed_forms():
    z = np.array([0.0, 1.0, -1.0, 40.0, -40.0, -800.0])
    s = oracle.silu(z)
    assert s[0] == 0.0
    assert abs(s[1] - 1.0 / (1.0 + np.exp(-1.0))) < 1e-16
    assert abs(s[1] - s[2] - 1.0) < 1e-15  # silu(z) - silu(-z) = z
    assert abs(s[3] - 40.0) < 1e-12 and abs(s[4]) < 1e-15 and s[5] == 0.0


def test_swiglu_hand_values_fix_branch_roles():
    # d = 1, f = 1: W2 * silu(W1 x) * (W3 x); swapping W1 and W3 changes the value
    x = np.array([[2.0]])
    y = oracle.swiglu(x, np.array([[0.5]]), np.array([[3.0]]), np.array([[-2.0]]))
    want = -2.0 * (1.0 / (1.0 + np.exp(-1.0))) * 6.0
    assert abs(y[0, 0] - want) < 1e-14
    y_swapped = oracle.swiglu(x, np.array([[3.0]]), np.array([[0.5]]), np.array([[-2.0]]))
    assert abs(y_swapped[0, 0] - want) > 0.1


def test_swiglu_nonsquare_layout():
    # W1, W3 are [f, d]; W2 is [d, f]; a transposed operand fails on shapes or values
    x = np.array([[1.0, 0.0, -1.0]])                     # d = 3
    w1 = np.array([[1.0, 0.0, 0.0], [0.0, 0.0, -1.0]])   # f = 2
    w3 = np.array([[2.0, 0.0, 0.0], [0.0, 1.0, 1.0]])
    w2 = np.array([[1.0, 0.0], [0.0, 1.0], [1.0, 1.0]])
    h = oracle.silu(np.array([1.0, 1.0])) * np.array([2.0, -1.0])
    want = np.array([h[0], h[1], h[0] + h[1]])
    assert np.allclose(oracle.swiglu(x, w1, w3, w2)[0], want, rtol=0, atol=1e-15)


def test_swiglu_zero_gate_or_up_and_linearity_in_down():
    rng = np.random.default_rng(1)
    x = rng.standard_normal((5, 8))
    w1, w3, w2 = rng.standard_normal((6, 8)), rng.standard_normal((6, 8)), rng.standard_normal((8, 6))
    assert np.all(oracle.swiglu(x, np.zeros_like(w1), w3, w2) == 0)
    assert np.all(oracle.swiglu(x, w1, np.zeros_like(w3), w2) == 0)
    assert np.allclose(oracle.swiglu(x, w1, w3, 3 * w2), 3 * oracle.swiglu(x, w1, w3, w2), rtol=1e-13)


def test_single_routed_expert_is_a_dense_swiglu():
    rng = np.random.default_rng(2)
    d, f, T = 16, 8, 9
    u = rng.standard_normal((T, d))
    w1, w3, w2 = rng.standard_normal((1, f, d)), rng.standard_normal((1, f, d)), rng.standard_normal((1, d, f))
    r = oracle.forward(u, rng.standard_normal((1, d)), w1, w3, w2, 1)
    assert np.all(r["topk_w"] == 1.0)
    assert np.allclose(r["out"], oracle.swiglu(u, w1[0], w3[0], w2[0]), rtol=1e-14, atol=0)


# -------------------------------------------------------------------------- shared
def test_zero_routed_down_leaves_exactly_the_shared_output():
    wl, f = _small("tiny_f32", 32)
    r = _fwd(wl, f, w2=np.zeros_like(f["w2"]))
    assert np.array_equal(r["out"], oracle.swiglu(f["u"], f["w1s"], f["w3s"], f["w2s"]))


def test_shared_term_is_independent_of_the_router_and_never_gated():
    wl, f = _small("tiny_f32", 32)
    base = _fwd(wl, f)
    other = _fwd(wl, f, w_router=5.0 * f["w_router"][::-1].copy())
    assert np.array_equal(base["y_shared"], other["y_shared"])
    assert np.allclose(base["out"] - base["routed"], base["y_shared"], rtol=0, atol=1e-14)
    # dropping the shared expert removes exactly the shared term
    nos = _fwd(wl, f, w1s=None, w3s=None, w2s=None)
    assert np.allclose(base["out"] - nos["out"], base["y_shared"], rtol=0, atol=1e-14)


def test_fused_shared_equals_sum_of_separate_experts():
    rng = np.random.default_rng(3)
    d, f, T = 32, 12, 10
    u = rng.standard_normal((T, d))
    a = [rng.standard_normal((f, d)), rng.standard_normal((f, d)), rng.standard_normal((d, f))]
    b = [rng.standard_normal((f, d)), rng.standard_normal((f, d)), rng.standard_normal((d, f))]
    fused = oracle.swiglu(u, np.vstack([a[0], b[0]]), np.vstack([a[1], b[1]]), np.hstack([a[2], b[2]]))
    sep = oracle.swiglu(u, *a) + oracle.swiglu(u, *b)
    assert np.allclose(fused, sep, rtol=1e-12, atol=1e-12)


def test_fused_shared_workload_two_shared_experts():
    wl, f = _small("dsmoe16b", 3)
    assert f["w1s"].shape == (2 * wl.d_ff, wl.d) and f["w2s"].shape == (wl.d, 2 * wl.d_ff)
    h = wl.d_ff
    sep = (oracle.swiglu(f["u"], f["w1s"][:h], f["w3s"][:h], f["w2s"][:, :h])
           + oracle.swiglu(f["u"], f["w1s"][h:], f["w3s"][h:], f["w2s"][:, h:]))
    assert np.allclose(oracle.swiglu(f["u"], f["w1s"], f["w3s"], f["w2s"]), sep, rtol=1e-12, atol=1e-12)


# ----------------------------------------------------------------------- whole layer
@pytest.mark.parametrize("name,T", [("tiny_f32", 24), ("eqbudget_coarse", 20), ("eqbudget_fine", 20)])
def test_sparse_equals_dense_bruteforce(name, T):
    wl, f = _small(name, T, seed=1)
    r = _fwd(wl, f)
    dense = oracle.forward_dense(f["u"], f["w_router"], f["w1"], f["w3"], f["w2"], wl.top_k, f["router_bias"],
                                 f["w1s"], f["w3s"], f["w2s"])
    assert np.array_equal(r["topk_idx"], dense["topk_idx"])
    scale = np.sqrt(np.mean(dense["out"] ** 2))
    assert np.max(np.abs(r["out"] - dense["out"])) <= 1e-12 * scale


def test_sparse_equals_dense_bruteforce_with_bias():
    wl = workloads.Workload("skew_small", 16, 64, 24, 32, 1, 3, "bf16", "zipf1.2", "skew_small", "test")
    inp = workloads.make_inputs(wl, seed=2)
    f = {k: workloads.to_f64(v) for k, v in inp.items()}
    r = _fwd(wl, f)
    dense = oracle.forward_dense(f["u"], f["w_router"], f["w1"], f["w3"], f["w2"], wl.top_k, f["router_bias"],
                                 f["w1s"], f["w3s"], f["w2s"])
    assert np.array_equal(r["topk_idx"], dense["topk_idx"])
    assert np.max(np.abs(r["out"] - dense["out"])) <= 1e-12 * np.sqrt(np.mean(dense["out"] ** 2))
    # the Zipf bias pulls tokens to the low-index experts
    assert np.bincount(r["topk_idx"].ravel(), minlength=24)[:3].sum() > 16


def test_k_equals_n_is_the_full_soft_mixture():
    wl, f = _small("eqbudget_coarse", 12)
    r = _fwd(wl, f, k=wl.n_routed)
    p = oracle.softmax(f["u"] @ f["w_router"].T)
    want = sum(p[:, e, None] * oracle.swiglu(f["u"], f["w1"][e], f["w3"][e], f["w2"][e]) for e in range(wl.n_routed))
    assert np.allclose(r["out"], want, rtol=0, atol=1e-13 * np.abs(want).max())


def test_token_permutation_equivariance_and_single_token():
    wl, f = _small("tiny_f32", 40, seed=3)
    r = _fwd(wl, f)
    perm = np.random.default_rng(9).permutation(40)
    rp = _fwd(wl, f, u=f["u"][perm])
    assert np.array_equal(rp["topk_idx"], r["topk_idx"][perm])
    assert np.allclose(rp["out"], r["out"][perm], rtol=0, atol=1e-14)
    one = _fwd(wl, f, u=f["u"][17:18])
    assert np.array_equal(one["topk_idx"][0], r["topk_idx"][17])
    assert np.allclose(one["out"][0], r["out"][17], rtol=0, atol=1e-14)


def test_no_residual_added():
    # zero every weight: the layer output is exactly zero (u itself is not added)
    wl, f = _small("tiny_f32", 8)
    z = {k: (None if v is None else np.zeros_like(v)) for k, v in f.items()}
    r = _fwd(wl, z, u=f["u"])
    assert np.all(r["out"] == 0)


def test_routed_part_is_gate_weighted_sum_of_selected_experts():
    wl, f = _small("eqbudget_fine", 6, seed=4)
    r = _fwd(wl, f)
    for t in range(6):
        want = sum(r["topk_w"][t, j] * oracle.swiglu(f["u"][t:t + 1], f["w1"][e], f["w3"][e], f["w2"][e])[0]
                   for j, e in enumerate(r["topk_idx"][t]))
        assert np.allclose(r["out"][t], want, rtol=0, atol=1e-15)
