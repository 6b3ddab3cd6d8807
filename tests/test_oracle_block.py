"""Pins of the oracle's RMSNorm, bf16 rounding, pre-norm block, dense prefix FFN and capacity limit."""
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
import workloads


def _all_finite_bf16() -> np.ndarray:
    """Every finite bf16 value, decoded from its 16-bit pattern (the top half of an fp32)."""
    with np.errstate(invalid="ignore"):
        bits = (np.arange(1 << 16, dtype=np.uint32) << 16).view(np.float32).astype(np.float64)
    return bits[np.isfinite(bits)]


# ----------------------------------------------------------------- bf16 rounding
def test_bf16_ties_go_to_even():
    x = np.array([1 + 2.0 ** -8, 1 + 3 * 2.0 ** -8, -(1 + 2.0 ** -8), 2.0 ** -134, 1.5 * 2.0 ** -133])
    want = [1.0, 1 + 2.0 ** -6, -1.0, 0.0, 2.0 * 2.0 ** -133]
    assert oracle.round_to_bf16(x).tolist() == want


def test_bf16_representable_values_are_fixed_points():
    v = _all_finite_bf16()
    assert np.array_equal(oracle.round_to_bf16(v), v)


def test_bf16_overflow_edge():
    top = (2 - 2.0 ** -7) * 2.0 ** 127  # largest finite bf16
    mid = (2 - 2.0 ** -8) * 2.0 ** 127  # half-way to 2^128: ties to even rounds up, to infinity
    r = oracle.round_to_bf16(np.array([top, mid, -mid, np.inf, np.nan]))
    assert r[0] == top and r[1] == np.inf and r[2] == -np.inf and r[3] == np.inf and np.isnan(r[4])


def test_bf16_nearest_by_brute_force():
    grid = np.unique(_all_finite_bf16())  # sorted, -0.0 and 0.0 merged
    rng = np.random.default_rng(3)
    x = np.concatenate([rng.standard_normal(4000) * 10.0 ** rng.integers(-40, 38, 4000),
                        rng.standard_normal(500) * 2.0 ** -128])
    r = oracle.round_to_bf16(x)
    i = np.clip(np.searchsorted(grid, x), 1, grid.size - 1)
    lo, hi = grid[i - 1], grid[i]
    dlo, dhi = x - lo, hi - x
    pat = lambda v: (np.abs(v).astype(np.float32).view(np.uint32) >> 16) & 1  # last kept mantissa bit
    want = np.where(dlo < dhi, lo, np.where(dhi < dlo, hi, np.where(pat(lo) == 0, lo, hi)))
    assert np.array_equal(r, want)


def test_bf16_matches_torch_on_fp32_inputs():
    # for values already in fp32, rounding once to bf16 is torch's fp32 -> bf16 conversion (ties to even)
    rng = np.random.default_rng(4)
    x32 = (rng.standard_normal(20000) * 10.0 ** rng.integers(-30, 30, 20000)).astype(np.float32)
    want = torch.from_numpy(x32).to(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(oracle.round_to_bf16(x32.astype(np.float64)), want)


# ----------------------------------------------------------------------- RMSNorm
def test_rmsnorm_hand_values():
    u = oracle.rms_norm(np.array([[3.0, 4.0]]), np.ones(2), 0.0)
    assert np.allclose(u, [[3 / np.sqrt(12.5), 4 / np.sqrt(12.5)]], rtol=1e-15, atol=0)
    u = oracle.rms_norm(np.array([[1.0, 1.0]]), np.ones(2), 1.0)  # mean 1 plus eps 1
    assert np.allclose(u, [[2 ** -0.5, 2 ** -0.5]], rtol=1e-15, atol=0)
    u = oracle.rms_norm(np.array([[2.0, 2.0]]), np.array([2.0, -1.0]), 0.0)  # per-channel gain
    assert np.allclose(u, [[2.0, -1.0]], rtol=1e-15, atol=0)


def test_rmsnorm_scale_invariance_and_unit_rms():
    rng = np.random.default_rng(5)
    x = rng.standard_normal((7, 96))
    u = oracle.rms_norm(x, np.ones(96), 0.0)
    assert np.allclose(np.mean(u * u, axis=1), 1.0, rtol=1e-14)
    assert np.allclose(oracle.rms_norm(37.5 * x, np.ones(96), 0.0), u, rtol=1e-14, atol=0)


# ------------------------------------------------------------------- dense FFN
def test_dense_ffn_hand_value():
    s = lambda z: z / (1 + np.exp(-z))
    y = oracle.dense_ffn(np.array([[2.0]]), np.array([[1.0], [-1.0]]), np.array([[1.0], [2.0]]),
                         np.array([[1.0, 1.0]]))
    assert abs(y[0, 0] - (s(2.0) * 2.0 + s(-2.0) * 4.0)) < 1e-14


def test_dense_ffn_width_splits_into_a_sum():
    rng = np.random.default_rng(6)
    d, W = 16, 24
    x = rng.standard_normal((5, d))
    w1, w3, w2 = rng.standard_normal((W, d)), rng.standard_normal((W, d)), rng.standard_normal((d, W))
    parts = sum(oracle.dense_ffn(x, w1[a:a + 8], w3[a:a + 8], w2[:, a:a + 8]) for a in range(0, W, 8))
    assert np.allclose(oracle.dense_ffn(x, w1, w3, w2), parts, rtol=1e-12, atol=1e-12)


# --------------------------------------------------------------- pre-norm block
def _block_case(name="tiny_f32", T=40, seed=0):
    wl = workloads.get(name).with_T(T)
    inp = workloads.make_block_inputs(wl, seed=seed)
    f = {k: workloads.to_f64(v) for k, v in inp.items()}
    return wl, f


def _block(wl, f, x=None, gamma=None, **over):
    a = dict(w_router=f["w_router"], w1=f["w1"], w3=f["w3"], w2=f["w2"], k=wl.top_k, bias=f["router_bias"],
             w1s=f["w1s"], w3s=f["w3s"], w2s=f["w2s"])
    a.update(over)
    return oracle.block_forward(f["x"] if x is None else x, f["gamma"] if gamma is None else gamma,
                                workloads.NORM_EPS, wl.dtype, **a)


def test_block_zero_gain_returns_the_raw_input():
    # u = 0: every logit ties (no bias) so experts 0..k-1 are chosen, every SwiGLU gives 0, out = x exactly
    wl, f = _block_case()
    r = _block(wl, f, gamma=np.zeros(wl.d))
    assert np.array_equal(r["u"], np.zeros_like(f["x"]))
    assert np.array_equal(r["topk_idx"], np.tile(np.arange(wl.top_k, dtype=np.int32), (wl.T, 1)))
    assert np.array_equal(r["out"], f["x"])


def test_block_is_residual_plus_layer_of_the_stored_norm():
    wl, f = _block_case()
    r = _block(wl, f)
    want_u = oracle.store(oracle.rms_norm(f["x"], f["gamma"], workloads.NORM_EPS), wl.dtype)
    assert np.array_equal(r["u"], want_u)
    lay = oracle.forward(want_u, f["w_router"], f["w1"], f["w3"], f["w2"], wl.top_k, f["router_bias"],
                         f["w1s"], f["w3s"], f["w2s"])
    assert np.array_equal(r["out"], f["x"] + lay["out"])


def test_block_ffn_sees_the_normalised_input():
    # scaling the raw stream by a power of two leaves u (eps = 0) and so the FFN part unchanged:
    # feeding the raw stream to the experts would scale it instead
    wl, f = _block_case()
    a = oracle.block_forward(f["x"], f["gamma"], 0.0, wl.dtype, f["w_router"], f["w1"], f["w3"], f["w2"],
                             wl.top_k, f["router_bias"], f["w1s"], f["w3s"], f["w2s"])
    b = oracle.block_forward(8.0 * f["x"], f["gamma"], 0.0, wl.dtype, f["w_router"], f["w1"], f["w3"], f["w2"],
                             wl.top_k, f["router_bias"], f["w1s"], f["w3s"], f["w2s"])
    assert np.array_equal(a["u"], b["u"])
    assert np.allclose(b["out"] - 8.0 * f["x"], a["out"] - f["x"], rtol=0, atol=1e-12)


def test_dense_block_is_residual_plus_swiglu():
    wl, f = _block_case("dense_small", T=24)
    r = oracle.block_forward(f["x"], f["gamma"], workloads.NORM_EPS, wl.dtype, w1s=f["w1s"], w3s=f["w3s"],
                             w2s=f["w2s"])
    z = oracle.block_forward(f["x"], np.zeros(wl.d), workloads.NORM_EPS, wl.dtype, w1s=f["w1s"], w3s=f["w3s"],
                             w2s=f["w2s"])
    assert np.array_equal(z["out"], f["x"])
    assert np.array_equal(r["out"], f["x"] + oracle.swiglu(r["u"], f["w1s"], f["w3s"], f["w2s"]))


# -------------------------------------------------------------- capacity limit
@pytest.mark.parametrize("cf,T,k,E,want", [(1.0, 16384, 8, 256, 512), (1.25, 16384, 8, 256, 640),
                                           (1.1, 16384, 8, 256, 564), (0.5, 3, 2, 3, 1),
                                           (Fraction(1, 3), 3, 1, 1, 1), (2, 5, 1, 4, 3)])
def test_capacity_seats_hand_values(cf, T, k, E, want):
    assert oracle.capacity_seats(cf, T, k, E) == want


def _seat_walk(idx, E, C):
    """Brute force: walk the tokens in order, each expert hands out seats until it has none."""
    used = [0] * E
    kept = np.zeros(idx.shape, dtype=bool)
    for t in range(idx.shape[0]):
        for j in range(idx.shape[1]):
            e = int(idx[t, j])
            if used[e] < C:
                used[e] += 1
                kept[t, j] = True
    return kept, np.array(used)


@pytest.mark.parametrize("C", [0, 1, 3, 7, 50])
def test_capacity_keeps_first_seats_in_token_order(C):
    rng = np.random.default_rng(7)
    T, k, E = 60, 3, 9
    p = rng.dirichlet(np.ones(E) * 0.3)  # uneven loads, so some experts overflow
    idx = np.stack([rng.choice(E, size=k, replace=False, p=p) for _ in range(T)])
    counts, offsets, row_token, token_row = oracle.permute(idx, E, capacity=C)
    kept, used = _seat_walk(idx, E, C)
    assert np.array_equal(counts, used) and np.array_equal(np.diff(offsets), counts) and offsets[0] == 0
    assert np.array_equal(token_row >= 0, kept)
    full = oracle.permute(idx, E)
    for e in range(E):  # each kept group is the first counts[e] rows of the uncapped group
        a, b = offsets[e], offsets[e + 1]
        assert row_token[a:b].tolist() == full[2][full[1][e]:full[1][e] + counts[e]].tolist()
    for t in range(T):
        for j in range(k):
            r = token_row[t, j]
            if r >= 0:
                assert row_token[r] == t and offsets[idx[t, j]] <= r < offsets[idx[t, j] + 1]


def test_capacity_at_least_the_largest_load_changes_nothing():
    rng = np.random.default_rng(8)
    idx = np.stack([rng.choice(11, size=4, replace=False) for _ in range(100)])
    big = int(np.bincount(idx.ravel()).max())
    for a, b in zip(oracle.permute(idx, 11), oracle.permute(idx, 11, capacity=big)):
        assert np.array_equal(a, b)


def test_capacity_zero_leaves_exactly_the_shared_output():
    # every routed assignment dropped: the shared expert still gives a non-zero output
    # ("Shared and fine-grained experts", Researcher level, on shared-expert isolation)
    wl = workloads.get("tiny_f32").with_T(30)
    f = {k: workloads.to_f64(v) for k, v in workloads.make_inputs(wl).items()}
    r = oracle.forward(f["u"], f["w_router"], f["w1"], f["w3"], f["w2"], wl.top_k, f["router_bias"],
                       f["w1s"], f["w3s"], f["w2s"], capacity=0)
    assert np.all(r["token_row"] == -1) and r["offsets"][-1] == 0
    shared = oracle.swiglu(f["u"], f["w1s"], f["w3s"], f["w2s"])
    assert np.array_equal(r["out"], shared) and np.any(shared != 0)


def test_capacity_drops_contribute_nothing():
    wl = workloads.get("tiny_f32").with_T(64)
    f = {k: workloads.to_f64(v) for k, v in workloads.make_inputs(wl).items()}
    C = 9
    r = oracle.forward(f["u"], f["w_router"], f["w1"], f["w3"], f["w2"], wl.top_k, f["router_bias"],
                       f["w1s"], f["w3s"], f["w2s"], capacity=C)
    assert (r["token_row"] == -1).any()
    for t in range(0, wl.T, 7):
        want = oracle.swiglu(f["u"][t:t + 1], f["w1s"], f["w3s"], f["w2s"])[0]
        for j in range(wl.top_k):
            if r["token_row"][t, j] >= 0:
                e = r["topk_idx"][t, j]
                want = want + r["topk_w"][t, j] * oracle.swiglu(f["u"][t:t + 1], f["w1"][e], f["w3"][e], f["w2"][e])[0]
        assert np.allclose(r["out"][t], want, rtol=1e-12, atol=1e-14)
