"""Pins of the oracle's accounting to the values the pages print (tests/golden)."""
import json
import os

import pytest

from oracle import accounting as acc

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "pages_printed_values.json")))


def test_granularity_loop_printed_rows():
    g = GOLD["granularity_loop"]
    rows = acc.granularity_rows(g["base_ff"], g["n0"], g["k0"], [r["m"] for r in g["rows"]])
    for got, want in zip(rows, g["rows"]):
        for key in ("experts", "top_k", "expert_ff", "active_ff"):
            assert got[key] == want[key], (key, got, want)
        assert got["combinations"] == int(want["combinations"])


def test_active_ff_invariant_under_segmentation():
    # the active width k*f never changes: the constraint the whole idea is built on
    g = GOLD["granularity_loop"]
    rows = acc.granularity_rows(g["base_ff"], g["n0"], g["k0"], [1, 2, 4, 8, 16])
    assert {r["active_ff"] for r in rows} == {28672}


def test_try_it_yourself_m16():
    g = GOLD["try_it_yourself"]
    rows = acc.granularity_rows(GOLD["granularity_loop"]["base_ff"], 16, 2, [g["m"]])
    assert rows[0]["expert_ff"] == g["expert_ff"]


@pytest.mark.parametrize("row", GOLD["real_shapes"]["rows"] + GOLD["segmentation_example"]["rows"])
def test_combination_counts(row):
    assert acc.combinations(row["experts"], row["top_k"]) == int(row["combinations"])


def test_combinations_small_brute_force():
    from itertools import combinations as it_comb
    for n in range(0, 11):
        for k in range(0, n + 1):
            assert acc.combinations(n, k) == sum(1 for _ in it_comb(range(n), k))


def test_dsv3_accounting():
    g = GOLD["dsv3_accounting"]
    a = acc.layer_accounting(g["d_model"], g["d_ff"], g["n_routed"], g["n_shared"], g["top_k"])
    assert a["per_expert"] == g["per_expert"]
    assert a["total"] == g["total"]
    assert a["active"] == g["active"]
    assert f"{100 * a['active_fraction']:.2f}" == g["active_fraction_pct_2dp"]
    assert a["shared_params"] == g["shared_params"]
    assert f"{100 * a['shared_share']:.0f}" == g["shared_share_pct_0dp"]


def test_equal_budget_identity():
    g = GOLD["equal_budget"]
    res = [acc.expert_budget(g["d"], c["intermediate"], c["routed"], c["top_k"], c["shared"])
           for c in (g["coarse"], g["fine"], g["with_shared"])]
    assert res[0] == res[1] == res[2] == tuple(g["expected"])
    assert sum(r * c for _, r, c in acc.swiglu_matrix_shapes(g["d"], 256)) == g["per_expert_f256"]
    e = g["eight_plus_shared"]
    _, active = acc.expert_budget(g["d"], e["intermediate"], e["routed"], e["top_k"], e["shared"])
    assert active == e["active"]
    assert f"{100 * (active / g['expected'][1] - 1):.1f}" == e["increase_pct"]


@pytest.mark.parametrize("bad", [(0, 64, 8, 2, 0), (128, 64, 8, 9, 0), (128, 64, 8, 2, -1), (128, 0, 8, 2, 0)])
def test_equal_budget_rejects_invalid(bad):
    with pytest.raises(ValueError):
        acc.expert_budget(*bad)


def test_sparsity_figures():
    rows = GOLD["sparsity"]["rows"]
    assert 100 * acc.sparsity(rows[0]["experts"], rows[0]["top_k"]) == rows[0]["active_pct"]
    assert round(100 * acc.sparsity(rows[1]["experts"], rows[1]["top_k"])) == rows[1]["active_pct_approx"]
    assert acc.capacity_to_compute(rows[1]["experts"], rows[1]["top_k"]) == rows[1]["capacity_to_compute"]
