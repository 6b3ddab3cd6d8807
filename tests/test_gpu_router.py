"""GPU parity of the router's wide tiles (64 tokens x 256 experts per work-group)
and of the two top-k kernels' division of labour.

The bf16 router takes these tiles when they alone give at least 256
work-groups, with at least 192 routed experts.  The cases below sit just past
that threshold with ragged token counts, expert counts that leave the last
expert tile partly empty or span two tiles, an odd expert count (scalar logit
stores), and depths of 1, 2, 3 and 5 k-tiles of 64 (every path through the
3-stage ring).  Routing is compared with the oracle on every token, bit for
bit, and the kept gates to the usual tolerance.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads
from fine_grained_routed_amd import PATH_PREFILL, MoELayer
from tests.parity import GATE_TOL, check_case, gpu_inputs, log, oracle_args

pytestmark = pytest.mark.gpu

# name, T, d, E, k, bias
CASES = [
    ("E200_d256", 16384 + 29, 256, 200, 6, "zipf1.2"),
    ("E300_d192", 8192 + 7, 192, 300, 4, None),
    ("E255_d128", 16384 + 1, 128, 255, 8, "zipf1.2"),
    ("E256_d64", 16384 + 63, 64, 256, 8, None),
    ("E512_d320", 8192 + 33, 320, 512, 10, "zipf1.2"),
]


def _wide_tiles(T: int, E: int) -> int:
    return -(-T // 64) * -(-E // 256)


@pytest.mark.parametrize("name,T,d,E,k,bias", CASES, ids=[c[0] for c in CASES])
def test_wide_router_tiles_match_the_oracle(lib, name, T, d, E, k, bias):
    assert E >= 192 and _wide_tiles(T, E) >= 256  # the case takes the wide tiles
    wl = workloads.Workload(name, T, d, E, 64, 1, k, "bf16", bias, f"router_{name}", "router wide tiles")
    inp = gpu_inputs(wl, seed=5)
    layer = MoELayer({kk: vv for kk, vv in inp.items() if kk != "u"}, k)
    idx, gw = layer.router_topk(inp["u"])
    diag = layer.diagnostics()
    a = oracle_args(inp)
    idx_o, gw_o, _, n_exact = oracle.route(workloads.to_f64(inp["u"]), a["w_router"], k, a["bias"])
    idx_g = idx.cpu().numpy()
    bad = np.nonzero((idx_g != idx_o).any(axis=1))[0]
    log(f"[router] {name} T={T}: {bad.size} tokens differ; diagnostics {diag}, oracle exact {n_exact}")
    assert bad.size == 0, (bad[:5], idx_g[bad[:3]], idx_o[bad[:3]])
    gerr = float(np.max(np.abs(gw.cpu().numpy().astype(np.float64) - gw_o)))
    assert gerr <= GATE_TOL, gerr
    assert diag["flags"] == 0, diag


# ------------------------------------------------------------- top-k kernels
# Above 1024 tokens the top-k runs one wavefront per token (levels 1 and 2)
# and lists the tokens that need exact keys for the cooperative kernel; up to
# 1024 it runs the cooperative kernel (four wavefronts per token) for every
# token.  These cases drive the list and the switch.

def _tie_case(T, **kw):
    # zero router: every logit is exactly 0, so every round of every token
    # needs exact keys (the lower index wins)
    wl = workloads.Workload("tie_big", T, 256, 64, 128, 1, 6, "bf16", None, "tie_big", "edge case")
    inp = gpu_inputs(wl)
    inp["w_router"].zero_()
    layer = MoELayer({k: v for k, v in inp.items() if k != "u"}, wl.top_k, **kw)
    return wl, inp, layer


def test_large_batch_exact_ties_go_through_the_list(lib):
    wl, inp, layer = _tie_case(1500)
    r = check_case(layer, inp, wl, path=PATH_PREFILL, sample=256)
    assert r["diag"]["tokens_exact"] == 1500
    assert r["diag"]["exact_keys"] > 0


def test_large_batch_group_limit_with_ties(lib):
    wl, inp, layer = _tie_case(1200, n_group=16, topk_group=2)
    check_case(layer, inp, wl, path=PATH_PREFILL, sample=256)


def test_topk_kernels_agree_across_the_switch(lib):
    # the same tokens routed by the cooperative kernel (a batch of 1024) and by
    # the one-wavefront kernel (the same 1024 tokens plus one)
    wl = workloads.Workload("switch", 1025, 512, 256, 64, 1, 8, "bf16", "zipf1.2", "switch", "top-k switch")
    inp = gpu_inputs(wl, seed=3)
    layer = MoELayer({k: v for k, v in inp.items() if k != "u"}, wl.top_k)
    idx_a, gw_a = layer.router_topk(inp["u"][:1024].contiguous())
    diag_a = layer.diagnostics()
    idx_b, gw_b = layer.router_topk(inp["u"])
    log(f"[router] switch: coop diagnostics {diag_a}, one-wave {layer.diagnostics()}")
    assert torch.equal(idx_a, idx_b[:1024])
    # refined logits may differ in their last bits (different fp64 sum orders)
    assert float((gw_a - gw_b[:1024]).abs().max()) <= 1e-6
    a = oracle_args(inp)
    idx_o, _, _, _ = oracle.route(workloads.to_f64(inp["u"]), a["w_router"], wl.top_k, a["bias"])
    assert np.array_equal(idx_b.cpu().numpy(), idx_o)
