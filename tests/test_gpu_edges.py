"""GPU edge cases: exact ties, sub-ulp near-ties, degenerate routing, N_r = 1,
k = N_r, bf16 output, determinism, invalid indices fed to moe_permute."""
import numpy as np
import pytest
import torch

import workloads
from fine_grained_routed_amd import PATH_DECODE, PATH_PREFILL, MoELayer
from tests.parity import check_case, gpu_inputs, rel_err, TOL

pytestmark = pytest.mark.gpu


def _wl(T, d, E, f, n_shared, k, dtype="bf16", bias=None, name="edge"):
    return workloads.Workload(name, T, d, E, f, n_shared, k, dtype, bias, name, "edge case")


def _layer(inp, wl, **kw):
    return MoELayer({k: v for k, v in inp.items() if k != "u"}, wl.top_k, **kw)


@pytest.mark.parametrize("path", [PATH_PREFILL, PATH_DECODE])
def test_all_logits_tie(lib, path):
    # zero router: every logit is exactly 0, the k lowest experts win in order, gates 1/N_r
    wl = _wl(150, 256, 64, 128, 1, 6, name="tie_all")
    inp = gpu_inputs(wl)
    inp["w_router"].zero_()
    r = check_case(_layer(inp, wl), inp, wl, path=path)
    assert r["diag"]["tokens_exact"] == 150


def test_duplicate_router_rows_tie_to_lower_index(lib):
    wl = _wl(400, 512, 32, 64, 0, 4, name="tie_dup")
    inp = gpu_inputs(wl)
    inp["w_router"][2] = inp["w_router"][5]
    inp["w_router"][9] = inp["w_router"][5]
    layer = _layer(inp, wl)
    check_case(layer, inp, wl)
    idx = layer.router_topk(inp["u"])[0].cpu().numpy()
    both = [(list(r).index(2), list(r).index(5)) for r in idx if 2 in r and 5 in r]
    assert both and all(a < b for a, b in both)


def test_sub_ulp_near_tie(lib):
    # l0 = 1 and l1 = 1 + 2^-60 exactly; fp32 and fp64 both round them to 1
    wl = _wl(8, 64, 4, 64, 0, 1, name="near_tie")
    inp = gpu_inputs(wl)
    u = torch.zeros((8, 64), dtype=torch.float32)
    u[:, 0] = 1.0
    u[:, 1] = 2.0 ** -60
    wr = torch.zeros((4, 64), dtype=torch.float32)
    wr[0, 0] = 1.0
    wr[1, 0] = 1.0
    wr[1, 1] = 1.0
    wr[2, 0] = 0.5
    wr[3, 0] = -1.0
    inp["u"] = u.to(torch.bfloat16).cuda()
    inp["w_router"] = wr.to(torch.bfloat16).cuda()
    layer = _layer(inp, wl)
    idx, _ = layer.router_topk(inp["u"])
    assert idx.cpu().numpy().ravel().tolist() == [1] * 8
    check_case(layer, inp, wl)


@pytest.mark.parametrize("path", [PATH_PREFILL, PATH_DECODE])
def test_one_expert_takes_every_token(lib, path):
    wl = _wl(700, 256, 16, 128, 1, 2, bias="zipf1.2", name="hot")
    inp = gpu_inputs(wl)
    inp["router_bias"] = torch.zeros(16, dtype=torch.float32, device="cuda")
    inp["router_bias"][3] = 100.0
    layer = _layer(inp, wl)
    check_case(layer, inp, wl, path=path)
    idx = layer.router_topk(inp["u"])[0].cpu().numpy()
    assert (idx[:, 0] == 3).all()


def test_single_routed_expert(lib):
    wl = _wl(77, 128, 1, 64, 1, 1, name="single")
    inp = gpu_inputs(wl)
    layer = _layer(inp, wl)
    check_case(layer, inp, wl)
    assert (layer.router_topk(inp["u"])[1] == 1.0).all()


def test_k_equals_n_routed(lib):
    wl = _wl(300, 128, 8, 64, 0, 8, name="full_mix")
    inp = gpu_inputs(wl)
    check_case(_layer(inp, wl), inp, wl)


def test_f32_larger_shapes(lib):
    wl = _wl(130, 256, 40, 128, 2, 5, dtype="f32", name="f32_more")
    inp = gpu_inputs(wl)
    check_case(_layer(inp, wl), inp, wl)


def test_bf16_output(lib):
    wl = workloads.get("dsmoe16b").with_T(200)
    inp = gpu_inputs(wl, seed=3)
    l32 = _layer(inp, wl)
    l16 = _layer(inp, wl, out_dtype=torch.bfloat16)
    o32 = l32.forward(inp["u"]).double().cpu().numpy()
    o16 = l16.forward(inp["u"]).double().cpu().numpy()
    assert rel_err(o16, o32) <= 2 ** -8 * 4
    assert torch.equal(l16.forward(inp["u"]), torch.from_numpy(o32).to(torch.bfloat16).cuda())


@pytest.mark.parametrize("name,T", [("dsmoe16b", 1000), ("skew512", 900)])
def test_deterministic(lib, name, T):
    wl = workloads.get(name).with_T(T)
    inp = gpu_inputs(wl, seed=4)
    layer = _layer(inp, wl)
    a = layer.forward(inp["u"]).clone()
    b = layer.forward(inp["u"]).clone()
    assert torch.equal(a, b)
    c = layer.forward(inp["u"], path=PATH_DECODE)
    assert torch.equal(c, layer.forward(inp["u"], path=PATH_DECODE))


def test_paths_agree(lib):
    wl = workloads.get("dsv3_decode")
    inp = gpu_inputs(wl)
    layer = _layer(inp, wl)
    p = layer.forward(inp["u"], path=PATH_PREFILL).double().cpu().numpy()
    q = layer.forward(inp["u"], path=PATH_DECODE).double().cpu().numpy()
    assert rel_err(q, p) <= 1e-2


@pytest.mark.parametrize("T", [300, 200], ids=["blocks", "one_launch"])
def test_permute_flags_bad_indices(lib, T):
    # 300 tokens: the three-launch permutation; 200: the one-launch form
    wl = _wl(T, 128, 8, 64, 0, 2, name="bad_idx")
    inp = gpu_inputs(wl)
    layer = _layer(inp, wl)
    idx = torch.tensor([[0, 1]] * T, dtype=torch.int32, device="cuda")
    idx[7, 1] = 8        # out of range
    idx[9] = torch.tensor([3, 3], dtype=torch.int32)  # duplicate
    counts, offsets, row_token, token_row = layer.permute(idx)
    torch.cuda.synchronize()
    diag = layer.diagnostics()
    assert diag["flags"] & 2 and diag["flags"] & 4
    assert token_row[7, 1].item() == -1
    assert counts.sum().item() == offsets[-1].item()


def test_decode_matches_prefill_prefix(lib):
    # the decode workload's tokens are the first 64 tokens of the prefill workload
    dec = workloads.get("dsv3_decode")
    pre = workloads.get("dsv3_prefill").with_T(128)
    ud = workloads.make_u(dec, device="cuda")
    up = workloads.make_u(pre, device="cuda")
    assert torch.equal(ud, up[:64])


@pytest.mark.parametrize("path", [PATH_PREFILL, PATH_DECODE])
@pytest.mark.parametrize("T,d,E,f,k", [
    (100, 32768, 16, 64, 4),   # widest model dimension the interface accepts
    (300, 64, 1024, 64, 16),   # most experts and the largest top-k, narrowest model dimension
], ids=["d32768", "E1024_k16"])
def test_interface_limits(lib, path, T, d, E, f, k):
    wl = _wl(T, d, E, f, 1, k, name=f"limits_{d}_{E}")
    inp = gpu_inputs(wl, seed=9)
    check_case(_layer(inp, wl), inp, wl, path=path)


@pytest.mark.parametrize("path", [PATH_PREFILL, PATH_DECODE])
def test_wide_rows_with_large_top_k(lib, path):
    # rows wider than 2048 columns with top-k above 9: the combine keeps two
    # 2048-column chunks per thread in flight, the second one partly past d
    wl = _wl(200, 2560, 32, 128, 1, 12, name="wide_k12")
    inp = gpu_inputs(wl, seed=5)
    check_case(_layer(inp, wl), inp, wl, path=path)
