"""GPU parity of the steps next to the layer, through the C ABI:

* the dense prefix FFN (a layer with no routed experts: only the MLP of width
  d_ff_shared, through the shared-group kernels of both paths);
* the pre-norm block: RMSNorm before the layer (bit-exact against the oracle's
  once-rounded normalisation) and the residual after it;
* the per-expert capacity limit (seats kept in token order; the grouping is
  compared bit for bit, outputs to the layer's tolerance).

Outputs are compared with the oracle to 2e-2 (bf16) / 1e-4 (fp32) of the RMS
of the oracle's FFN output (the residual itself is compared exactly)."""
import numpy as np
import pytest
import torch

import oracle
import workloads
from fine_grained_routed_amd import PATH_AUTO, PATH_DECODE, PATH_PREFILL, MoELayer
from tests.parity import TOL, check_case, gpu_inputs, log, oracle_args, rel_err

pytestmark = pytest.mark.gpu

EPS = workloads.NORM_EPS
_NOT_WEIGHTS = ("u", "x", "gamma")


def _layer(inp, wl, **kw):
    return MoELayer({k: v for k, v in inp.items() if k not in _NOT_WEIGHTS}, wl.top_k, **kw)


def _f64(t):
    return workloads.to_f64(t)


# ------------------------------------------------------------------ dense FFN
def _check_dense(wl, inp, path, out_dtype=torch.float32, sample=None):
    layer = _layer(inp, wl, out_dtype=out_dtype)
    u = inp["u"]
    T = u.shape[0]
    log(f"[dense] {wl.name} T={T} path={path} out={out_dtype} sample={sample}")
    out = layer.forward(u, path=path)
    _, y_sh = layer.expert_ffn(u, None, None, None, path=path)  # the stage calls give the same bytes
    out_stages = layer.combine(None, y_sh, None, None)
    torch.cuda.synchronize()
    assert torch.equal(out, out_stages)
    toks = np.arange(T) if sample is None else workloads.sample_tokens(T, sample, 0)
    want = oracle.dense_ffn(_f64(u)[toks], _f64(inp["w1s"]), _f64(inp["w3s"]), _f64(inp["w2s"]))
    got = _f64(out[torch.from_numpy(toks).to(u.device)])
    err = rel_err(got, want)
    log(f"[dense] {wl.name} T={T}: err {err:.3e}")
    assert err <= TOL[wl.dtype], err
    return out


DENSE = [
    ("dense_small", None, PATH_PREFILL),
    ("dense_small", None, PATH_DECODE),
    ("dense_small", 1, PATH_AUTO),
    ("dense_small", 32, PATH_AUTO),
    ("dense_small", 63, PATH_AUTO),
    ("dense_small", 129, PATH_AUTO),
    ("dense_small", 257, PATH_AUTO),
    ("dense_small", 257, PATH_PREFILL),
    ("dense_small_f32", None, PATH_AUTO),
    ("dsv3_dense_prefill", 300, PATH_PREFILL),
    ("dsv3_dense_decode", None, PATH_DECODE),
]


@pytest.mark.parametrize("name,T,path", DENSE, ids=[f"{c[0]}-T{c[1]}-p{c[2]}" for c in DENSE])
def test_dense_ffn_parity(lib, name, T, path):
    wl = workloads.get(name)
    if T is not None:
        wl = wl.with_T(T)
    _check_dense(wl, gpu_inputs(wl, seed=1), path)


# a model width that is an odd multiple of 64 (the gate/up batches fall back to
# 64-deep ones) and output widths that leave ragged column groups, on passes
# that take either decode kernel, a ragged 64-row block and a short last pass
ODD = [20, 33, 64, 100, 300]


@pytest.mark.parametrize("T", ODD)
def test_dense_decode_odd_width(lib, T):
    import dataclasses
    wl = dataclasses.replace(workloads.get("dense_small"), name="dense_odd", d=320, d_ff=192, family="dodd", T=T)
    _check_dense(wl, gpu_inputs(wl, seed=4), PATH_DECODE)


@pytest.mark.parametrize("T", [100, 256, 300])
def test_dense_decode_full_width_sampled(lib, T):
    # one and two slices per pass, and a 44-row last pass, at the DeepSeek-V3 dense shape
    wl = workloads.get("dsv3_dense_decode").with_T(T)
    _check_dense(wl, gpu_inputs(wl, seed=5), PATH_DECODE)


def test_dense_ffn_bf16_output_and_paths_agree(lib):
    wl = workloads.get("dense_small").with_T(48)
    inp = gpu_inputs(wl, seed=2)
    a = _check_dense(wl, inp, PATH_PREFILL, out_dtype=torch.bfloat16)
    b = _check_dense(wl, inp, PATH_DECODE, out_dtype=torch.bfloat16)
    assert rel_err(_f64(a), _f64(b)) <= TOL["bf16"]


def test_dense_ffn_full_size_sampled(lib):
    wl = workloads.get("dsv3_dense_prefill")
    _check_dense(wl, gpu_inputs(wl, seed=0), PATH_AUTO, sample=512)


# -------------------------------------------------------------------- RMSNorm
def _near_midpoint(v, got, want):
    """Mismatches are allowed only where the exact normalised value lies within
    fp64 rounding of the midpoint between the two neighbouring stored values."""
    mid = 0.5 * (got + want)
    return np.abs(v - mid) <= 1e-14 * np.abs(v)


@pytest.mark.parametrize("name,T", [("tiny_f32", 300), ("dsmoe16b", 333), ("skew512", 64), ("dsv3_prefill", 16384)])
def test_rmsnorm_is_the_once_rounded_normalisation(lib, name, T):
    wl = workloads.get(name).with_T(T)
    x = workloads.make_x(wl, seed=3, device="cuda")
    gamma = workloads.make_gamma(wl, seed=3, device="cuda")
    fake = {"w1s": torch.empty((64, wl.d), dtype=x.dtype, device="cuda")}  # a dense shell: only d and dtype matter
    layer = MoELayer({**fake, "w3s": fake["w1s"], "w2s": torch.empty((wl.d, 64), dtype=x.dtype, device="cuda")}, 0)
    u = layer.rmsnorm(x, gamma, EPS)
    torch.cuda.synchronize()
    v = oracle.rms_norm(_f64(x), _f64(gamma), EPS)
    want = oracle.store(v, wl.dtype)
    got = _f64(u)
    bad = got != want
    log(f"[rmsnorm] {wl.name} T={T}: {int(bad.sum())} of {bad.size} differ")
    assert np.all(_near_midpoint(v[bad], got[bad], want[bad])), "a stored value is not the once-rounded norm"
    assert bad.sum() <= 2


# ---------------------------------------------------------------------- block
BLOCK = [
    ("tiny_f32", 200, PATH_PREFILL),
    ("dsmoe16b", 333, PATH_PREFILL),
    ("dsmoe16b", 40, PATH_DECODE),
    ("skew512", 300, PATH_PREFILL),
    ("dsv3_prefill", 300, PATH_PREFILL),
    ("dense_small", 300, PATH_PREFILL),
    ("dense_small", 30, PATH_DECODE),
]


def _oracle_block(wl, inp, toks):
    a = oracle_args(inp) if wl.top_k else {}
    x64 = _f64(inp["x"])[toks]
    g64 = _f64(inp["gamma"])
    if wl.top_k:
        return oracle.block_forward(x64, g64, EPS, wl.dtype, a["w_router"], a["w1"], a["w3"], a["w2"], wl.top_k,
                                    a["bias"], a["w1s"], a["w3s"], a["w2s"])
    return oracle.block_forward(x64, g64, EPS, wl.dtype, w1s=_f64(inp["w1s"]), w3s=_f64(inp["w3s"]),
                                w2s=_f64(inp["w2s"]))


def _check_block(wl, inp, path, out_dtype=torch.float32, sample=None):
    layer = _layer(inp, wl, out_dtype=out_dtype)
    x, gamma = inp["x"], inp["gamma"]
    T = x.shape[0]
    log(f"[block] {wl.name} T={T} path={path} out={out_dtype} sample={sample}")
    out = layer.block_forward(x, gamma, EPS, path=path)
    u = layer.rmsnorm(x, gamma, EPS)
    lay = MoELayer(layer.w, wl.top_k, out_dtype=torch.float32).forward(u, path=path)
    torch.cuda.synchronize()
    # the residual is added in fp32 after the layer's own fp32 sum, then rounded once
    assert torch.equal(out, (x.float() + lay).to(out_dtype))
    toks = np.arange(T) if sample is None else workloads.sample_tokens(T, sample, 0)
    r = _oracle_block(wl, inp, toks)
    sel = torch.from_numpy(toks).to(x.device)
    assert np.array_equal(_f64(u[sel]), r["u"]), "normalised input differs from the oracle's"
    if wl.top_k:
        idx, _ = layer.router_topk(u)
        assert np.array_equal(idx[sel].cpu().numpy(), r["topk_idx"])
    err = rel_err(_f64(lay[sel]), r["ffn"])
    log(f"[block] {wl.name} T={T}: ffn err {err:.3e}")
    assert err <= TOL[wl.dtype], err


@pytest.mark.parametrize("name,T,path", BLOCK, ids=[f"{c[0]}-T{c[1]}-p{c[2]}" for c in BLOCK])
def test_block_parity(lib, name, T, path):
    wl = workloads.get(name).with_T(T)
    _check_block(wl, workloads.make_block_inputs(wl, seed=4, device="cuda"), path)


def test_block_bf16_output(lib):
    wl = workloads.get("dsmoe16b").with_T(129)
    _check_block(wl, workloads.make_block_inputs(wl, seed=5, device="cuda"), PATH_PREFILL, out_dtype=torch.bfloat16)


def test_block_full_size_sampled(lib):
    wl = workloads.get("dsv3_prefill")
    _check_block(wl, workloads.make_block_inputs(wl, seed=0, device="cuda"), PATH_AUTO, sample=512)


# ------------------------------------------------------------ capacity limit
CAP = [
    ("skew512", 517, 1.0, PATH_PREFILL),
    ("skew512", 517, 1.25, PATH_PREFILL),
    ("skew128_top1", 700, 1.0, PATH_PREFILL),
    ("dsmoe16b", 333, 0.5, PATH_PREFILL),
    ("dsmoe16b", 40, 1.0, PATH_DECODE),
    ("eqbudget_fine", None, 1.0, PATH_PREFILL),
    ("tiny_f32", None, 0.3, PATH_PREFILL),
]


@pytest.mark.parametrize("name,T,cf,path", CAP, ids=[f"{c[0]}-T{c[1]}-cf{c[2]}-p{c[3]}" for c in CAP])
def test_capacity_parity(lib, name, T, cf, path):
    wl = workloads.get(name)
    if T is not None:
        wl = wl.with_T(T)
    C = oracle.capacity_seats(cf, wl.T, wl.top_k, wl.n_routed)
    inp = gpu_inputs(wl, seed=6)
    r = check_case(_layer(inp, wl, capacity=C), inp, wl, path=path)
    log(f"[capacity] {wl.name} cf={cf} C={C}: {r['dropped']} of {wl.T * wl.top_k} pairs dropped")
    if cf <= 1.0:
        assert r["dropped"] > 0


def test_capacity_one_seat(lib):
    wl = workloads.get("dsmoe16b").with_T(100)
    inp = gpu_inputs(wl, seed=7)
    layer = _layer(inp, wl, capacity=1)
    r = check_case(layer, inp, wl, path=PATH_PREFILL)
    chosen = int(torch.unique(layer.router_topk(inp["u"])[0]).numel())
    assert r["dropped"] == wl.T * wl.top_k - chosen  # one pair kept per chosen expert


def test_capacity_above_the_largest_load_changes_nothing(lib):
    wl = workloads.get("skew512").with_T(300)
    inp = gpu_inputs(wl, seed=8)
    free = _layer(inp, wl)
    counts = free.permute(free.router_topk(inp["u"])[0])[0]
    capped = _layer(inp, wl, capacity=int(counts.max().item()))
    a, b = free.forward(inp["u"]), capped.forward(inp["u"])
    torch.cuda.synchronize()
    assert torch.equal(a, b)


def test_capacity_full_size_sampled(lib):
    wl = workloads.get("dsv3_prefill")
    inp = gpu_inputs(wl, seed=0)
    C = oracle.capacity_seats(1.0, wl.T, wl.top_k, wl.n_routed)
    r = check_case(_layer(inp, wl, capacity=C), inp, wl, sample=512)
    log(f"[capacity] dsv3_prefill C={C}: {r['dropped']} pairs dropped")


# ---------------------------------------------------------- group-limited top-k
GROUPS = [
    ("dsv3_prefill", 300, 8, 4, PATH_PREFILL),
    ("dsv3_decode", None, 8, 4, PATH_DECODE),
    ("skew512", 517, 8, 2, PATH_PREFILL),
    ("dsmoe16b", 333, 4, 1, PATH_PREFILL),
    ("eqbudget_fine", None, 8, 3, PATH_PREFILL),
    ("skew128_top1", 400, 16, 1, PATH_PREFILL),
]


@pytest.mark.parametrize("name,T,ng,tg,path", GROUPS, ids=[f"{c[0]}-T{c[1]}-g{c[2]}x{c[3]}-p{c[4]}" for c in GROUPS])
def test_group_limited_parity(lib, name, T, ng, tg, path):
    wl = workloads.get(name)
    if T is not None:
        wl = wl.with_T(T)
    inp = gpu_inputs(wl, seed=9)
    layer = _layer(inp, wl, n_group=ng, topk_group=tg)
    check_case(layer, inp, wl, path=path)
    idx = layer.router_topk(inp["u"])[0].cpu().numpy()
    G = wl.n_routed // ng
    assert max(len({int(e) // G for e in row}) for row in idx) <= tg


def test_group_limit_changes_routing_at_the_deepseek_v3_shape(lib):
    wl = workloads.get("dsv3_prefill").with_T(512)
    inp = gpu_inputs(wl, seed=10)
    plain = _layer(inp, wl).router_topk(inp["u"])[0]
    grouped = _layer(inp, wl, n_group=8, topk_group=4).router_topk(inp["u"])[0]
    all_groups = _layer(inp, wl, n_group=8, topk_group=8).router_topk(inp["u"])[0]
    torch.cuda.synchronize()
    changed = int((plain != grouped).any(dim=1).sum())
    log(f"[groups] dsv3 T=512: {changed} tokens routed differently under 8 groups / keep 4")
    assert changed > 0 and torch.equal(plain, all_groups)
    assert torch.equal(plain[:, 0], grouped[:, 0])  # the best expert is always kept


def test_group_limit_with_every_logit_tied(lib):
    # zero router: all keys tie, the walk meets expert 0 first, so group 0 is kept first
    wl = workloads.Workload("tie_groups", 100, 256, 64, 128, 1, 6, "bf16", None, "tie_groups", "edge case")
    inp = gpu_inputs(wl)
    inp["w_router"].zero_()
    check_case(_layer(inp, wl, n_group=16, topk_group=2), inp, wl, path=PATH_PREFILL)


def test_group_limit_full_size_sampled(lib):
    wl = workloads.get("dsv3_prefill")
    inp = gpu_inputs(wl, seed=0)
    check_case(_layer(inp, wl, n_group=8, topk_group=4), inp, wl, sample=512)


# --------------------------------------------- features combined on one layer
COMBO = [("dsv3_prefill", 300, 8, 4, 0.75, PATH_PREFILL), ("dsv3_decode", None, 8, 4, 0.75, PATH_DECODE),
         ("dsmoe16b", 517, 4, 1, 0.5, PATH_PREFILL), ("dsmoe16b", 40, 4, 1, 0.5, PATH_DECODE),
         ("skew512", 333, 8, 2, 1.0, PATH_AUTO)]


@pytest.mark.parametrize("name,T,ng,tg,cf,path", COMBO, ids=[f"{c[0]}-T{c[1]}-g{c[2]}x{c[3]}-cf{c[4]}-p{c[5]}"
                                                               for c in COMBO])
def test_capacity_with_group_limited_routing(lib, name, T, ng, tg, cf, path):
    # the seat limit applies to the group-limited choice: grouping bit-exact,
    # outputs to the layer tolerance, against the oracle's two rules composed
    wl = workloads.get(name)
    if T is not None:
        wl = wl.with_T(T)
    inp = gpu_inputs(wl, seed=7)
    C = oracle.capacity_seats(cf, wl.T, wl.top_k, wl.n_routed)
    r = check_case(_layer(inp, wl, capacity=C, n_group=ng, topk_group=tg), inp, wl, path=path)
    log(f"[combo] {name} T={wl.T} C={C}: {r['dropped']} pairs dropped")


@pytest.mark.parametrize("path", [PATH_PREFILL, PATH_DECODE])
def test_block_with_capacity_and_group_limited_routing(lib, path):
    # the pre-norm block around a layer with both limits equals x + that layer
    # of the block's own normalisation, and that layer matches the oracle
    wl = workloads.get("dsmoe16b").with_T(129)
    binp = workloads.make_block_inputs(wl, seed=8, device="cuda")
    C = oracle.capacity_seats(0.5, wl.T, wl.top_k, wl.n_routed)
    layer = _layer(binp, wl, capacity=C, n_group=4, topk_group=2)
    x, gamma = binp["x"], binp["gamma"]
    out = layer.block_forward(x, gamma, EPS, path=path)
    u = layer.rmsnorm(x, gamma, EPS)
    lay = layer.forward(u, path=path)
    torch.cuda.synchronize()
    assert torch.equal(out, x.float() + lay)
    inp = {k: v for k, v in binp.items() if k not in ("x", "gamma")}
    inp["u"] = u
    check_case(layer, inp, wl, path=path)
