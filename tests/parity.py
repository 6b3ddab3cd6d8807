"""Run one layer case through the C ABI on the GPU and compare it with the oracle.

Not a test module: the GPU tests, smoke() share these helpers.  Inputs are
drawn once on the GPU; the oracle receives exact fp64 copies of the same bytes.
"""
from __future__ import annotations

import sys
from typing import Optional

import numpy as np
import torch

import oracle
import workloads

TOL = {"bf16": 2e-2, "f32": 1e-4}  # max |gpu - oracle| / RMS(oracle)
GATE_TOL = 1e-5  # absolute, on the kept softmax probabilities


def log(msg: str):
    print(msg, flush=True)
    sys.stdout.flush()


def rel_err(got: np.ndarray, want: np.ndarray) -> float:
    rms = float(np.sqrt(np.mean(want * want)))
    if rms == 0.0:
        return float(np.max(np.abs(got - want)))
    return float(np.max(np.abs(got - want)) / rms)


def rel_err_per_token(got: np.ndarray, want: np.ndarray) -> float:
    """max over tokens of max|got - want| / RMS(want) within the token's row.  A wrong
    expert or gate makes a token's routed part wrong by O(1) of its own size;
    rounding stays a small fraction of it whatever the spread of magnitudes
    across tokens."""
    rms = np.sqrt(np.mean(want * want, axis=1))
    err = np.max(np.abs(got - want), axis=1)
    ok = rms > 0
    worst = np.max(err[ok] / rms[ok]) if ok.any() else 0.0
    return float(max(worst, np.max(err[~ok]) if (~ok).any() else 0.0))


def gpu_inputs(wl: workloads.Workload, seed: int = 0, T: Optional[int] = None):
    return workloads.make_inputs(wl, seed=seed, device="cuda", T=T)


def oracle_args(inp):
    return dict(
        w_router=workloads.to_f64(inp["w_router"]),
        w1=workloads.F64Experts(inp["w1"]), w3=workloads.F64Experts(inp["w3"]), w2=workloads.F64Experts(inp["w2"]),
        bias=workloads.to_f64(inp["router_bias"]),
        w1s=workloads.to_f64(inp["w1s"]), w3s=workloads.to_f64(inp["w3s"]), w2s=workloads.to_f64(inp["w2s"]),
    )


def run_stages(layer, u, path: int):
    """Every boundary entry point in turn, then the fused layer call."""
    idx, gw = layer.router_topk(u)
    counts, offsets, row_token, token_row = layer.permute(idx)
    y_rows, y_sh = layer.expert_ffn(u, counts, offsets, row_token, path=path)
    out_stages = layer.combine(y_rows, y_sh, gw, token_row)
    routed = layer.combine(y_rows, None, gw, token_row)
    out = layer.forward(u, path=path)
    diag = layer.diagnostics()
    torch.cuda.synchronize()
    return dict(idx=idx, gw=gw, counts=counts, offsets=offsets, row_token=row_token, token_row=token_row,
                out_stages=out_stages, routed=routed, out=out, diag=diag)


def oracle_outputs(u64, toks, a, k, idx_o, token_row_o, capacity, groups=(None, None)):
    """Oracle layer output and routed-only part for the tokens toks.  With a
    capacity, which pairs keep a seat depends on the whole batch: the kept mask
    comes from the oracle's permutation of all tokens, and a dropped pair's gate
    is zeroed (its expert output then adds exactly nothing)."""
    r = oracle.forward(u64[toks], a["w_router"], a["w1"], a["w3"], a["w2"], k, a["bias"],
                       a["w1s"], a["w3s"], a["w2s"], n_group=groups[0], topk_group=groups[1])
    assert np.array_equal(r["topk_idx"], idx_o[toks])
    if not capacity:
        return r["out"], r["routed"]
    gates = r["topk_w"] * (token_row_o[toks] >= 0)
    return (oracle.combine(r["y_rows"], r["y_shared"], gates, r["token_row"]),
            oracle.combine(r["y_rows"], None, gates, r["token_row"]))


def check_case(layer, inp, wl: workloads.Workload, path: int = 0, sample: Optional[int] = None, seed: int = 0,
               gate_tol: float = GATE_TOL):
    """Full parity check of one case.  sample=None compares every token's output;
    otherwise routing is compared on all tokens and outputs on a seeded sample.
    A layer built with a capacity is checked against the oracle's capacity rule."""
    u = inp["u"]
    T = u.shape[0]
    cap = getattr(layer, "capacity", 0) or None
    groups = (getattr(layer, "n_group", 0) or None, getattr(layer, "topk_group", 0) or None)
    log(f"[parity] {wl.name} T={T} path={path} sample={sample} capacity={cap}")
    g = run_stages(layer, u, path)
    a = oracle_args(inp)
    u64 = workloads.to_f64(u)
    # -- routing, bit-exact on every token
    idx_o, gw_o, _, n_exact = oracle.route(u64, a["w_router"], wl.top_k, a["bias"], *groups)
    idx_g = g["idx"].cpu().numpy()
    bad = np.nonzero((idx_g != idx_o).any(axis=1))[0]
    assert bad.size == 0, (f"top-k differs on {bad.size} tokens, first {bad[:5]}: gpu {idx_g[bad[:3]]} "
                           f"oracle {idx_o[bad[:3]]}; diagnostics {g['diag']}")
    gerr = float(np.max(np.abs(g["gw"].cpu().numpy().astype(np.float64) - gw_o)))
    assert gerr <= gate_tol, f"gate error {gerr} > {gate_tol}"
    counts_o, offsets_o, row_token_o, token_row_o = oracle.permute(idx_o, wl.n_routed, cap)
    assert np.array_equal(g["counts"].cpu().numpy(), counts_o)
    assert np.array_equal(g["offsets"].cpu().numpy(), offsets_o)
    # rows past offsets[N_r] exist only when pairs were dropped, and are left unwritten
    assert np.array_equal(g["row_token"].cpu().numpy()[:offsets_o[-1]], row_token_o)
    assert np.array_equal(g["token_row"].cpu().numpy(), token_row_o)
    assert g["diag"]["flags"] == 0, g["diag"]
    # -- the fused call equals the stage-by-stage calls bit for bit
    assert torch.equal(g["out"], g["out_stages"])
    # -- outputs
    toks = np.arange(T) if sample is None else workloads.sample_tokens(T, sample, seed)
    want_out, want_routed = oracle_outputs(u64, toks, a, wl.top_k, idx_o, token_row_o, cap, groups)
    out_g = g["out"][torch.from_numpy(toks).to(u.device)].to(torch.float64).cpu().numpy()
    routed_g = g["routed"][torch.from_numpy(toks).to(u.device)].to(torch.float64).cpu().numpy()
    e_out = rel_err(out_g, want_out)
    e_routed = rel_err_per_token(routed_g, want_routed)
    tol = TOL[wl.dtype]
    log(f"[parity] {wl.name} T={T}: out err {e_out:.3e}, routed-only err {e_routed:.3e}, gate err {gerr:.2e}, "
        f"exact-ranked tokens gpu {g['diag']['tokens_exact']} oracle {n_exact}")
    assert e_out <= tol, f"output error {e_out} > {tol}"
    assert e_routed <= tol, f"routed-only output error (per token) {e_routed} > {tol}"
    return dict(out_err=e_out, routed_err=e_routed, gate_err=gerr, diag=g["diag"], out=g["out"],
                dropped=int((token_row_o < 0).sum()))
