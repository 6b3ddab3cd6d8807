"""The largest token batch the prefill path accepts at the DeepSeek-V3 shape.
The prefill GEMMs address every operand through 32-bit buffer offsets, and the
host rejects a batch whose hidden activations [T*k, f] (bf16) would reach
4 GiB: T = 2^32 / (k * f * 2) - 1 = 131071 is the largest that runs.  At that
size the offsets into H come within 32 KiB of the limit.  Routing and outputs
are compared with the oracle on sampled tokens that include the first and the
last rows; the grouping is checked for consistency on every token."""
import numpy as np
import pytest
import torch

import oracle
import workloads
from fine_grained_routed_amd import PATH_PREFILL, MoELayer
from tests.parity import GATE_TOL, TOL, gpu_inputs, log, oracle_args, rel_err

pytestmark = pytest.mark.gpu


def test_largest_prefill_batch_at_the_deepseek_v3_shape(lib):
    wl0 = workloads.get("dsv3_prefill")
    T = (1 << 32) // (wl0.top_k * wl0.d_ff * 2) - 1
    assert T * wl0.top_k * wl0.d_ff * 2 < (1 << 32) <= (T + 1) * wl0.top_k * wl0.d_ff * 2
    wl = wl0.with_T(T)
    log(f"[limits] drawing inputs, T={T}")
    inp = gpu_inputs(wl, seed=0)
    layer = MoELayer({k: v for k, v in inp.items() if k != "u"}, wl.top_k)
    u = inp["u"]
    out = layer.forward(u, path=PATH_PREFILL)
    idx, gw = layer.router_topk(u)
    counts, offsets, row_token, token_row = layer.permute(idx)
    torch.cuda.synchronize()
    log(f"[limits] forward done, T={T}")
    # grouping consistent on every token
    R = T * wl.top_k
    c = counts.cpu().numpy().astype(np.int64)
    assert c.sum() == R and np.array_equal(offsets.cpu().numpy(), np.concatenate([[0], np.cumsum(c)]))
    tr = token_row.cpu().numpy()
    rt = row_token.cpu().numpy()
    assert np.array_equal(rt[tr], np.repeat(np.arange(T), wl.top_k).reshape(T, wl.top_k))
    # oracle on sampled tokens, first and last rows included
    toks = np.unique(np.concatenate([workloads.sample_tokens(T, 40, 0), [0, 1, T - 2, T - 1]]))
    a = oracle_args(inp)
    u64 = workloads.to_f64(u[torch.from_numpy(toks).to(u.device)])
    r = oracle.forward(u64, a["w_router"], a["w1"], a["w3"], a["w2"], wl.top_k, a["bias"], a["w1s"], a["w3s"],
                       a["w2s"])
    assert np.array_equal(idx.cpu().numpy()[toks], r["topk_idx"])
    gerr = float(np.max(np.abs(gw.cpu().numpy()[toks].astype(np.float64) - r["topk_w"])))
    assert gerr <= GATE_TOL, gerr
    got = workloads.to_f64(out[torch.from_numpy(toks).to(u.device)])
    err = rel_err(got, r["out"])
    log(f"[limits] T={T}: out err {err:.3e} on {toks.size} tokens, gate err {gerr:.2e}")
    assert err <= TOL["bf16"], err
