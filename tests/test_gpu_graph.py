"""The whole layer captured into a HIP graph (torch.cuda.CUDAGraph) and
replayed: the library makes no allocation, memset, copy or synchronisation
inside a forward, so a captured call is the same launch sequence.  Every
replay, with new inputs copied into the captured buffer and eager work plus a
synchronisation between replays, must equal the eager call bit for bit."""
import pytest
import torch

import workloads
from fine_grained_routed_amd import PATH_AUTO, PATH_DECODE, PATH_PREFILL, MoELayer
from tests.parity import gpu_inputs, log

pytestmark = pytest.mark.gpu

# skew512 at its full 8192 tokens takes the router's wide tiles and the two
# top-k kernels (one wavefront per token, then the exact-key list)
CASES = [("dsmoe16b", 200, PATH_PREFILL), ("dsv3_decode", None, PATH_DECODE), ("tiny_f32", None, PATH_AUTO),
         ("dense_small", 300, PATH_AUTO), ("skew512", None, PATH_PREFILL)]


@pytest.mark.parametrize("name,T,path", CASES, ids=[f"{c[0]}-T{c[1]}-p{c[2]}" for c in CASES])
def test_graph_replays_equal_eager(lib, name, T, path):
    wl = workloads.get(name)
    if T is not None:
        wl = wl.with_T(T)
    inp = gpu_inputs(wl, seed=12)
    layer = MoELayer({k: v for k, v in inp.items() if k != "u"}, wl.top_k)
    u = inp["u"]
    static_u = u.clone()
    layer.forward(static_u, path=path)  # sizes the workspace before capture
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        static_out = layer.forward(static_u, path=path)
    torch.cuda.synchronize()
    scratch = torch.empty(1 << 20, device="cuda")
    for rep in range(4):
        x = (u * (1.0 + 0.125 * rep)).contiguous() if rep else u
        static_u.copy_(x)
        g.replay()
        torch.cuda.synchronize()
        got = static_out.clone()
        scratch.fill_(float(rep))  # eager work between replays
        want = layer.forward(x, path=path)
        torch.cuda.synchronize()
        log(f"[graph] {name} T={u.shape[0]} path={path} replay {rep}")
        assert torch.equal(got, want), f"replay {rep}: max diff {(got - want).abs().max().item()}"
