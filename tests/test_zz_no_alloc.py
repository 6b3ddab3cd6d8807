"""The layer through moe_layer_forward_static, the entry point that allocates
nothing (its workspace is the library's own static device array), against
moe_layer_forward with a caller workspace: equal bit for bit, on two calls in
a row, the second with a smaller batch, on the decode and the prefill paths
and for the fp32 layer."""
import pytest
import torch

import workloads
from fine_grained_routed_amd import PATH_AUTO, PATH_PREFILL, MoELayer
from tests.parity import gpu_inputs, log

pytestmark = pytest.mark.gpu

# (workload, first T, second T, path); each call's workspace fits the 64 MiB scratch
CASES = [
    ("dsv3_decode", 64, 17, PATH_AUTO),      # decode path at the DeepSeek-V3 shape (26 MB, then 7 MB)
    ("dsv3_prefill", 128, 40, PATH_PREFILL),  # prefill GEMMs at the DeepSeek-V3 shape (45 MB)
    ("dsmoe16b", 300, 129, PATH_AUTO),        # 16B shape, 2 shared experts fused
    ("tiny_f32", 256, 100, PATH_AUTO),        # fp32 layer
]


@pytest.mark.parametrize("name,T1,T2,path", CASES, ids=[f"{c[0]}-{c[1]}-{c[2]}" for c in CASES])
def test_static_scratch_equals_workspace_call(lib, name, T1, T2, path):
    wl = workloads.get(name).with_T(T1)
    inp = gpu_inputs(wl, seed=21)
    layer = MoELayer({k: v for k, v in inp.items() if k != "u"}, wl.top_k)
    for T in (T1, T2):
        u = inp["u"][:T].contiguous()
        log(f"[static] {name} T={T} path={path}")
        want = layer.forward(u, path=path)
        got = torch.full_like(want, float("nan"))
        lib.layer_forward_static(layer.dims, T, u, layer.cw, got, lib.options(path))
        torch.cuda.synchronize()
        assert torch.equal(got, want), f"{name} T={T}: static-scratch output differs"
