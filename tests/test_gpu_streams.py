"""Stream discipline through the C ABI: every launch goes to the caller's
stream (the library holds no stream of its own), and two layers with separate
workspaces run concurrently on two streams with the results of running alone."""
import pytest
import torch

import workloads
from fine_grained_routed_amd import PATH_DECODE, PATH_PREFILL, MoELayer
from tests.parity import gpu_inputs, log

pytestmark = pytest.mark.gpu


def _layer(inp, wl, **kw):
    return MoELayer({k: v for k, v in inp.items() if k != "u"}, wl.top_k, **kw)


@pytest.mark.parametrize("path", [PATH_PREFILL, PATH_DECODE])
def test_side_stream_gives_the_default_stream_result(lib, path):
    wl = workloads.get("dsmoe16b").with_T(200)
    inp = gpu_inputs(wl, seed=9)
    layer = _layer(inp, wl)
    want = layer.forward(inp["u"], path=path).clone()
    torch.cuda.synchronize()
    side = torch.cuda.Stream()  # default priority
    u2 = inp["u"].clone()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        got = layer.forward(u2, path=path)
        got2 = got.clone()  # ordered after the layer on the side stream
    side.synchronize()
    log(f"[streams] side stream path={path}")
    assert torch.equal(got2, want)


def test_two_layers_on_two_streams_concurrently(lib):
    wa, wb = workloads.get("dsmoe16b").with_T(300), workloads.get("skew512").with_T(257)
    ia, ib = gpu_inputs(wa, seed=10), gpu_inputs(wb, seed=11)
    la, lb = _layer(ia, wa), _layer(ib, wb)
    want_a = la.forward(ia["u"]).clone()
    want_b = lb.forward(ib["u"]).clone()
    torch.cuda.synchronize()
    sa, sb = torch.cuda.Stream(), torch.cuda.Stream()
    outs = []
    for s, layer, u in ((sa, la, ia["u"]), (sb, lb, ib["u"])):
        s.wait_stream(torch.cuda.current_stream())
    for rep in range(3):
        for s, layer, u in ((sa, la, ia["u"]), (sb, lb, ib["u"])):
            with torch.cuda.stream(s):
                outs.append(layer.forward(u).clone())
    torch.cuda.synchronize()
    log("[streams] two layers, two streams, 3 rounds")
    for rep in range(3):
        assert torch.equal(outs[2 * rep], want_a), f"layer a, round {rep}"
        assert torch.equal(outs[2 * rep + 1], want_b), f"layer b, round {rep}"
