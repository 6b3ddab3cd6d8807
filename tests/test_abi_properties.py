"""Property checks of the host-side C ABI logic, no GPU: for any layer shape,
moe_workspace_size either rejects it with a documented status or returns a size
that holds every buffer the layer needs; it never crashes (a division by zero in
the sizing rules would end the process).  Only validation and sizing run here:
no call below reaches a kernel launch."""
import pytest
from hypothesis import HealthCheck, given, settings
from hypothesis import strategies as st

import fine_grained_routed_amd as fgr
from fine_grained_routed_amd import _binding as B

OK_OR_REJECTED = {B.MOE_OK, B.MOE_ERR_INVALID_VALUE, B.MOE_ERR_UNSUPPORTED}


@pytest.fixture(scope="module")
def lib():
    return fgr.load()


def _edge_ints(lo, hi, extra=()):
    return st.one_of(st.integers(lo, hi), st.sampled_from(sorted(set(extra))))


dims_st = st.fixed_dictionaries(dict(
    d_model=st.one_of(st.integers(1, 40).map(lambda m: 64 * m), _edge_ints(-64, 40000, (0, 63, 100, 7168, 32768))),
    n_routed=_edge_ints(-2, 1100, (0, 1, 8, 64, 256, 512, 1024, 1025)),
    d_ff=st.one_of(st.integers(0, 40).map(lambda m: 64 * m), st.sampled_from([-64, 96, 65536, 65600])),
    d_ff_shared=st.one_of(st.integers(0, 300).map(lambda m: 64 * m), st.sampled_from([-64, 96, 65600])),
    top_k=_edge_ints(-1, 20, (0, 1, 8, 16, 17)),
    dtype=st.sampled_from([B.MOE_BF16, B.MOE_F32, 7]),
    out_dtype=st.sampled_from([B.MOE_BF16, B.MOE_F32, 3]),
    capacity=_edge_ints(-3, 5000, (0, 1)),
    n_group=_edge_ints(-1, 70, (0, 1, 8, 64, 65)),
    topk_group=_edge_ints(-1, 70, (0, 1, 4, 8)),
))
T_st = st.one_of(st.integers(-2, 70000), st.sampled_from([0, 1, 33, 255, 256, 257, 16384, 1 << 20]))


@settings(max_examples=600, deadline=None, derandomize=True, database=None,
          suppress_health_check=[HealthCheck.function_scoped_fixture])
@given(kw=dims_st, T=T_st)
def test_workspace_size_rejects_or_holds_every_buffer(lib, kw, T):
    import ctypes
    d = lib.dims(**kw)
    out = ctypes.c_size_t(0)
    status = lib.lib.moe_workspace_size(ctypes.byref(d), T, ctypes.byref(out))
    assert status in OK_OR_REJECTED, (status, lib.last_error())
    if status != B.MOE_OK:
        assert lib.last_error()  # a rejection always says why
        return
    assert T >= 0 and kw["d_model"] % 64 == 0
    size = out.value
    k, dm, f, fs = kw["top_k"], kw["d_model"], kw["d_ff"], kw["d_ff_shared"]
    eb = 2 if kw["dtype"] == B.MOE_BF16 else 4
    R = T * k
    need = 4 * R * dm + 4 * T * dm * (fs > 0)  # fp32 Y rows and Y_sh
    need += eb * (R * f + T * fs)              # hidden activations
    need += 8 * T * kw["n_routed"]             # fp64 logits
    assert size >= need, (size, need)
    assert size % 256 == 0


@settings(max_examples=300, deadline=None, derandomize=True, database=None,
          suppress_health_check=[HealthCheck.function_scoped_fixture])
@given(kw=dims_st, T=st.integers(1, 5000))
def test_forward_with_null_inputs_is_rejected_not_launched(lib, kw, T):
    # whatever the shape, a forward whose input pointer is NULL fails on the
    # host with a status, before anything is enqueued
    d = lib.dims(**kw)
    with pytest.raises(fgr.MoeError) as ei:
        lib.layer_forward(d, T, None, lib.weights(), None, None, None, ws_bytes=0, stream=0)
    assert ei.value.status in (B.MOE_ERR_INVALID_VALUE, B.MOE_ERR_UNSUPPORTED, B.MOE_ERR_WORKSPACE)
