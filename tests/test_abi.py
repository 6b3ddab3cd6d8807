"""C ABI checks that need no GPU: the library loads, exports every function the
header declares, and rejects bad arguments on the host before any HIP call."""
import ctypes
import os
import re

import pytest

import fine_grained_routed_amd as fgr
from fine_grained_routed_amd import _binding as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
FAKE = 1 << 20  # an aligned, never-dereferenced address: every call below fails validation first


@pytest.fixture(scope="module")
def lib():
    return fgr.load()


def header_functions():
    text = open(os.path.join(ROOT, "include", "moe.h")).read()
    return sorted(set(re.findall(r"^(?:moe_status|const char \*)\s*(moe_\w+)\(", text, re.M)))


def test_header_declares_the_boundary():
    fns = header_functions()
    for name in ("moe_router_topk", "moe_permute", "moe_expert_ffn", "moe_combine", "moe_layer_forward"):
        assert name in fns
    assert set(fns) == set(B.EXPORTS)


def test_library_exports_every_declared_symbol(lib):
    raw = ctypes.CDLL(lib.path)
    for name in header_functions():
        assert hasattr(raw, name), name


def test_struct_sizes_match_header():
    assert ctypes.sizeof(B.Dims) == 40
    assert ctypes.sizeof(B.Weights) == 64
    assert ctypes.sizeof(B.Diag) == 16


def _dims(lib, **kw):
    a = dict(d_model=128, n_routed=8, d_ff=64, d_ff_shared=64, top_k=2, dtype=fgr.MOE_BF16, out_dtype=fgr.MOE_F32)
    a.update(kw)
    return lib.dims(**a)


@pytest.mark.parametrize("kw,status", [
    (dict(top_k=9), B.MOE_ERR_INVALID_VALUE),        # k > N_r
    (dict(top_k=0), B.MOE_ERR_INVALID_VALUE),
    (dict(n_routed=0), B.MOE_ERR_INVALID_VALUE),
    (dict(top_k=17, n_routed=64), B.MOE_ERR_UNSUPPORTED),
    (dict(n_routed=1025), B.MOE_ERR_UNSUPPORTED),
    (dict(dtype=7), B.MOE_ERR_UNSUPPORTED),
    (dict(out_dtype=3), B.MOE_ERR_UNSUPPORTED),
    (dict(d_model=100), B.MOE_ERR_UNSUPPORTED),
    (dict(d_ff=96), B.MOE_ERR_UNSUPPORTED),
    (dict(d_ff_shared=32), B.MOE_ERR_UNSUPPORTED),
    (dict(d_ff_shared=-64), B.MOE_ERR_INVALID_VALUE),
    (dict(n_routed=0, top_k=0, d_ff_shared=0), B.MOE_ERR_INVALID_VALUE),  # a dense layer needs its MLP
    (dict(capacity=-1), B.MOE_ERR_INVALID_VALUE),
    (dict(n_group=3, topk_group=1), B.MOE_ERR_INVALID_VALUE),   # 8 experts do not split into 3 groups
    (dict(n_group=4, topk_group=0), B.MOE_ERR_INVALID_VALUE),
    (dict(n_group=4, topk_group=5), B.MOE_ERR_INVALID_VALUE),
    (dict(n_group=8, topk_group=1), B.MOE_ERR_INVALID_VALUE),   # one expert per group, top-2 needs 2 groups
    (dict(n_routed=128, n_group=128, topk_group=2), B.MOE_ERR_UNSUPPORTED),
])
def test_bad_dims(lib, kw, status):
    with pytest.raises(fgr.MoeError) as ei:
        lib.workspace_size(_dims(lib, **kw), 16)
    assert ei.value.status == status
    assert lib.last_error()


def test_negative_T_and_huge_T(lib):
    with pytest.raises(fgr.MoeError) as ei:
        lib.workspace_size(_dims(lib), -1)
    assert ei.value.status == B.MOE_ERR_INVALID_VALUE
    with pytest.raises(fgr.MoeError) as ei:
        lib.workspace_size(_dims(lib, top_k=8), 1 << 28)
    assert ei.value.status == B.MOE_ERR_UNSUPPORTED


def test_token_cap(lib):
    # every per-token dispatch (combine: 512 work-items a token) stays under
    # the 2^32 work-items of one dispatch packet
    d = _dims(lib, top_k=1)
    assert lib.workspace_size(d, 1 << 22) > 0
    with pytest.raises(fgr.MoeError) as ei:
        lib.workspace_size(d, (1 << 22) + 1)
    assert ei.value.status == B.MOE_ERR_UNSUPPORTED and "tokens per call" in str(ei.value)


@pytest.mark.parametrize("kw,T,path", [
    # fp32 GEMM: (2^26 / 64 row tiles) x (65536 / 32 column tiles) work-groups
    (dict(d_model=64, n_routed=16, d_ff=65536, d_ff_shared=0, top_k=16, dtype=fgr.MOE_F32), 1 << 22, 0),
    # forced decode path: (2^25 / 16 row tiles) x 16 column slices
    (dict(d_model=7168, n_routed=256, d_ff=2048, d_ff_shared=2048, top_k=8), 1 << 22, 2),
])
def test_expert_ffn_grid_limit(lib, kw, T, path):
    # rejected on the host before anything is enqueued (the pointers are never used)
    d = _dims(lib, **kw)
    w = _full_weights(lib, shared=kw["d_ff_shared"] > 0)
    with pytest.raises(fgr.MoeError) as ei:
        lib.layer_forward(d, T, FAKE, w, FAKE, lib.options(path), FAKE, ws_bytes=1 << 62, stream=0)
    assert ei.value.status == B.MOE_ERR_UNSUPPORTED and "work-items" in str(ei.value)


def test_static_scratch_rejects_a_large_call(lib):
    # a call whose workspace exceeds the library's 64 MiB scratch is refused on
    # the host, before the scratch is looked up or anything is enqueued
    d = _dims(lib, d_model=7168, n_routed=256, d_ff=2048, d_ff_shared=2048, top_k=8)
    assert lib.workspace_size(d, 16384) > B.STATIC_WS_BYTES
    with pytest.raises(fgr.MoeError) as ei:
        lib.layer_forward_static(d, 16384, FAKE, _full_weights(lib), FAKE, None, stream=0)
    assert ei.value.status == B.MOE_ERR_WORKSPACE and "scratch" in str(ei.value)
    lib.layer_forward_static(d, 0, None, lib.weights(), None, None, stream=0)  # T = 0: no-op


def test_workspace_size_grows_with_T(lib):
    d = _dims(lib)
    assert lib.workspace_size(d, 0) > 0
    assert lib.workspace_size(d, 1000) > lib.workspace_size(d, 10)


@pytest.mark.parametrize("kw", [dict(d_ff_shared=0), dict(n_routed=0, top_k=0, d_ff=0, d_ff_shared=640),
                                dict(n_routed=0, top_k=0, d_ff=0, d_ff_shared=640, dtype=fgr.MOE_F32),
                                dict(d_ff_shared=0, dtype=fgr.MOE_F32)])
def test_workspace_size_of_every_layer_kind(lib, kw):
    # routed layers without a shared MLP and dense layers (whose decode path
    # sizes split-reduction partials per pass) at pass boundaries and ragged T
    d = _dims(lib, **kw)
    sizes = [lib.workspace_size(d, T) for T in (0, 1, 32, 33, 64, 255, 256, 257, 300, 513, 4096)]
    assert all(s > 0 for s in sizes)
    assert sizes[-1] >= sizes[1]


def test_T_zero_is_a_noop_even_with_null_pointers(lib):
    d = _dims(lib)
    lib.layer_forward(d, 0, None, lib.weights(), None, None, None, ws_bytes=0, stream=0)
    lib.router_topk(d, 0, None, None, None, None, None, None, ws_bytes=0, stream=0)
    lib.permute(d, 0, None, None, None, None, None, None, ws_bytes=0, stream=0)
    lib.combine(d, 0, None, None, None, None, None, stream=0)


def _full_weights(lib, shared=True):
    return lib.weights(FAKE, None, FAKE, FAKE, FAKE, FAKE if shared else None, FAKE if shared else None,
                       FAKE if shared else None)


def test_null_and_misaligned_pointers(lib):
    d = _dims(lib)
    ws_bytes = lib.workspace_size(d, 4)
    with pytest.raises(fgr.MoeError) as ei:
        lib.layer_forward(d, 4, None, _full_weights(lib), FAKE, None, FAKE, ws_bytes=ws_bytes, stream=0)
    assert ei.value.status == B.MOE_ERR_INVALID_VALUE and "u" in str(ei.value)
    with pytest.raises(fgr.MoeError) as ei:
        lib.layer_forward(d, 4, FAKE + 2, _full_weights(lib), FAKE, None, FAKE, ws_bytes=ws_bytes, stream=0)
    assert ei.value.status == B.MOE_ERR_INVALID_VALUE and "aligned" in str(ei.value)
    with pytest.raises(fgr.MoeError) as ei:  # shared experts declared, shared weights missing
        lib.layer_forward(d, 4, FAKE, _full_weights(lib, shared=False), FAKE, None, FAKE, ws_bytes=ws_bytes, stream=0)
    assert ei.value.status == B.MOE_ERR_INVALID_VALUE and "w1s" in str(ei.value)
    d0 = _dims(lib, d_ff_shared=0)
    with pytest.raises(fgr.MoeError) as ei:  # shared weights given, no shared experts declared
        lib.layer_forward(d0, 4, FAKE, _full_weights(lib), FAKE, None, FAKE, ws_bytes=ws_bytes, stream=0)
    assert ei.value.status == B.MOE_ERR_INVALID_VALUE
    with pytest.raises(fgr.MoeError) as ei:
        lib.router_topk(d, 4, FAKE, FAKE, FAKE + 1, FAKE, FAKE, FAKE, ws_bytes=ws_bytes, stream=0)
    assert ei.value.status == B.MOE_ERR_INVALID_VALUE  # misaligned bias


def test_workspace_too_small(lib):
    d = _dims(lib)
    need = lib.workspace_size(d, 4)
    with pytest.raises(fgr.MoeError) as ei:
        lib.layer_forward(d, 4, FAKE, _full_weights(lib), FAKE, None, FAKE, ws_bytes=need - 1, stream=0)
    assert ei.value.status == B.MOE_ERR_WORKSPACE
    with pytest.raises(fgr.MoeError) as ei:
        lib.permute(d, 4, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, ws_bytes=16, stream=0)
    assert ei.value.status == B.MOE_ERR_WORKSPACE


def test_bad_options(lib):
    d = _dims(lib)
    need = lib.workspace_size(d, 4)
    with pytest.raises(fgr.MoeError) as ei:
        lib.layer_forward(d, 4, FAKE, _full_weights(lib), FAKE, lib.options(path=5), FAKE, ws_bytes=need, stream=0)
    assert ei.value.status == B.MOE_ERR_INVALID_VALUE
    bad = B.Options(0, 3, None)
    with pytest.raises(fgr.MoeError) as ei:
        lib.layer_forward(d, 4, FAKE, _full_weights(lib), FAKE, bad, FAKE, ws_bytes=need, stream=0)
    assert ei.value.status == B.MOE_ERR_INVALID_VALUE


def test_missing_library_fails_loudly(tmp_path):
    with pytest.raises(FileNotFoundError):
        B.Library(str(tmp_path / "libmoe.so"))


def test_prefill_operand_limit_is_checked_before_any_launch(lib):
    # u [T, d] of 4 GiB or more cannot be addressed by the prefill GEMMs' 32-bit
    # offsets: rejected on the host, while the decode path has no such limit
    d = _dims(lib, d_model=7168, n_routed=256, d_ff=2048, d_ff_shared=2048, top_k=8)
    T = (1 << 32) // (7168 * 2) + 1
    need = lib.workspace_size(d, T)
    with pytest.raises(fgr.MoeError) as ei:
        lib.layer_forward(d, T, FAKE, _full_weights(lib), FAKE, lib.options(path=fgr.PATH_PREFILL), FAKE,
                          ws_bytes=need, stream=0)
    assert ei.value.status == B.MOE_ERR_UNSUPPORTED and "4 GiB" in str(ei.value)
    with pytest.raises(fgr.MoeError) as ei:
        lib.expert_ffn(d, T, FAKE, _full_weights(lib), FAKE, FAKE, FAKE, FAKE, FAKE, None, FAKE, ws_bytes=need,
                       stream=0)
    assert ei.value.status == B.MOE_ERR_UNSUPPORTED


def test_dense_layer_dims_are_valid_and_routing_calls_refuse_them(lib):
    d = _dims(lib, n_routed=0, top_k=0, d_ff=0, d_ff_shared=640)
    need = lib.workspace_size(d, 100)
    assert need > 0
    with pytest.raises(fgr.MoeError) as ei:
        lib.router_topk(d, 4, FAKE, FAKE, None, FAKE, FAKE, FAKE, ws_bytes=need, stream=0)
    assert ei.value.status == B.MOE_ERR_INVALID_VALUE and "routed" in str(ei.value)
    with pytest.raises(fgr.MoeError) as ei:
        lib.permute(d, 4, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, ws_bytes=need, stream=0)
    assert ei.value.status == B.MOE_ERR_INVALID_VALUE
    with pytest.raises(fgr.MoeError) as ei:  # the dense MLP's weights are required
        lib.layer_forward(d, 4, FAKE, lib.weights(), FAKE, None, FAKE, ws_bytes=need, stream=0)
    assert ei.value.status == B.MOE_ERR_INVALID_VALUE and "w1s" in str(ei.value)
    with pytest.raises(fgr.MoeError) as ei:  # combine of a dense layer needs y_shared
        lib.combine(d, 4, None, None, None, None, FAKE, stream=0)
    assert ei.value.status == B.MOE_ERR_INVALID_VALUE and "y_shared" in str(ei.value)


def test_capacity_seats_exact():
    assert fgr.capacity_seats(1.0, 16384, 8, 256) == 512
    assert fgr.capacity_seats(1.1, 16384, 8, 256) == 564
    assert fgr.capacity_seats(0.5, 3, 2, 3) == 1


def test_rmsnorm_and_block_validation(lib):
    d = _dims(lib)
    lib.rmsnorm(d, 0, None, None, 1e-6, None, stream=0)  # T = 0: no-op
    lib.block_forward(d, 0, None, None, 1e-6, lib.weights(), None, None, None, ws_bytes=0, stream=0)
    with pytest.raises(fgr.MoeError) as ei:
        lib.rmsnorm(d, 4, FAKE, None, 1e-6, FAKE * 2, stream=0)
    assert ei.value.status == B.MOE_ERR_INVALID_VALUE and "norm_weight" in str(ei.value)
    for eps in (-1.0, float("nan"), float("inf")):
        with pytest.raises(fgr.MoeError) as ei:
            lib.rmsnorm(d, 4, FAKE, FAKE, eps, FAKE * 2, stream=0)
        assert ei.value.status == B.MOE_ERR_INVALID_VALUE and "eps" in str(ei.value)
    with pytest.raises(fgr.MoeError) as ei:  # u overlaps x
        lib.rmsnorm(d, 4, FAKE, FAKE, 1e-6, FAKE + 256, stream=0)
    assert ei.value.status == B.MOE_ERR_INVALID_VALUE and "overlaps" in str(ei.value)
    need = lib.workspace_size(d, 4)
    with pytest.raises(fgr.MoeError) as ei:  # out aliases x
        lib.block_forward(d, 4, FAKE, FAKE, 1e-6, _full_weights(lib), FAKE, None, FAKE * 2, ws_bytes=need, stream=0)
    assert ei.value.status == B.MOE_ERR_INVALID_VALUE and "overlaps" in str(ei.value)
    with pytest.raises(fgr.MoeError) as ei:
        lib.block_forward(d, 4, FAKE, FAKE, 1e-6, _full_weights(lib), FAKE * 2, None, FAKE * 4, ws_bytes=need - 1,
                          stream=0)
    assert ei.value.status == B.MOE_ERR_WORKSPACE
