"""ctypes binding of libmoe.so: the C ABI declared in include/moe.h, same names.

Argument marshalling only: tensors become device pointers, the current torch
stream becomes the hipStream_t, status codes become exceptions.  Every step of
the layer runs in the library's HIP kernels.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence

_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libmoe.so")

MOE_OK, MOE_ERR_INVALID_VALUE, MOE_ERR_UNSUPPORTED, MOE_ERR_WORKSPACE, MOE_ERR_HIP = range(5)
MOE_F32, MOE_BF16 = 0, 1
PATH_AUTO, PATH_PREFILL, PATH_DECODE = 0, 1, 2

STATUS_NAMES = {0: "MOE_OK", 1: "MOE_ERR_INVALID_VALUE", 2: "MOE_ERR_UNSUPPORTED",
                3: "MOE_ERR_WORKSPACE", 4: "MOE_ERR_HIP"}

# the functions include/moe.h declares
EXPORTS = ("moe_workspace_size", "moe_router_topk", "moe_permute", "moe_expert_ffn", "moe_combine",
           "moe_layer_forward", "moe_layer_forward_static", "moe_rmsnorm", "moe_block_forward",
           "moe_read_diagnostics", "moe_last_error")
STATIC_WS_BYTES = 64 << 20  # MOE_STATIC_WS_BYTES


class MoeError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"{STATUS_NAMES.get(status, status)}: {msg}")
        self.status = status


class Dims(ctypes.Structure):
    _fields_ = [("d_model", ctypes.c_int32), ("n_routed", ctypes.c_int32), ("d_ff", ctypes.c_int32),
                ("d_ff_shared", ctypes.c_int32), ("top_k", ctypes.c_int32), ("dtype", ctypes.c_int32),
                ("out_dtype", ctypes.c_int32), ("capacity", ctypes.c_int32), ("n_group", ctypes.c_int32),
                ("topk_group", ctypes.c_int32)]


class Weights(ctypes.Structure):
    _fields_ = [("w_router", ctypes.c_void_p), ("router_bias", ctypes.c_void_p), ("w1", ctypes.c_void_p),
                ("w3", ctypes.c_void_p), ("w2", ctypes.c_void_p), ("w1s", ctypes.c_void_p),
                ("w3s", ctypes.c_void_p), ("w2s", ctypes.c_void_p)]


class Options(ctypes.Structure):
    _fields_ = [("path", ctypes.c_int32), ("n_events", ctypes.c_int32), ("events", ctypes.POINTER(ctypes.c_void_p))]


class Diag(ctypes.Structure):
    _fields_ = [("flags", ctypes.c_uint32), ("tokens_exact", ctypes.c_uint32), ("exact_keys", ctypes.c_uint32),
                ("refinements", ctypes.c_uint32)]

    def as_dict(self):
        return {f: getattr(self, f) for f, _ in self._fields_}


_P = ctypes.c_void_p
_I64 = ctypes.c_int64
_SIG = {
    "moe_workspace_size": [ctypes.POINTER(Dims), _I64, ctypes.POINTER(ctypes.c_size_t)],
    "moe_router_topk": [ctypes.POINTER(Dims), _I64, _P, _P, _P, _P, _P, _P, ctypes.c_size_t, _P],
    "moe_permute": [ctypes.POINTER(Dims), _I64, _P, _P, _P, _P, _P, _P, ctypes.c_size_t, _P],
    "moe_expert_ffn": [ctypes.POINTER(Dims), _I64, _P, ctypes.POINTER(Weights), _P, _P, _P, _P, _P,
                       ctypes.POINTER(Options), _P, ctypes.c_size_t, _P],
    "moe_combine": [ctypes.POINTER(Dims), _I64, _P, _P, _P, _P, _P, _P],
    "moe_layer_forward": [ctypes.POINTER(Dims), _I64, _P, ctypes.POINTER(Weights), _P, ctypes.POINTER(Options), _P,
                          ctypes.c_size_t, _P],
    "moe_layer_forward_static": [ctypes.POINTER(Dims), _I64, _P, ctypes.POINTER(Weights), _P,
                                 ctypes.POINTER(Options), _P],
    "moe_rmsnorm": [ctypes.POINTER(Dims), _I64, _P, _P, ctypes.c_double, _P, _P],
    "moe_block_forward": [ctypes.POINTER(Dims), _I64, _P, _P, ctypes.c_double, ctypes.POINTER(Weights), _P,
                          ctypes.POINTER(Options), _P, ctypes.c_size_t, _P],
    "moe_read_diagnostics": [_P, ctypes.POINTER(Diag), _P],
}


def _ptr(x) -> Optional[int]:
    if x is None:
        return None
    if isinstance(x, int):
        return x
    return x.data_ptr()


def _stream(stream) -> Optional[int]:
    if stream is not None:
        return stream if isinstance(stream, int) else stream.cuda_stream
    import torch
    return torch.cuda.current_stream().cuda_stream


class Library:
    """The loaded C-ABI library.  Method names are the C names without the prefix."""

    def __init__(self, path: str = _LIB_PATH):
        if not os.path.exists(path):
            raise FileNotFoundError(f"{path} is missing: build it with __graft_entry__.build() "
                                    "or python -m fine_grained_routed_amd.build")
        self.path = path
        self.lib = ctypes.CDLL(path)
        for name, argtypes in _SIG.items():
            fn = getattr(self.lib, name)
            fn.argtypes = argtypes
            fn.restype = ctypes.c_int
        self.lib.moe_last_error.argtypes = []
        self.lib.moe_last_error.restype = ctypes.c_char_p

    # ---------------------------------------------------------------- helpers
    def last_error(self) -> str:
        return self.lib.moe_last_error().decode()

    def _check(self, status: int):
        if status != MOE_OK:
            raise MoeError(status, self.last_error())

    @staticmethod
    def dims(d_model, n_routed, d_ff, d_ff_shared, top_k, dtype=MOE_BF16, out_dtype=MOE_F32, capacity=0,
             n_group=0, topk_group=0) -> Dims:
        return Dims(d_model, n_routed, d_ff, d_ff_shared, top_k, dtype, out_dtype, capacity, n_group, topk_group)

    @staticmethod
    def weights(w_router=None, router_bias=None, w1=None, w3=None, w2=None, w1s=None, w3s=None, w2s=None) -> Weights:
        return Weights(_ptr(w_router), _ptr(router_bias), _ptr(w1), _ptr(w3), _ptr(w2), _ptr(w1s), _ptr(w3s),
                       _ptr(w2s))

    @staticmethod
    def options(path: int = PATH_AUTO, events: Optional[Sequence[int]] = None) -> Options:
        if not events:
            return Options(path, 0, None)
        arr = (ctypes.c_void_p * len(events))(*events)
        o = Options(path, len(events), ctypes.cast(arr, ctypes.POINTER(ctypes.c_void_p)))
        o._keep = arr  # keep the array alive with the struct
        return o

    # ------------------------------------------------------------- the C ABI
    def workspace_size(self, dims: Dims, T: int) -> int:
        out = ctypes.c_size_t(0)
        self._check(self.lib.moe_workspace_size(ctypes.byref(dims), T, ctypes.byref(out)))
        return out.value

    def router_topk(self, dims, T, u, w_router, router_bias, topk_idx, topk_w, ws, ws_bytes=None, stream=None):
        self._check(self.lib.moe_router_topk(ctypes.byref(dims), T, _ptr(u), _ptr(w_router), _ptr(router_bias),
                                             _ptr(topk_idx), _ptr(topk_w), _ptr(ws),
                                             ws.numel() * ws.element_size() if ws_bytes is None else ws_bytes,
                                             _stream(stream)))

    def permute(self, dims, T, topk_idx, counts, offsets, row_token, token_row, ws, ws_bytes=None, stream=None):
        self._check(self.lib.moe_permute(ctypes.byref(dims), T, _ptr(topk_idx), _ptr(counts), _ptr(offsets),
                                         _ptr(row_token), _ptr(token_row), _ptr(ws),
                                         ws.numel() * ws.element_size() if ws_bytes is None else ws_bytes,
                                         _stream(stream)))

    def expert_ffn(self, dims, T, u, weights: Weights, counts, offsets, row_token, y_rows, y_shared,
                   options: Optional[Options], ws, ws_bytes=None, stream=None):
        self._check(self.lib.moe_expert_ffn(ctypes.byref(dims), T, _ptr(u), ctypes.byref(weights), _ptr(counts),
                                            _ptr(offsets), _ptr(row_token), _ptr(y_rows), _ptr(y_shared),
                                            None if options is None else ctypes.byref(options), _ptr(ws),
                                            ws.numel() * ws.element_size() if ws_bytes is None else ws_bytes,
                                            _stream(stream)))

    def combine(self, dims, T, y_rows, y_shared, topk_w, token_row, out, stream=None):
        self._check(self.lib.moe_combine(ctypes.byref(dims), T, _ptr(y_rows), _ptr(y_shared), _ptr(topk_w),
                                         _ptr(token_row), _ptr(out), _stream(stream)))

    def layer_forward(self, dims, T, u, weights: Weights, out, options: Optional[Options], ws, ws_bytes=None,
                      stream=None):
        self._check(self.lib.moe_layer_forward(ctypes.byref(dims), T, _ptr(u), ctypes.byref(weights), _ptr(out),
                                               None if options is None else ctypes.byref(options), _ptr(ws),
                                               ws.numel() * ws.element_size() if ws_bytes is None else ws_bytes,
                                               _stream(stream)))

    def layer_forward_static(self, dims, T, u, weights: Weights, out, options: Optional[Options], stream=None):
        self._check(self.lib.moe_layer_forward_static(ctypes.byref(dims), T, _ptr(u), ctypes.byref(weights),
                                                      _ptr(out), None if options is None else ctypes.byref(options),
                                                      _stream(stream)))

    def rmsnorm(self, dims, T, x, norm_weight, eps, u, stream=None):
        self._check(self.lib.moe_rmsnorm(ctypes.byref(dims), T, _ptr(x), _ptr(norm_weight), float(eps), _ptr(u),
                                         _stream(stream)))

    def block_forward(self, dims, T, x, norm_weight, eps, weights: Weights, out, options: Optional[Options], ws,
                      ws_bytes=None, stream=None):
        self._check(self.lib.moe_block_forward(ctypes.byref(dims), T, _ptr(x), _ptr(norm_weight), float(eps),
                                               ctypes.byref(weights), _ptr(out),
                                               None if options is None else ctypes.byref(options), _ptr(ws),
                                               ws.numel() * ws.element_size() if ws_bytes is None else ws_bytes,
                                               _stream(stream)))

    def read_diagnostics(self, ws, stream=None) -> dict:
        d = Diag()
        self._check(self.lib.moe_read_diagnostics(_ptr(ws), ctypes.byref(d), _stream(stream)))
        return d.as_dict()


_LOADED: Optional[Library] = None


def load(path: str = _LIB_PATH) -> Library:
    """Load libmoe.so once; raises if it has not been built (no fallback path exists)."""
    global _LOADED
    if _LOADED is None or _LOADED.path != path:
        _LOADED = Library(path)
    return _LOADED
