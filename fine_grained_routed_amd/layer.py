"""Torch-facing convenience wrapper: allocates outputs and workspace with torch,
then calls the C ABI.  No arithmetic of the layer happens here."""
from __future__ import annotations

from typing import Dict, Optional, Sequence

import torch

from ._binding import MOE_BF16, MOE_F32, PATH_AUTO, Library, load

_DT = {torch.bfloat16: MOE_BF16, torch.float32: MOE_F32}


class MoELayer:
    """One shared + routed MoE FFN layer whose weights live on the GPU.

    weights: dict with w_router [N_r,d], w1/w3 [N_r,f,d], w2 [N_r,d,f],
    optional w1s/w3s [f_s,d], w2s [d,f_s] and router_bias [N_r] fp32.
    """

    def __init__(self, weights: Dict[str, Optional[torch.Tensor]], top_k: int, out_dtype=torch.float32,
                 lib: Optional[Library] = None):
        self.lib = lib or load()
        self.w = weights
        wr, w1 = weights["w_router"], weights["w1"]
        for name, t in weights.items():
            if t is not None and not t.is_contiguous():
                raise ValueError(f"{name} must be contiguous")
        self.E, self.d = wr.shape
        self.f = w1.shape[1]
        self.fs = 0 if weights.get("w1s") is None else weights["w1s"].shape[0]
        self.k = top_k
        self.dtype = wr.dtype
        self.out_dtype = out_dtype
        self.dims = self.lib.dims(self.d, self.E, self.f, self.fs, top_k, _DT[wr.dtype], _DT[out_dtype])
        self.cw = self.lib.weights(wr, weights.get("router_bias"), w1, weights["w3"], weights["w2"],
                                   weights.get("w1s"), weights.get("w3s"), weights.get("w2s"))
        self._ws = None

    @property
    def device(self):
        return self.w["w_router"].device

    def workspace(self, T: int) -> torch.Tensor:
        need = self.lib.workspace_size(self.dims, T)
        if self._ws is None or self._ws.numel() < need:
            self._ws = torch.empty(max(need, 256), dtype=torch.uint8, device=self.device)
        return self._ws

    # ------------------------------------------------------------- whole layer
    def forward(self, u: torch.Tensor, out: Optional[torch.Tensor] = None, path: int = PATH_AUTO,
                events: Optional[Sequence[int]] = None) -> torch.Tensor:
        T = u.shape[0]
        if out is None:
            out = torch.empty((T, self.d), dtype=self.out_dtype, device=self.device)
        ws = self.workspace(T)
        self.lib.layer_forward(self.dims, T, u, self.cw, out, self.lib.options(path, events), ws)
        return out

    __call__ = forward

    def diagnostics(self) -> dict:
        return self.lib.read_diagnostics(self._ws)

    # --------------------------------------------------------------- stages
    def router_topk(self, u: torch.Tensor):
        T = u.shape[0]
        idx = torch.empty((T, self.k), dtype=torch.int32, device=self.device)
        w = torch.empty((T, self.k), dtype=torch.float32, device=self.device)
        self.lib.router_topk(self.dims, T, u, self.w["w_router"], self.w.get("router_bias"), idx, w,
                             self.workspace(T))
        return idx, w

    def permute(self, topk_idx: torch.Tensor):
        T = topk_idx.shape[0]
        dev = self.device
        counts = torch.empty(self.E, dtype=torch.int32, device=dev)
        offsets = torch.empty(self.E + 1, dtype=torch.int32, device=dev)
        row_token = torch.empty(T * self.k, dtype=torch.int32, device=dev)
        token_row = torch.empty((T, self.k), dtype=torch.int32, device=dev)
        self.lib.permute(self.dims, T, topk_idx, counts, offsets, row_token, token_row, self.workspace(T))
        return counts, offsets, row_token, token_row

    def expert_ffn(self, u, counts, offsets, row_token, path: int = PATH_AUTO, events=None):
        T = u.shape[0]
        y_rows = torch.empty((T * self.k, self.d), dtype=torch.float32, device=self.device)
        y_sh = torch.empty((T, self.d), dtype=torch.float32, device=self.device) if self.fs else None
        self.lib.expert_ffn(self.dims, T, u, self.cw, counts, offsets, row_token, y_rows, y_sh,
                            self.lib.options(path, events), self.workspace(T))
        return y_rows, y_sh

    def combine(self, y_rows, y_shared, topk_w, token_row, out_dtype=None):
        T = topk_w.shape[0]
        out = torch.empty((T, self.d), dtype=out_dtype or self.out_dtype, device=self.device)
        dims = self.dims
        if out_dtype is not None and _DT[out_dtype] != dims.out_dtype:
            dims = self.lib.dims(self.d, self.E, self.f, self.fs, self.k, dims.dtype, _DT[out_dtype])
        self.lib.combine(dims, T, y_rows, y_shared, topk_w, token_row, out)
        return out
