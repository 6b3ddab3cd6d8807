"""Torch-facing convenience wrapper: allocates outputs and workspace with torch,
then calls the C ABI.  No arithmetic of the layer happens here."""
from __future__ import annotations

from typing import Dict, Optional, Sequence

import torch

from ._binding import MOE_BF16, MOE_F32, PATH_AUTO, Library, load

_DT = {torch.bfloat16: MOE_BF16, torch.float32: MOE_F32}


def capacity_seats(capacity_factor, T: int, top_k: int, n_routed: int) -> int:
    """Caller-side sizing of the per-expert seat limit the library takes as an
    integer: ceil(cf * T * top_k / n_routed), in exact rational arithmetic on
    the value of cf (a float counts as its binary value).  "What is an
    'expert', really?", glossary: capacity is a seat limit per expert, set as
    a multiple of the even share of the batch's assignments."""
    from fractions import Fraction
    q = Fraction(capacity_factor) * T * top_k / n_routed
    return -((-q.numerator) // q.denominator)


class MoELayer:
    """One shared + routed MoE FFN layer (or a dense FFN layer) whose weights live on the GPU.

    weights: dict with w_router [N_r,d], w1/w3 [N_r,f,d], w2 [N_r,d,f],
    optional w1s/w3s [f_s,d], w2s [d,f_s] and router_bias [N_r] fp32.  A dense
    layer has top_k == 0 and no routed experts (w_router None or with 0 rows);
    its MLP is w1s/w3s/w2s.  capacity: seats per routed expert (0 = no limit).
    n_group, topk_group: group-limited routing (n_group <= 1: none).
    """

    def __init__(self, weights: Dict[str, Optional[torch.Tensor]], top_k: int, out_dtype=torch.float32,
                 lib: Optional[Library] = None, capacity: int = 0, n_group: int = 0, topk_group: int = 0):
        self.lib = lib or load()
        self.w = weights
        for name, t in weights.items():
            if t is not None and not t.is_contiguous():
                raise ValueError(f"{name} must be contiguous")
        wr, w1, w1s = weights.get("w_router"), weights.get("w1"), weights.get("w1s")
        ref = w1s if wr is None or wr.shape[0] == 0 else wr
        self.E = 0 if wr is None else wr.shape[0]
        self.d = ref.shape[1]
        self.f = 0 if w1 is None or self.E == 0 else w1.shape[1]
        self.fs = 0 if w1s is None else w1s.shape[0]
        self.k = top_k
        self.dtype = ref.dtype
        self.out_dtype = out_dtype
        self.capacity = capacity
        self.n_group, self.topk_group = n_group, topk_group
        self.dims = self.lib.dims(self.d, self.E, self.f, self.fs, top_k, _DT[ref.dtype], _DT[out_dtype], capacity,
                                  n_group, topk_group)
        routed = self.E > 0
        self.cw = self.lib.weights(wr if routed else None, weights.get("router_bias") if routed else None,
                                   w1 if routed else None, weights.get("w3") if routed else None,
                                   weights.get("w2") if routed else None, w1s, weights.get("w3s"), weights.get("w2s"))
        self._ws = None

    @property
    def device(self):
        return next(t for t in self.w.values() if t is not None).device

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

    def block_forward(self, x: torch.Tensor, norm_weight: torch.Tensor, eps: float,
                      out: Optional[torch.Tensor] = None, path: int = PATH_AUTO,
                      events: Optional[Sequence[int]] = None) -> torch.Tensor:
        """Pre-norm block: x + layer(RMSNorm(x)); norm_weight [d] fp32."""
        T = x.shape[0]
        if out is None:
            out = torch.empty((T, self.d), dtype=self.out_dtype, device=self.device)
        ws = self.workspace(T)
        self.lib.block_forward(self.dims, T, x, norm_weight, eps, self.cw, out, self.lib.options(path, events), ws)
        return out

    def rmsnorm(self, x: torch.Tensor, norm_weight: torch.Tensor, eps: float) -> torch.Tensor:
        u = torch.empty_like(x)
        self.lib.rmsnorm(self.dims, x.shape[0], x, norm_weight, eps, u)
        return u

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
        T = (topk_w if topk_w is not None else y_shared).shape[0]
        out = torch.empty((T, self.d), dtype=out_dtype or self.out_dtype, device=self.device)
        dims = self.dims
        if out_dtype is not None and _DT[out_dtype] != dims.out_dtype:
            dims = self.lib.dims(self.d, self.E, self.f, self.fs, self.k, dims.dtype, _DT[out_dtype], self.capacity,
                                 self.n_group, self.topk_group)
        self.lib.combine(dims, T, y_rows, y_shared, topk_w, token_row, out)
        return out
