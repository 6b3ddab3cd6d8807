"""Workload table and seeded synthetic inputs for one DeepSeekMoE-style MoE FFN layer.

This module is shared by the CPU oracle (``oracle/``), the tests and ``bench.py``.
It holds *no* arithmetic of the layer itself: it only draws the input tensors
(token activations ``u``, router weights, expert weights and an optional router
bias) from seeded generators, so that the oracle and the HIP path consume the
exact same bytes.

Recipe (the shapes come from the pages; the distributions are the workload's):

* ``u``: x ~ N(0, 1) drawn in fp32, RMS-normalised per token in fp64
  (u = x / sqrt(mean(x^2) + 1e-6), gain 1), rounded to fp32 (RNE), then to
  bf16 (RNE) for the bf16 workloads.  The layer input is already behind the
  block's pre-norm ("Shared Expert" page on DeepSeek-V3, How it works), so the
  normalisation belongs to the input recipe, not to the layer.
* every weight: 0.02 * N(0, 1) computed in fp32 (0.02 is the standard
  deviation), then rounded to bf16 (RNE) for the bf16 workloads.
* block inputs (the pre-norm residual stream, for the block entry point):
  x[t, :] = s_t * z_t with z_t ~ N(0, 1) and a per-token scale
  s_t = 2^N(0, 1) (so token norms spread over about a factor 4 either way),
  computed in fp32 and rounded to the workload dtype; the RMSNorm gain
  gamma = 1 + 0.1 * N(0, 1) in fp32; eps = NORM_EPS.
* dense workloads (no routed experts, top-k 0): the dense prefix FFN, whose
  weights are the "shared" triple w1s, w3s, w2s of width d_ff.
* skewed workloads: a per-expert router bias b_e = -1.2 * ln(e + 1) (a Zipf
  s = 1.2 profile over expert rank e + 1), rounded to fp32.  It is added to the
  router logits before the softmax.

Seeding: every (tensor, expert) slice and every 64-row block of ``u`` has its
own generator, seeded from (seed, family, tensor id, index).  The two DeepSeek-V3
workloads share a family, so the decode workload's 64 tokens are the first 64
tokens of the prefill workload and both use the same weights.  Tensors are drawn
with ``torch`` generators on the device they will live on (CPU: mt19937, GPU:
Philox), so CPU-drawn and GPU-drawn inputs differ; every comparison feeds both
sides from one draw.
"""
from __future__ import annotations

import dataclasses
import hashlib
from typing import Dict, Optional

import numpy as np
import torch

__all__ = [
    "Workload",
    "WORKLOADS",
    "get",
    "make_inputs",
    "to_f64",
    "sample_tokens",
    "ROW_BLOCK",
    "F64Experts",
    "make_block_inputs",
    "make_x",
    "make_gamma",
    "NORM_EPS",
]

ROW_BLOCK = 64  # rows of u drawn per generator
NORM_EPS = 1e-6  # RMSNorm epsilon of the block workloads


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    T: int
    d: int
    n_routed: int
    d_ff: int
    n_shared: int
    top_k: int
    dtype: str  # "f32" or "bf16": dtype of u and of every weight
    bias: Optional[str]  # None or "zipf1.2"
    family: str  # seed family: workloads that share weights share a family
    what: str

    @property
    def d_ff_shared(self) -> int:
        return self.n_shared * self.d_ff

    @property
    def rows(self) -> int:
        return self.T * self.top_k

    def with_T(self, T: int) -> "Workload":
        return dataclasses.replace(self, T=T)

    def flops(self, T: Optional[int] = None) -> int:
        """Algorithmic FLOP of one forward: router GEMM plus the 3 expert GEMMs
        of the k routed experts and the fused shared expert (2 FLOP per MAC)."""
        T = self.T if T is None else T
        return 2 * T * (self.d * self.n_routed + 3 * self.d * (self.top_k * self.d_ff + self.d_ff_shared))


# Shapes: "Shared and fine-grained experts" (granularity table; DeepSeek-V3 accounting),
# the equal-budget example on the Chinese page (先把"预算一样"算明白), "Expert Count
# Selection" (DeepSeek-MoE: 64 routed, top-6, 2 shared) and "Shared Expert" (fused
# shared width 2 x 1408; V3: 1 shared, 256 routed of width 2048).
WORKLOADS: Dict[str, Workload] = {
    w.name: w
    for w in [
        Workload("tiny_f32", 256, 128, 31, 64, 1, 7, "f32", None, "tiny",
                 "d=128, 31 routed f=64 + 1 shared f=64, top-7, fp32"),
        Workload("eqbudget_coarse", 4096, 128, 8, 256, 0, 2, "bf16", None, "eqc",
                 "equal budget (a): d=128, 8 routed f=256 top-2, no shared"),
        Workload("eqbudget_fine", 4096, 128, 32, 64, 0, 8, "bf16", None, "eqf",
                 "equal budget (b): d=128, 32 routed f=64 top-8, no shared"),
        Workload("dsmoe16b", 8192, 2048, 64, 1408, 2, 6, "bf16", None, "ds16b",
                 "DeepSeekMoE-16B-like: d=2048, 64 routed f=1408, 2 shared fused to 2816, top-6"),
        Workload("dsv3_prefill", 16384, 7168, 256, 2048, 1, 8, "bf16", None, "dsv3",
                 "DeepSeek-V3 MoE layer, prefill: d=7168, 256 routed f=2048 + 1 shared, top-8, T=16384"),
        Workload("dsv3_decode", 64, 7168, 256, 2048, 1, 8, "bf16", None, "dsv3",
                 "DeepSeek-V3 MoE layer, decode: same layer, T=64"),
        Workload("skew512", 8192, 2048, 512, 512, 1, 10, "bf16", "zipf1.2", "skew512",
                 "512 routed f=512 + 1 shared, top-10, Zipf(1.2) router bias"),
        Workload("skew128_top1", 8192, 2048, 128, 512, 1, 1, "bf16", "zipf1.2", "skew128",
                 "128 routed f=512 + 1 shared, top-1, Zipf(1.2) router bias"),
        Workload("dense_small", 1000, 256, 0, 640, 1, 0, "bf16", None, "dsmall",
                 "dense SwiGLU FFN (no routed experts): d=256, width 640"),
        Workload("dense_small_f32", 300, 128, 0, 192, 1, 0, "f32", None, "dsmallf",
                 "dense SwiGLU FFN (no routed experts): d=128, width 192, fp32"),
        Workload("dsv3_dense_prefill", 16384, 7168, 0, 18432, 1, 0, "bf16", None, "dsv3dense",
                 "DeepSeek-V3 dense prefix layer FFN: d=7168, width 18432, T=16384"),
        Workload("dsv3_dense_decode", 64, 7168, 0, 18432, 1, 0, "bf16", None, "dsv3dense",
                 "DeepSeek-V3 dense prefix layer FFN: same weights, T=64"),
    ]
}

TENSOR_IDS = {"u": 0, "w_router": 1, "w1": 2, "w3": 3, "w2": 4, "w1s": 5, "w3s": 6, "w2s": 7, "x": 8, "gamma": 9,
              "xscale": 10}


def get(name: str) -> Workload:
    return WORKLOADS[name]


def _seed(seed: int, family: str, tensor: str, index: int) -> int:
    key = f"{seed}/{family}/{TENSOR_IDS[tensor]}/{index}".encode()
    return int.from_bytes(hashlib.blake2b(key, digest_size=8).digest(), "little") & ((1 << 63) - 1)


def _randn(shape, seed: int, device) -> torch.Tensor:
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return torch.randn(shape, generator=g, device=device, dtype=torch.float32)


def _tdtype(dtype: str) -> torch.dtype:
    return {"f32": torch.float32, "bf16": torch.bfloat16}[dtype]


def make_u(wl: Workload, seed: int = 0, device="cpu", T: Optional[int] = None) -> torch.Tensor:
    """Token activations [T, d], RMS-normalised, in the workload dtype (row-major)."""
    T = wl.T if T is None else T
    out = torch.empty((T, wl.d), dtype=_tdtype(wl.dtype), device=device)
    for b in range((T + ROW_BLOCK - 1) // ROW_BLOCK):
        x = _randn((ROW_BLOCK, wl.d), _seed(seed, wl.family, "u", b), device).to(torch.float64)
        u = x / torch.sqrt((x * x).mean(dim=1, keepdim=True) + 1e-6)
        rows = min(ROW_BLOCK, T - b * ROW_BLOCK)
        out[b * ROW_BLOCK: b * ROW_BLOCK + rows] = u[:rows].to(torch.float32).to(out.dtype)
    return out


def _weight(shape, seed: int, dtype: str, device) -> torch.Tensor:
    return (_randn(shape, seed, device) * 0.02).to(_tdtype(dtype))


def make_weights(wl: Workload, seed: int = 0, device="cpu") -> Dict[str, Optional[torch.Tensor]]:
    """Router and expert weights in nn.Linear [out, in] layout, all row-major:
    w_router [N_r, d]; w1, w3 [N_r, f, d]; w2 [N_r, d, f];
    w1s, w3s [N_s*f, d]; w2s [d, N_s*f] (None when there is no shared expert);
    router_bias [N_r] fp32 or None."""
    dt = _tdtype(wl.dtype)
    E, d, f, fs = wl.n_routed, wl.d, wl.d_ff, wl.d_ff_shared
    w = {"w_router": _weight((E, d), _seed(seed, wl.family, "w_router", 0), wl.dtype, device)}
    for name, shp in (("w1", (f, d)), ("w3", (f, d)), ("w2", (d, f))):
        t = torch.empty((E,) + shp, dtype=dt, device=device)
        for e in range(E):
            t[e] = _weight(shp, _seed(seed, wl.family, name, e), wl.dtype, device)
        w[name] = t
    if fs > 0:
        w["w1s"] = _weight((fs, d), _seed(seed, wl.family, "w1s", 0), wl.dtype, device)
        w["w3s"] = _weight((fs, d), _seed(seed, wl.family, "w3s", 0), wl.dtype, device)
        w["w2s"] = _weight((d, fs), _seed(seed, wl.family, "w2s", 0), wl.dtype, device)
    else:
        w["w1s"] = w["w3s"] = w["w2s"] = None
    if wl.bias == "zipf1.2":
        ranks = np.arange(1, E + 1, dtype=np.float64)
        w["router_bias"] = torch.from_numpy((-1.2 * np.log(ranks)).astype(np.float32)).to(device)
    else:
        w["router_bias"] = None
    return w


def make_inputs(wl: Workload, seed: int = 0, device="cpu", T: Optional[int] = None):
    """All inputs of one layer forward: dict with ``u`` plus the weights."""
    inp = make_weights(wl, seed, device)
    inp["u"] = make_u(wl, seed, device, T)
    return inp


def make_x(wl: Workload, seed: int = 0, device="cpu", T: Optional[int] = None) -> torch.Tensor:
    """Raw residual stream [T, d] (before the pre-norm), in the workload dtype."""
    T = wl.T if T is None else T
    out = torch.empty((T, wl.d), dtype=_tdtype(wl.dtype), device=device)
    for b in range((T + ROW_BLOCK - 1) // ROW_BLOCK):
        z = _randn((ROW_BLOCK, wl.d), _seed(seed, wl.family, "x", b), device)
        s = torch.exp2(_randn((ROW_BLOCK, 1), _seed(seed, wl.family, "xscale", b), device))
        rows = min(ROW_BLOCK, T - b * ROW_BLOCK)
        out[b * ROW_BLOCK: b * ROW_BLOCK + rows] = (z * s)[:rows].to(out.dtype)
    return out


def make_gamma(wl: Workload, seed: int = 0, device="cpu") -> torch.Tensor:
    """RMSNorm gain [d] fp32."""
    return 1.0 + 0.1 * _randn((wl.d,), _seed(seed, wl.family, "gamma", 0), device)


def make_block_inputs(wl: Workload, seed: int = 0, device="cpu", T: Optional[int] = None):
    """Inputs of one pre-norm block: the weights, the raw stream ``x`` and the
    RMSNorm gain ``gamma`` [d] fp32 (no ``u``: the block computes it)."""
    inp = make_weights(wl, seed, device)
    inp["x"] = make_x(wl, seed, device, T)
    inp["gamma"] = make_gamma(wl, seed, device)
    return inp


def to_f64(t: Optional[torch.Tensor]) -> Optional[np.ndarray]:
    """Exact conversion of a bf16/fp32 tensor (any device) to a host fp64 array."""
    if t is None:
        return None
    return t.detach().to("cpu").to(torch.float64).numpy()


def sample_tokens(T: int, n: int, seed: int = 0) -> np.ndarray:
    """A seeded, sorted sample of n distinct token indices in [0, T)."""
    n = min(n, T)
    rng = np.random.default_rng([seed, T, n, 7])
    return np.sort(rng.choice(T, size=n, replace=False)).astype(np.int64)


class F64Experts:
    """Indexable view of a stacked weight tensor [E, ...] (any device) whose
    item e is expert e's matrix as a host fp64 array (exact widening).  Lets
    the oracle walk large expert stacks one expert at a time."""

    def __init__(self, t: torch.Tensor):
        self.t = t

    def __len__(self):
        return self.t.shape[0]

    def __getitem__(self, e: int) -> np.ndarray:
        return self.t[e].to(torch.float64).to("cpu").numpy()
