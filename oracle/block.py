"""Oracle of the steps on either side of the MoE layer, and of the dense prefix FFN.

TEST INFRASTRUCTURE ONLY (see the package docstring).  Shares no code with the
HIP path.

* The pre-norm block: the layer input is the RMS-normalised residual stream
  and the block adds its output back to the raw stream ("Shared Expert" page on
  DeepSeek-V3: How it works -- eq. 12's leading residual term, applied at block
  level in the official graph, while MoE.forward returns shared + routed only;
  Watch-outs -- the shared experts sit behind the FFN pre-norm too).
* The dense prefix layers: "Shared and fine-grained experts" (Developer
  level, after the table of configs: DeepSeek-V3's first three layers have no
  experts, and their feed-forward block is a plain SwiGLU 18432 wide) and "Shared Expert"
  (Official code: the MLP class is the same SwiGLU as a dense prefix layer).

Readings taken where the pages are silent (each also listed in the design
notes): RMSNorm is x / sqrt(mean(x^2) + eps) times a per-channel gain; the
normalised input is stored in the layer's compute dtype (rounded once, to
nearest, ties to even) before the layer reads it; the residual added is the
raw, un-normalised block input.
"""
from __future__ import annotations

from typing import Optional

import numpy as np

from .moe_oracle import forward, swiglu


def _f64(x) -> np.ndarray:
    return np.asarray(x, dtype=np.float64)


def round_to_bf16(x) -> np.ndarray:
    """Nearest bfloat16 value of each fp64 element, ties to even, as fp64.

    bfloat16 keeps 8 significant bits and fp32's exponent range: normal values
    in [2^e', 2^(e'+1)) sit on a grid of spacing 2^(e'-7); below 2^-126 the
    grid spacing stays 2^-133 (subnormals); magnitudes that round to 2^128 or
    beyond overflow to infinity.  Written from that definition: scale by the
    grid spacing, round to the nearest integer with ties to even, scale back.
    """
    x = _f64(x)
    out = x.copy()
    fin = np.isfinite(x) & (x != 0.0)
    _, e = np.frexp(x[fin])  # |x| = m * 2^e with 0.5 <= m < 1, so 2^(e-1) <= |x| < 2^e
    q = np.maximum(e - 8, -133)  # grid spacing 2^q
    r = np.ldexp(np.rint(np.ldexp(x[fin], -q)), q)
    r[np.abs(r) >= 2.0 ** 128] = np.copysign(np.inf, r[np.abs(r) >= 2.0 ** 128])
    out[fin] = r
    return out


def store(x, dtype: str) -> np.ndarray:
    """Round fp64 values to the stored dtype ("bf16" or "f32"), returned as fp64."""
    if dtype == "bf16":
        return round_to_bf16(x)
    if dtype == "f32":
        return _f64(x).astype(np.float32).astype(np.float64)
    raise ValueError(dtype)


def rms_norm(x, gamma, eps: float) -> np.ndarray:
    """RMSNorm of each row in fp64, unrounded: x / sqrt(mean(x^2) + eps) * gamma."""
    x = _f64(x)
    ms = np.mean(x * x, axis=1, keepdims=True)
    return x / np.sqrt(ms + eps) * _f64(gamma)[None, :]


def dense_ffn(x, w1, w3, w2) -> np.ndarray:
    """The dense prefix layers' feed-forward block: one SwiGLU over all tokens,
    W2 (SiLU(W1 x) * W3 x), weights [width, d], [width, d], [d, width]."""
    return swiglu(x, w1, w3, w2)


def block_forward(x, gamma, eps: float, dtype: str, w_router=None, w1=None, w3=None, w2=None, k: int = 0,
                  bias=None, w1s=None, w3s=None, w2s=None, capacity: Optional[int] = None):
    """Pre-norm FFN block: h' = x + FFN(u) with u = RMSNorm(x) stored in ``dtype``.

    With routed experts (k >= 1) FFN is the MoE layer (shared + routed); with
    none (w_router None, k = 0) it is the dense SwiGLU of the shared weights
    (a dense prefix layer).  Returns a dict with the stored u, the FFN output
    and the block output ``out``."""
    x = _f64(x)
    u = store(rms_norm(x, gamma, eps), dtype)
    if k == 0:
        r = {"ffn": dense_ffn(u, w1s, w3s, w2s)}
    else:
        r = forward(u, w_router, w1, w3, w2, k, bias, w1s, w3s, w2s, capacity)
        r["ffn"] = r["out"]
    r["u"] = u
    r["out"] = x + r["ffn"]
    return r
