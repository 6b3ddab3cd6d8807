"""Parameter and combination accounting for fine-grained and shared experts.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Every function restates a counting rule from the pages in plain integer
arithmetic.  Nothing here is used by the HIP path.
"""
from __future__ import annotations

from typing import List, Tuple


def combinations(n_experts: int, top_k: int) -> int:
    """Number of distinct expert sets a top-k router can pick from n experts.

    "Shared and fine-grained experts", Researcher level, "Why segmentation
    helps": the reachable function class is indexed by the selected set, so its
    size is the binomial coefficient C(N, K); segmentation by m turns it into
    C(mN, mK).  Computed here as the product formula over exact integers.
    """
    if top_k < 0 or top_k > n_experts:
        return 0
    k = min(top_k, n_experts - top_k)
    num = 1
    den = 1
    for i in range(k):
        num *= n_experts - i
        den *= i + 1
    assert num % den == 0
    return num // den


def swiglu_matrix_shapes(d_model: int, d_ff: int) -> List[Tuple[str, int, int]]:
    """(name, rows, columns) of the three matrices one SwiGLU expert holds: the
    gate and up projections map the d_model-wide token to d_ff, the down
    projection maps back ("Shared Expert", How it works: FFN(u) = W2 (SiLU(W1 u)
    * W3 u), with W1, W3 of shape d_ff x d_model and W2 of shape d_model x d_ff)."""
    return [("gate", d_ff, d_model), ("up", d_ff, d_model), ("down", d_model, d_ff)]


def expert_budget(d_model: int, d_ff: int, n_routed: int, top_k: int, n_shared: int = 0) -> Tuple[int, int]:
    """(stored, active) expert weights of one MoE layer (biases ignored).

    MoE page in Chinese on fine-grained and shared experts, the section that
    equalises the budget: the stored count covers every routed and shared
    expert, the active count per token covers the top_k routed experts the
    router picks plus the always-on shared ones.  One expert's size is the
    sum of its matrices' element counts.  Shapes that cannot describe a layer
    raise ValueError.
    """
    if d_model < 1 or d_ff < 1:
        raise ValueError(f"expert matrices need positive sizes, got d_model={d_model}, d_ff={d_ff}")
    if n_routed < 1 or not 1 <= top_k <= n_routed:
        raise ValueError(f"need 1 <= top_k <= n_routed, got top_k={top_k}, n_routed={n_routed}")
    if n_shared < 0:
        raise ValueError(f"n_shared must be >= 0, got {n_shared}")
    size = sum(rows * cols for _, rows, cols in swiglu_matrix_shapes(d_model, d_ff))
    held = {"routed": n_routed, "shared": n_shared}
    used = {"routed": top_k, "shared": n_shared}
    return size * sum(held.values()), size * sum(used.values())


def layer_accounting(d_model: int, d_ff: int, n_routed: int, n_shared: int, top_k: int) -> dict:
    """Per-layer parameter accounting of a shared + routed MoE layer.

    "Shared and fine-grained experts", Developer level, DeepSeek-V3 accounting:
    each expert has gate, up and down projections (3*d*f); the layer stores all
    routed and shared experts plus the router (d weights per routed expert);
    a token activates its top-k routed experts, the shared experts and the
    whole router.
    """
    per_expert = 3 * d_model * d_ff
    router = d_model * n_routed
    total = (n_routed + n_shared) * per_expert + router
    active = (top_k + n_shared) * per_expert + router
    return {
        "per_expert": per_expert,
        "router": router,
        "total": total,
        "active": active,
        "active_fraction": active / total,
        "shared_params": n_shared * per_expert,
        # share of the active feed-forward work done by the shared experts
        "shared_share": n_shared / (top_k + n_shared),
    }


def granularity_rows(base_ff: int, n0: int, k0: int, ms: List[int]) -> List[dict]:
    """Fine-grained segmentation at constant compute per token.

    "Shared and fine-grained experts", Developer level, counting the
    combinations: splitting by m multiplies the expert count and top-k by m and
    divides the expert width by m (integer division), so the active width
    k*f stays fixed while the number of combinations grows.
    """
    rows = []
    for m in ms:
        n, k = n0 * m, k0 * m
        ff = base_ff // m
        rows.append({"m": m, "experts": n, "top_k": k, "expert_ff": ff,
                     "active_ff": k * ff, "combinations": combinations(n, k)})
    return rows


def sparsity(n_experts: int, top_k: int) -> float:
    """Fraction of routed experts active per token ("Expert Count Selection")."""
    return top_k / n_experts


def capacity_to_compute(n_experts: int, top_k: int) -> float:
    """Routed parameters held per routed parameter used ("Expert Count Selection")."""
    return n_experts / top_k

