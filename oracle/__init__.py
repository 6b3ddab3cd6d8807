"""CPU oracle for the DeepSeekMoE-style MoE FFN layer forward.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or run
anything in this package: only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` use it.  It shares no code with the HIP
path (``fine_grained_routed_amd``); the two meet only in the input bytes drawn
by ``workloads``.
"""
from .moe_oracle import (  # noqa: F401
    router_logits,
    exact_logit,
    route,
    softmax,
    permute,
    silu,
    swiglu,
    expert_ffn,
    combine,
    forward,
    forward_dense,
    capacity_seats,
)
from .block import (  # noqa: F401
    round_to_bf16,
    store,
    rms_norm,
    dense_ffn,
    block_forward,
)
from .accounting import (  # noqa: F401
    combinations,
    expert_budget,
    layer_accounting,
    granularity_rows,
)
