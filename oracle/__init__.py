"""CPU oracle for the routed MoE FFN forward pass -- test infrastructure only.

Only the tests, the smoke check and the benchmark's CPU-baseline leg may import
this package. The product path (the HIP library and its Python binding) never
imports it and shares no code with it. `oracle.balance` holds the two
load-balancing statistics (the auxiliary loss and Quantile Balancing) and
`oracle.latent` the Stable LatentMoE layer, `oracle.mx` the MX formats and
the MX expert FFN.
"""
from .moe_oracle import (  # noqa: F401
    combine,
    expert_ffn,
    expert_swiglu,
    forward,
    gate_logits,
    gather,
    permute,
    renormalise,
    route,
    silu,
    softmax,
    topk_indices,
)
