"""fp64 CPU oracle of the MiTA attention forward pass (test infrastructure).

Only the tests, the smoke check and the CPU-baseline leg of the benchmark may
import this package. The GPU library never calls it, and it shares no code with
the GPU path: both take their inputs from ``synth`` and nothing else.
"""
from .mita_oracle import (  # noqa: F401
    adaptive_windows,
    pool,
    scores,
    shared_expert,
    full_attention,
    topk_experts,
    route_scores,
    route,
    attend,
    forward,
    topk_margins,
    route_margins,
    pool_matrix,
    attend_backward,
    shared_expert_backward,
    backward,
)
from .validity import valid_topk_sets, valid_route_sets  # noqa: F401
