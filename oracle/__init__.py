"""CPU oracle for the hybrid attention prefill (test infrastructure only).

Only the tests, the smoke check and the bench's CPU-baseline leg import this
package; the product path never does."""
from .ea_oracle import (  # noqa: F401
    attention_weights,
    boundary_pool,
    boundary_rows,
    effective_flops,
    gelu,
    hybrid_attention,
    hybrid_attention_rows,
    linear,
    route,
    router_logits,
    router_param_count,
    sa_geometry,
    visible,
)
