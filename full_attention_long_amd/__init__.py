"""MI355X-native head-routed hybrid attention prefill (Elastic Attention's inference path).

The compute lives in libea.so (HIP for gfx950, C ABI in include/ea.h); this
package holds the ctypes binding and the host-side bookkeeping used to report
throughput.
"""
from .binding import (  # noqa: F401
    EAError,
    HEAD_CONFIGS,
    KVCache,
    KVCacheDesc,
    XAParams,
    ea_decode_step,
    ea_decode_workspace_size,
    ea_kvcache_bytes,
    ea_kvcache_init,
    ea_kvcache_prefill,
    ea_abi_version,
    ea_dual_prefill,
    ea_dual_prefill_workspace_size,
    ea_gumbel_route,
    ea_hybrid_backward,
    ea_hybrid_backward_workspace_size,
    ea_hybrid_prefill,
    ea_hybrid_prefill_noalloc,
    ea_hybrid_prefill_noalloc_max_workspace,
    ea_hybrid_prefill_plan,
    ea_hybrid_prefill_plan_layout,
    ea_hybrid_prefill_run,
    ea_hybrid_prefill_workspace_size,
    ea_last_error,
    ea_workspace_status,
    ea_mfma_probe,
    ea_route,
    ea_router_logit_grad,
    ea_router_logit_grad_workspace_size,
    ea_xa_prefill,
    ea_xa_prefill_plan,
    ea_xa_prefill_run,
    ea_xa_prefill_workspace_size,
    header_functions,
    lib,
)
