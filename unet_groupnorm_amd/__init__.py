"""MI355X-native 3D GroupNorm (NCDHW or channels-last; fp32, bf16 or fp16 in; fp32
statistics) behind a C ABI.

The kernels live in libgn.so (csrc/); this package is its torch binding.
"""
from .gn import (  # noqa: F401
    GnError,
    GroupNormFn,
    as_layout,
    gn_backward,
    gn_backward_apply,
    gn_backward_finish,
    gn_backward_partials,
    gn_backward_reduce,
    gn_backward_shard_merge,
    gn_backward_shard_sums,
    gn_forward,
    gn_forward_apply,
    gn_forward_finish,
    gn_forward_noalloc,
    gn_forward_partials,
    gn_forward_shard_merge,
    gn_forward_shard_stats,
    gn_forward_stats,
    gn_plan_query,
    gn_plan_query_cl,
    gn_workspace_bytes,
    group_norm,
    layout_of,
    workspace_for,
)
