"""MI355X-native 3D GroupNorm (NCDHW, bf16/fp32 in, fp32 statistics) behind a C ABI.

The kernels live in libgn.so (csrc/); this package is its torch binding.
"""
from .gn import (  # noqa: F401
    GnError,
    GroupNormFn,
    gn_backward,
    gn_backward_apply,
    gn_backward_reduce,
    gn_forward,
    gn_forward_apply,
    gn_forward_stats,
    gn_plan_query,
    gn_workspace_bytes,
    group_norm,
    workspace_for,
)
