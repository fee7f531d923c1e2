"""MI355X-native batched inverse fourth root for Shampoo-style block preconditioners (DASH).

The compute lives in ``libdash.so`` (hand-written HIP for gfx950, C ABI in ``include/dash.h``).
This package is its thin Python binding: every function takes torch tensors for device memory,
passes their pointers and the current HIP stream through ctypes, and raises :class:`DashError` on
a non-OK status.  There is no CPU fallback: if the library is missing, importing a call raises.
"""
from ._lib import (  # noqa: F401
    DASH_BF16,
    DASH_FP16,
    DASH_FP32,
    DASH_OP_APPLY,
    DASH_OP_CHEB,
    DASH_OP_CN,
    DASH_OP_EVD,
    DASH_OP_NDB,
    DASH_OP_SCALE,
    DASH_OP_STATS,
    DASH_SCALE_FROBENIUS,
    DASH_SCALE_POWER,
    DashError,
    dash_abi_version,
    dash_apply,
    dash_flops,
    dash_inverse_root_cheb,
    dash_inverse_root_cn,
    dash_inverse_root_cn_adaptive,
    dash_inverse_root_evd,
    dash_inverse_root_ndb,
    dash_inverse_root_ndb_adaptive,
    dash_inverse_root_ndb_half,
    dash_inverse_root_ndb_lowp,
    dash_scale,
    dash_solver_products,
    dash_stack,
    dash_status_string,
    dash_unstack,
    dash_update_stats,
    dash_workspace_size,
    library,
    library_path,
    workspace,
)
