"""Shared-prefix (cascade) attention for AMD MI355X (gfx950).

The compute path is ``libcascade_attn.so`` (C ABI in ``include/cascade_attn.h``):
a host planner in C++ and HIP kernels. This package only marshals arguments;
torch provides device memory and streams.
"""

from ._lib import (  # noqa: F401
    CascadeAttnError,
    Plan,
    cascade_attn_autotune,
    cascade_attn_autotune_record,
    cascade_attn_autotune_reset,
    cascade_attn_num_common_prefix_blocks,
    cascade_attn_plan,
    cascade_attn_plan_groups,
    cascade_attn_plan_info,
    cascade_attn_profile_enable,
    cascade_attn_profile_read,
    cascade_attn_run,
    cascade_attn_run_noalloc,
    cascade_attn_workspace_init,
    header_symbols,
    load,
)
from .api import kv_strides, plan_batch, run_batch  # noqa: F401
