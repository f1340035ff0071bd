"""MI355X (gfx950) fused reduce + residual-add + RMSNorm with a wave-aware
token-split planner, behind the C ABI in ``include/tokenweave.h``.

The Python names mirror the C entry points:

* :func:`tw_fused_reduce_rmsnorm` -- every row,
* :func:`tw_fused_reduce_rmsnorm_grid` -- every row on a fixed number of
  workgroups (the pages' few-CTA footprint),
* :func:`tw_shard_rmsnorm` -- one rank's token shard,
* :func:`tw_fused_launch_info` -- how a fused call would be launched (the
  geometry, the round of resident workgroups on the stream's CUs, the kernel),
* :func:`tw_split_plan` -- the prefix/suffix split plan,
* :func:`tw_split_plan_measured` -- the split plan with a measured per-shape
  offset table consulted first,
* :func:`tw_fused_reduce_rmsnorm_split` -- the two launches of a split,
* :func:`tw_reduce_partials`, :func:`tw_add_rmsnorm` and
  :func:`tw_unfused_reduce_rmsnorm` -- the unfused comparator (a standalone
  reduction, then a standard two-pass residual-add + RMSNorm).

:class:`PreparedFused` marshals a launch once for loops that repeat it, and
:class:`SplitPlanCache` keeps one split plan per token count, optionally taken
from a measured offline table (:func:`split_table_from_sweep`).
"""

from ._lib import (  # noqa: F401
    LIB_PATH,
    PLAN_REASONS,
    PreparedFused,
    SplitPlanCache,
    TokenWeaveError,
    declared_functions,
    load_library,
    split_table,
    split_table_from_sweep,
    tw_fused_reduce_rmsnorm,
    tw_fused_reduce_rmsnorm_grid,
    tw_fused_launch_info,
    tw_add_rmsnorm,
    tw_fused_reduce_rmsnorm_split,
    tw_reduce_partials,
    tw_set_pointer_checks,
    tw_shard_rmsnorm,
    tw_split_plan,
    tw_split_plan_measured,
    tw_unfused_reduce_rmsnorm,
)
