"""Plain, slow, obviously correct CPU oracle for the fused reduce + residual-add
+ RMSNorm step of TokenWeave and for its wave-aware split planner.

THIS PACKAGE IS TEST INFRASTRUCTURE.  Only the test suite (``tests/``), the
``smoke()`` entry of ``__graft_entry__`` and the ``cpu_baseline`` leg of
``bench.py`` may import it.  The product path (``reduce_rmsnorm_amd``) never
imports, calls or links anything here, and nothing here imports the product
path: the two share no code.

Sources, named by page title and section:

* [Blog] "TokenWeave: Why Hiding Tensor-Parallel Communication Needs Wave
  Arithmetic, Not Finer Tiles" (mohakchugh.is-a.dev), sections "The overlap
  trap", "Fix one: split at wave boundaries, unequally" and "Fix two: RMSNorm
  was never insignificant" (the per-CTA kernel sketch).
* [Guide] "TokenWeave Guide: Compute-Communication Overlap for LLMs"
  (aifetchly), section "Fused AllReduce-RMSNorm: Bypassing Global Memory",
  the RMSNorm equation.

``unfused`` holds the oracle of the unfused comparator (a standalone
reduction, then a standard two-pass residual-add + RMSNorm), [Blog] sections
"What it buys" and "Fix two".

Every numeric function is pinned by the ``-m "not gpu"`` tests against closed
forms, brute force with exact rationals, a library special case and the
worked wave example the pages print.  No function here is "parity unpinned".
"""

from .rmsnorm import (  # noqa: F401
    bf16_bits_to_f64,
    f32_to_f64,
    round_f64_to_bf16_bits,
    shard_rows,
    fused_reduce_rmsnorm,
    shard_rmsnorm,
)
from .unfused import (  # noqa: F401
    reduce_partials,
    add_rmsnorm_two_pass,
    unfused_reduce_rmsnorm,
)
from .planner import (  # noqa: F401
    DEFAULT_OFFSETS,
    REASON_SPLIT,
    REASON_BELOW_THRESHOLD,
    REASON_SINGLE_WAVE,
    REASON_NO_FEASIBLE_OFFSET,
    REASON_EMPTY,
    REASON_MEASURED_SPLIT,
    REASON_MEASURED_UNSPLIT,
    REASON_MEASURED_OVER_WAVES,
    ctas,
    waves,
    simulate_waves,
    split_plan,
    split_plan_measured,
)
