"""Plain fp64 CPU oracle for shared-prefix (cascade) attention.

TEST INFRASTRUCTURE ONLY. Nothing on the product path may import, call or
execute anything in this package: only ``tests/``, ``__graft_entry__.smoke()``
and the ``cpu_baseline`` leg of ``bench.py`` use it. It shares no code with the
HIP library (no kernels, headers, helpers or constants) and imports nothing
from it.

Sources (the pages the method is described on):

* [p2] "vLLM Cascade Attention：用法、场景与原理解析" (beaiera.top) -- the
  three-step method (section 1), the R1/R2 prefix/suffix example (section 4),
  the KV-load calculation (section 5), the trigger thresholds (section 3) and
  the scheduler / model-runner steps (section 8, Steps 1-5).
* [p3] "fix(v1/kv_cache): resolve async KV transfer bug in cascade attention
  #23485" -- the common-prefix block count is over the running requests only.
* [p1] "Diary - vLLM's cascade attention" -- cascade must not change the
  result; the failure it reports is output that depends on batch composition.

Every function in ``cascade_ref`` has at least one independent pin in
``tests/test_oracle.py``; none is "parity unpinned".
"""

from .cascade_ref import (  # noqa: F401
    attend,
    attention_full,
    merge_states,
    common_prefix_blocks,
    cascade_prefix_len,
    passes_cascade_gates,
    kv_tokens_standard,
    kv_tokens_cascade,
    level1_groups,
    kv_tokens_multilevel,
    tree_groups,
    kv_tokens_tree,
    fp8_e4m3_decode,
    MIN_PREFIX_TOKENS,
    MIN_NUM_REQS,
)
