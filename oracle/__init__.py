"""fp64 CPU oracle for core attention — TEST INFRASTRUCTURE ONLY.

This package is the checker, not the product.  Only the test suite, the
``smoke()`` self-check and the benchmark's ``cpu_baseline`` leg may import it.
It shares no code with the HIP library: it depends on numpy alone and imports
nothing from ``long_context_core_amd``.

Modules
-------
attention  forward / merge / backward / decode written as the plain definition
           of softmax(scale * Q K^T + mask) V, in float64.
counting   unmasked (query, key) pair counts and the FLOP convention.
scheduler  the profiler cost model, Appendix-B shard sizing and the
           communication-aware greedy placement of CA-tasks on servers.
paging     attention over paged K/V (block tables): the virtual K/V a table
           describes, then the plain forward.
ring       context-parallel ring planning: the pass-KV / pass-Q time model,
           thresholds and switching rules, load-balanced sharding, the pass-KV
           ring schedule and round-robin decode sharding.

Parity status of every function is stated in its own docstring; all of them
are pinned by ``tests/test_*oracle_pins.py`` except where a docstring says
"parity unpinned".
"""

from .attention import (  # noqa: F401
    TASK_FIELDS,
    MASK_FIELDS,
    bf16_bits_to_f64,
    visible_mask,
    forward,
    forward_rows,
    merge,
    backward,
    backward_dq_rows,
    forward_listed,
    backward_listed,
)
from .paging import virtual_rows, forward_paged, backward_paged  # noqa: F401
from .counting import (  # noqa: F401
    visible_pairs_task,
    visible_pairs_masked,
    visible_pairs,
    forward_flops,
    backward_flops,
)
