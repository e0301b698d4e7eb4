"""fp64 CPU oracle of the self-attention block -- test infrastructure only.

Only ``tests/``, ``__graft_entry__.smoke()`` and ``bench.py``'s ``cpu_baseline``
leg may import this package. The HIP library never does.
"""

from .mha import (  # noqa: F401
    as_f64, attention, block_forward, merge_heads, merge_partials,
    partial_attention, project, rms_norm, scale_query, split_heads, stack_forward,
)
from . import shares  # noqa: F401,E402
