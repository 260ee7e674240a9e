"""Seeded synthetic inputs for token-tree verification.

This module is shared by the tests, the benchmark and the smoke check. It only
draws random inputs: tree shapes (parent-pointer arrays), query rows, key/value
caches, target and draft logits and draft tokens. It computes none of the
verification method (no mask, no attention, no acceptance, no compaction), so
the CPU oracle and the HIP path stay independent of each other.

Every array is produced by ``numpy.random.Generator(PCG64(seed))``; bf16 values
are rounded from float32 with round-to-nearest-even and handed out as their raw
16-bit patterns, so both sides read identical bytes.
"""

from .workloads import (  # noqa: F401
    Workload,
    WORKLOADS,
    make_workload,
    build_workload,
    f32_to_bf16_bits,
    tree_complete_binary,
    tree_chain,
    tree_random_attach,
    tree_beam_plus_leaves,
)
from .model import model_config, model_weights  # noqa: F401,E402
from .candidates import make_candidates, TREE_BUILD_CASE  # noqa: F401,E402
from .paged import make_paged  # noqa: F401,E402
