"""CPU oracle for token-tree verification -- TEST INFRASTRUCTURE ONLY.

A plain, slow, obviously correct NumPy implementation (fp64 wherever floating
point is involved) of what the verification path computes: the ancestor mask
of a parent-pointer token tree, tree-masked attention over a shared prefix KV
cache, greedy and rejection-sampling acceptance down the tree, and compaction
of the accepted path's KV rows.  It exists to check the HIP library against.

Only the tests, ``__graft_entry__.smoke()`` and the benchmark's CPU-baseline
leg may import it.  It shares no code with the HIP path: it never imports the
``token_tree_verification_st_amd`` package and that package never imports it.

Sources (web pages, cited by title and section):
  [SpecInfer-news]  SpecInfer news article (sunluscious.com.cn), sections
                    "研究現狀" (incremental decoding) and "Token 樹驗證器"
                    (token tree, tree attention through a constructed mask,
                    depth-first KV-cache update)
  [SpecInfer-dev]   "SpecInfer：基于树结构的LLM推测性推理加速技术", §2.1
                    (tree node with parent pointer; tree_attention with a
                    [batch, heads, seq, seq] mask; longest verified prefix)
  [Specular]        Specular project page, "主要特性" (greedy output identical
                    to the original model's)
  [SpecDec]         speculative-decoding explainer (intelliparadigm.com),
                    §2.2 (acceptance probability min(1, p_main/p_draft),
                    left-to-right check, replacement at the first rejection,
                    equal-distribution guarantee), §3.2 (single forward pass)

Token-tree construction (build.py) merges candidate sequences into the tree
that verification takes; paged.py describes a paged KV pool by the contiguous
caches its block table names.

Every function is pinned by tests marked ``not gpu`` (closed forms, brute
force, invariants, library routines, hand-worked fixtures in tests/golden).
The exact decision rule of the stochastic walk (order of siblings, residual
renormalisation, inverse-CDF order) is a reading of the pages that they do
not fix bit for bit; its distributional behaviour is pinned, its bit-level
choices are "parity unpinned" beyond GPU-vs-oracle agreement.
"""

from .tree import (  # noqa: F401
    STATUS_BAD_PARENT,
    STATUS_BAD_TOKEN,
    STATUS_NONFINITE,
    STATUS_PATH_OVERFLOW,
    check_tree,
    root_path,
    depth_of,
    children_of,
    dense_tree_mask,
    pack_mask_bits,
    tree_mask,
)
from .attention import decode_values, tree_attention  # noqa: F401
from .philox import philox4x64_10, uniforms_for_node  # noqa: F401
from .verify import (nucleus, nucleus_variants, stochastic_outcomes,  # noqa: F401
                     verify_greedy, verify_stochastic)
from .compact import kv_compact  # noqa: F401
from .layer import (  # noqa: F401
    ROPE_THETA,
    ar_greedy_decode,
    linear,
    node_positions,
    prefix_cache,
    rope,
    rope_angles,
    tree_layer,
)
from .build import build_tree, pack_trees  # noqa: F401,E402
from .paged import gather_paged, kv_compact_paged, scatter_paged  # noqa: F401,E402
