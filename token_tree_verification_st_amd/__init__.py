"""Token-tree verification on MI355X (gfx950).

The target model's side of tree-based speculative decoding for one attention
layer, as hand-written HIP kernels behind a C ABI (include/st.h, libst.so):
ancestor mask, tree-masked split-KV attention, greedy and rejection-sampling
acceptance, KV compaction; and the layer pieces around them (embedding,
skinny bf16 projections, rotary embedding with the tree-KV append), and the
merge of candidate continuations into a token tree.  This package is the thin Python binding; torch
provides device memory and streams.
"""

from .binding import (  # noqa: F401
    LIB_PATH,
    ST_BF16,
    ST_F32,
    ST_MAX_NODES,
    Tree,
    decode_status,
    load_library,
    st_embed,
    st_kv_compact,
    st_kv_compact_paged,
    st_linear,
    st_linear_workspace,
    st_mask_words,
    st_status_str,
    st_stream_read,
    st_tree_attention,
    st_tree_attention_paged,
    st_tree_attention_workspace,
    st_tree_build,
    st_tree_mask,
    st_tree_rope_append,
    st_verification_step,
    st_verification_step_ex,
    st_verification_step_paged,
    st_verification_step_workspace,
    st_verify_greedy,
    st_verify_greedy_workspace,
    st_verify_stochastic,
    st_verify_stochastic_ex,
    st_verify_stochastic_workspace,
)
from .device_io import DeviceWorkload, to_device  # noqa: F401
from .policy import candidate_length  # noqa: F401
