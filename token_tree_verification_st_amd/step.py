"""One verification step of one attention layer, as a sequence of C-ABI calls
on the current stream: ancestor mask -> tree attention -> acceptance (greedy or
stochastic) -> KV compaction.  Every call only enqueues kernels."""

from __future__ import annotations

from .binding import (st_kv_compact, st_tree_attention, st_tree_mask, st_verify_greedy,
                      st_verify_stochastic)
from .device_io import DeviceWorkload


def run_mask(dw: DeviceWorkload):
    b = dw.buf
    st_tree_mask(dw.tree, b["mask"], b["depth"], b["status"])


def run_attention(dw: DeviceWorkload, scale=None):
    b = dw.buf
    st_tree_attention(dw.tree, dw.q, dw.k_cache, dw.v_cache, dw.prefix_len, dw.max_prefix,
                      b["mask"], b["out"], b["lse"], b["attn_ws"], scale=scale,
                      status=b["status"])


def run_verify(dw: DeviceWorkload, stochastic: bool):
    b = dw.buf
    if stochastic:
        st_verify_stochastic(dw.tree, dw.tokens, dw.logits, dw.draft_logits, dw.temperature,
                             dw.rng_seed, dw.rng_offset, b["accept_len"], b["accept_nodes"],
                             b["out_tokens"], b["verify_ws"], b["near_ties"], b["status"])
    else:
        st_verify_greedy(dw.tree, dw.tokens, dw.logits, b["accept_len"], b["accept_nodes"],
                         b["out_tokens"], b["verify_ws"], b["status"])


def run_compact(dw: DeviceWorkload):
    b = dw.buf
    st_kv_compact(dw.k_cache, dw.v_cache, dw.prefix_len, b["accept_len"], b["accept_nodes"],
                  b["src_slot"], b["new_len"], b["status"])


def verification_step(dw: DeviceWorkload, stochastic: bool = False, verify: bool = True,
                      compact: bool = True):
    """mask -> attention -> acceptance -> compaction (acceptance and compaction
    need logits)."""
    run_mask(dw)
    run_attention(dw)
    if verify and dw.V > 0:
        run_verify(dw, stochastic)
        if compact:
            run_compact(dw)
