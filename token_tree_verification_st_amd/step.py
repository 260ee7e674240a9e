"""One verification step of one attention layer on the current stream:
acceptance (greedy or stochastic), tree attention and KV compaction, either as
the one-call st_verification_step (ancestor masks derived inside attention,
compaction in the launch that merges the attention splits) or as the sequence
of separate entry points, mask first.  Every call only enqueues kernels."""

from __future__ import annotations

from .binding import (st_kv_compact, st_tree_attention, st_tree_mask, st_verification_step,
                      st_verification_step_ex, st_verify_greedy, st_verify_stochastic,
                      st_verify_stochastic_ex)
from .device_io import DeviceWorkload


def run_mask(dw: DeviceWorkload):
    b = dw.buf
    st_tree_mask(dw.tree, b["mask"], b["depth"], b["status"])


def run_attention(dw: DeviceWorkload, scale=None, derive_mask: bool = False):
    """derive_mask: pass no mask, so the kernel derives it from the tree."""
    b = dw.buf
    st_tree_attention(dw.tree, dw.q, dw.k_cache, dw.v_cache, dw.prefix_len, dw.max_prefix,
                      None if derive_mask else b["mask"], b["out"], b["lse"], b["attn_ws"],
                      scale=scale, status=b["status"])


def run_verify(dw: DeviceWorkload, stochastic: bool, top_p: float = 1.0, draft=None):
    """draft: probabilities [T][V] to use instead of the draft logits."""
    b = dw.buf
    if stochastic and (top_p < 1.0 or draft is not None):
        st_verify_stochastic_ex(dw.tree, dw.tokens, dw.logits,
                                dw.draft_logits if draft is None else draft, dw.temperature,
                                dw.rng_seed, dw.rng_offset, b["accept_len"], b["accept_nodes"],
                                b["out_tokens"], b["verify_ws"], b["near_ties"], b["status"],
                                top_p=top_p, draft_is_probs=draft is not None)
    elif stochastic:
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


def run_step(dw: DeviceWorkload, stochastic: bool, top_p: float = 1.0, draft=None):
    """The whole step in one C-ABI call (draft: probabilities [T][V] to use
    instead of the draft logits)."""
    b = dw.buf
    if stochastic and (top_p < 1.0 or draft is not None):
        st_verification_step_ex(dw.tree, dw.q, dw.k_cache, dw.v_cache, dw.prefix_len,
                                dw.max_prefix, b["out"], b["lse"], dw.tokens, dw.logits,
                                b["accept_len"], b["accept_nodes"], b["out_tokens"], b["src_slot"],
                                b["new_len"], b["step_ws"],
                                dw.draft_logits if draft is None else draft,
                                temperature=dw.temperature, seed=dw.rng_seed,
                                offset=dw.rng_offset, near_ties=b["near_ties"],
                                status=b["status"], top_p=top_p,
                                draft_is_probs=draft is not None)
        return
    st_verification_step(dw.tree, dw.q, dw.k_cache, dw.v_cache, dw.prefix_len, dw.max_prefix,
                         b["out"], b["lse"], dw.tokens, dw.logits, b["accept_len"],
                         b["accept_nodes"], b["out_tokens"], b["src_slot"], b["new_len"],
                         b["step_ws"], draft_logits=dw.draft_logits if stochastic else None,
                         temperature=dw.temperature, seed=dw.rng_seed, offset=dw.rng_offset,
                         near_ties=b["near_ties"] if stochastic else None, status=b["status"])


def verification_step(dw: DeviceWorkload, stochastic: bool = False, verify: bool = True,
                      compact: bool = True, fused: bool = True, top_p: float = 1.0, draft=None):
    """One step: the one-call path when it applies (logits present, acceptance
    and compaction wanted), else mask -> attention -> acceptance -> compaction."""
    if fused and verify and compact and dw.V > 0:
        run_step(dw, stochastic, top_p=top_p, draft=draft)
        return
    run_mask(dw)
    run_attention(dw)
    if verify and dw.V > 0:
        run_verify(dw, stochastic, top_p=top_p, draft=draft)
        if compact:
            run_compact(dw)
