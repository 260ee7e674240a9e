"""One attention layer of a target model verifying a token tree, as a
sequence of C-ABI calls on the current stream (plumbing only; every step runs
in the library's kernels):

    x = E[tokens]                          st_embed
    qkv = x Wqkv^T                         st_linear
    q, k, v -> rotary at P_b + depth,
    k, v appended at slots P_b + i         st_tree_rope_append
    a = tree attention (masks derived)     st_tree_attention
    h = x + a Wo^T                         st_linear (residual)
    logits = h Wlm^T                       st_linear (fp32 out)
    greedy or stochastic acceptance        st_verify_greedy / st_verify_stochastic
    accepted path moved to P_b..P_b+L      st_kv_compact

Weights are bf16 [out][in]; hidden size d = Hq * D."""

from __future__ import annotations

from dataclasses import dataclass, field
from typing import Dict, Optional

import torch

from .binding import (Tree, st_embed, st_kv_compact, st_linear, st_linear_workspace,
                      st_tree_attention, st_tree_attention_workspace, st_tree_rope_append,
                      st_verify_greedy, st_verify_greedy_workspace, st_verify_stochastic,
                      st_verify_stochastic_workspace)


@dataclass
class LayerWeights:
    E: torch.Tensor      # [V][d]
    Wqkv: torch.Tensor   # [(Hq + 2 Hkv) D][d]
    Wo: torch.Tensor     # [d][Hq D]
    Wlm: torch.Tensor    # [V][d]
    Hq: int
    Hkv: int
    D: int
    theta: float = 10000.0

    @property
    def V(self) -> int:
        return self.E.shape[0]

    @property
    def d(self) -> int:
        return self.E.shape[1]


@dataclass
class LayerBuffers:
    """Activations, outputs and workspaces of one layer step for T nodes."""
    T: int
    buf: Dict[str, torch.Tensor] = field(default_factory=dict)


def layer_buffers(w: LayerWeights, tree: Tree, max_prefix: int, stochastic: bool = False,
                  device="cuda") -> LayerBuffers:
    T, B = tree.T, tree.B
    Hq, Hkv, D, d, V = w.Hq, w.Hkv, w.D, w.d, w.V
    bf = dict(dtype=torch.bfloat16, device=device)
    i32 = dict(dtype=torch.int32, device=device)
    u8 = dict(dtype=torch.uint8, device=device)

    def ws(n):
        return torch.empty(max(int(n), 16), **u8)

    b = dict(
        x=torch.empty(T, d, **bf),
        qkv=torch.empty(T, (Hq + 2 * Hkv) * D, **bf),
        q=torch.empty(T, Hq, D, **bf),
        attn=torch.empty(T, Hq, D, **bf),
        h=torch.empty(T, d, **bf),
        logits=torch.empty(T, V, dtype=torch.float32, device=device),
        ws_qkv=ws(st_linear_workspace(T, (Hq + 2 * Hkv) * D, d)),
        ws_o=ws(st_linear_workspace(T, d, Hq * D)),
        ws_lm=ws(st_linear_workspace(T, V, d)),
        ws_attn=ws(st_tree_attention_workspace(tree, Hq, Hkv, D, torch.bfloat16, max_prefix)),
        ws_verify=ws(st_verify_stochastic_workspace(tree, V) if stochastic
                     else st_verify_greedy_workspace(tree, V)),
        accept_len=torch.empty(B, **i32),
        accept_nodes=torch.empty(B, tree.max_depth + 1, **i32),
        out_tokens=torch.empty(B, tree.max_depth + 2, **i32),
        near_ties=torch.empty(B, **i32),
        src_slot=torch.empty(B, tree.max_depth + 1, **i32),
        new_len=torch.empty(B, **i32),
        status=torch.zeros(1, **i32),
    )
    return LayerBuffers(T, b)


def layer_forward(w: LayerWeights, tree: Tree, tokens, prefix_len, max_prefix: int, k_cache,
                  v_cache, lb: LayerBuffers):
    """Embedding through the vocabulary projection: fills lb.buf["logits"] and
    appends the tree's keys and values to the caches."""
    b = lb.buf
    T = tree.T
    st_embed(tokens, w.E, b["x"], b["status"])
    st_linear(b["x"], w.Wqkv, b["qkv"], workspace=b["ws_qkv"])
    st_tree_rope_append(tree, b["qkv"], w.Hq, w.Hkv, prefix_len, max_prefix, b["q"], k_cache,
                        v_cache, theta=w.theta, status=b["status"])
    st_tree_attention(tree, b["q"], k_cache, v_cache, prefix_len, max_prefix, None, b["attn"],
                      None, b["ws_attn"], status=b["status"])
    st_linear(b["attn"].view(T, w.Hq * w.D), w.Wo, b["h"], residual=b["x"],
              workspace=b["ws_o"])
    st_linear(b["h"], w.Wlm, b["logits"], workspace=b["ws_lm"])


def layer_step(w: LayerWeights, tree: Tree, tokens, prefix_len, max_prefix: int, k_cache,
               v_cache, lb: LayerBuffers, draft_logits: Optional[torch.Tensor] = None,
               temperature: float = 1.0, seed: int = 0, offset: int = 0):
    """layer_forward, then acceptance (greedy when draft_logits is None) and
    compaction of the accepted paths in the caches."""
    b = lb.buf
    layer_forward(w, tree, tokens, prefix_len, max_prefix, k_cache, v_cache, lb)
    if draft_logits is None:
        st_verify_greedy(tree, tokens, b["logits"], b["accept_len"], b["accept_nodes"],
                         b["out_tokens"], b["ws_verify"], b["status"])
    else:
        st_verify_stochastic(tree, tokens, b["logits"], draft_logits, temperature, seed, offset,
                             b["accept_len"], b["accept_nodes"], b["out_tokens"],
                             b["ws_verify"], b["near_ties"], b["status"])
    st_kv_compact(k_cache, v_cache, prefix_len, b["accept_len"], b["accept_nodes"],
                  b["src_slot"], b["new_len"], b["status"])
