"""Tree-masked attention with an explicit dense mask, in fp64.

[SpecInfer-dev §2.1] gives tree attention as: scores = Q K^T, entries where the
tree mask is 0 set to -1e9, softmax over the last axis, times V.
[SpecInfer-news "研究現狀"]: the keys/values of already decoded tokens are
cached (incremental decoding), so the query rows are the tree nodes only.

Readings used here:
  * scores are scaled by ``scale`` (1/sqrt(D) by default): the verified output
    must equal the target model's own attention, which is scaled;
  * "-1e9" means exclusion: masked entries get weight exactly 0;
  * query rows are the N tree nodes of a request; keys are the P cached prefix
    tokens (always visible) followed by the N tree tokens, visible iff on the
    row's root path; the same mask holds for every head;
  * grouped-query attention: q-head h reads kv-head h // (Hq / Hkv).
"""

from __future__ import annotations

import numpy as np

from .tree import dense_tree_mask


def decode_values(arr: np.ndarray, dtype: str) -> np.ndarray:
    """Values as fp64.  ``bf16`` arrays hold raw 16-bit patterns: a bfloat16 is
    the upper half of a float32."""
    if dtype == "f64":
        return np.asarray(arr, dtype=np.float64)
    if dtype == "f32":
        return np.asarray(arr, dtype=np.float32).astype(np.float64)
    if dtype == "bf16":
        bits = np.asarray(arr, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
        return bits.view(np.float32).astype(np.float64)
    raise ValueError(dtype)


def request_mask(parent_local, prefix_len: int) -> np.ndarray:
    """Boolean [N][P+N]: prefix columns all True, tree columns = ancestor mask."""
    n = len(parent_local)
    m = np.zeros((n, prefix_len + n), dtype=bool)
    m[:, :prefix_len] = True
    m[:, prefix_len:] = dense_tree_mask(parent_local)
    return m


def tree_attention(q, k_cache, v_cache, dtype, Hq, Hkv, node_off, parent, prefix_len,
                   scale=None, nodes=None, heads=None):
    """Attention output [T][Hq][D] and log-sum-exp [T][Hq] in fp64.

    ``nodes`` / ``heads`` optionally restrict the computation to some global
    node indices / q-heads (others are left NaN), for spot checks of large
    workloads.
    """
    T, _, D = q.shape
    G = Hq // Hkv
    if scale is None:
        scale = 1.0 / np.sqrt(D)
    out = np.full((T, Hq, D), np.nan)
    lse = np.full((T, Hq), np.nan)
    want_nodes = None if nodes is None else set(int(x) for x in nodes)
    head_list = range(Hq) if heads is None else [int(h) for h in heads]
    for b in range(len(node_off) - 1):
        lo, hi = int(node_off[b]), int(node_off[b + 1])
        rows = [t for t in range(lo, hi) if want_nodes is None or t in want_nodes]
        if not rows:
            continue
        P = int(prefix_len[b])
        n = hi - lo
        mask = request_mask([int(x) for x in parent[lo:hi]], P)[[t - lo for t in rows]]
        kv = {}
        for h in head_list:
            g = h // G
            if g not in kv:                                            # decoded once per kv-head
                kv = {g: (decode_values(k_cache[b, g, :P + n, :], dtype),      # [P+N, D]
                          decode_values(v_cache[b, g, :P + n, :], dtype))}
            K, Vv = kv[g]
            Q = decode_values(q[rows, h, :], dtype)                    # [r, D]
            S = (Q @ K.T) * scale
            S = np.where(mask, S, -np.inf)
            mx = S.max(axis=1, keepdims=True)
            E = np.exp(S - mx)
            l = E.sum(axis=1, keepdims=True)
            out[rows, h, :] = (E / l) @ Vv
            lse[rows, h] = (mx + np.log(l))[:, 0]
    return out, lse
