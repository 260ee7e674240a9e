"""Compaction of the accepted path's KV rows.

[SpecInfer-news "Token 樹驗證器"] mentions a depth-first KV-cache update that
verifies every tree path without extra storage, with no further detail.

Reading used here: during verification node i of request b has its keys and
values at cache slot P_b + i.  After acceptance the accepted root path
path[0..L] (path[0] = 0, the root) is gathered so that slot P_b + j holds what
slot P_b + path[j] held before; the committed length becomes P_b + L + 1.  A
node's slot after the move is P_b + depth, its position in the sequence, so
position-encoded keys stay valid.  Every copy reads the state before the call.
A root path strictly increases (parents precede children); a path that does not,
or that leaves the cache, is rejected (status bit 1) and nothing moves.
"""

from __future__ import annotations

import numpy as np

from .tree import STATUS_BAD_PARENT, STATUS_PATH_OVERFLOW


def kv_compact(k_cache, v_cache, prefix_len, accept_len, accept_nodes, max_path: int):
    """Returns (k_new, v_new, src_slot [B][max_path], new_len [B], status).
    The inputs are not modified."""
    B, _, S_max, _ = k_cache.shape
    k_new = k_cache.copy()
    v_new = v_cache.copy()
    src_slot = np.full((B, max_path), -1, dtype=np.int32)
    new_len = np.zeros(B, dtype=np.int32)
    status = 0
    for b in range(B):
        L = int(accept_len[b])
        P = int(prefix_len[b])
        if L < 0 or L + 1 > max_path:
            status |= STATUS_PATH_OVERFLOW
            new_len[b] = P
            continue
        path = [int(x) for x in accept_nodes[b, :L + 1]]
        increasing = all(path[j] > path[j - 1] for j in range(1, len(path)))
        if not increasing or any(not (0 <= n and P + n < S_max) for n in path):
            status |= STATUS_BAD_PARENT
            new_len[b] = P
            continue
        for j, n in enumerate(path):
            src_slot[b, j] = P + n
            k_new[b, :, P + j, :] = k_cache[b, :, P + n, :]
            v_new[b, :, P + j, :] = v_cache[b, :, P + n, :]
        new_len[b] = P + L + 1
    return k_new, v_new, src_slot, new_len, status
