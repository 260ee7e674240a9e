"""Paged KV memory: keys and values kept in fixed-size blocks named by a
per-request block table, instead of one contiguous run per request.

Sources:
  [SpecInfer-news "研究現狀"] the KV cache of incremental decoding grows with
      every token; paged KV memory is contrasted with contiguous per-request
      KV (the vAttention notes on the same page: contiguous virtual memory
      versus paging).

Reading used here (the pages give no layout): the pool is
[n_blocks][Hkv][block_size][D]; logical slot k of request b (the slot the
contiguous layout would use: prefix keys k < P_b, tree node i at P_b + i) is
row k % block_size of block block_table[b][k // block_size].  Verification
over a paged pool computes exactly what it computes over the contiguous
caches that the table describes; compaction moves logical slots.
"""

from __future__ import annotations

import numpy as np

from .compact import kv_compact


def gather_paged(pool, block_table, block_size: int):
    """The contiguous caches [B][Hkv][max_blocks * block_size][D] that the
    pool and table describe (every logical slot, used or not)."""
    B, MB = block_table.shape
    _, Hkv, bs, D = pool.shape
    assert bs == block_size
    out = np.empty((B, Hkv, MB * bs, D), dtype=pool.dtype)
    for b in range(B):
        for j in range(MB):
            out[b, :, j * bs:(j + 1) * bs, :] = pool[int(block_table[b, j])]
    return out


def scatter_paged(caches, pool, block_table, block_size: int):
    """Write contiguous caches back into a copy of the pool through the table
    (the inverse of gather_paged on the blocks the table names)."""
    new = pool.copy()
    B, MB = block_table.shape
    bs = block_size
    for b in range(B):
        for j in range(MB):
            new[int(block_table[b, j])] = caches[b, :, j * bs:(j + 1) * bs, :]
    return new


def kv_compact_paged(k_pool, v_pool, block_table, block_size: int, prefix_len, accept_len,
                     accept_nodes, max_path: int):
    """Compaction on a paged pool: the contiguous compaction of the gathered
    caches, written back through the table.  Returns (k_pool', v_pool',
    src_slot, new_len, status); the inputs are not modified."""
    kc = gather_paged(k_pool, block_table, block_size)
    vc = gather_paged(v_pool, block_table, block_size)
    k2, v2, src, nl, st = kv_compact(kc, vc, prefix_len, accept_len, accept_nodes, max_path)
    return (scatter_paged(k2, k_pool, block_table, block_size),
            scatter_paged(v2, v_pool, block_table, block_size), src, nl, st)
