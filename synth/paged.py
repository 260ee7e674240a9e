"""Seeded paged layouts of a workload's caches: the contiguous caches cut
into blocks and scattered over a larger pool in a random order, with the
unused blocks filled with values that a wrong address would pick up.  Pure
data movement; nothing of the method is computed here."""

from __future__ import annotations

import numpy as np


def make_paged(seed: int, k_cache, v_cache, block_size: int, spare: int = 3):
    """Returns (k_pool, v_pool, block_table int32 [B][max_blocks]).  The
    caches [B][Hkv][S_max][D] are padded to whole blocks; the pool holds
    B * max_blocks + spare blocks, permuted by PCG64(seed)."""
    rng = np.random.Generator(np.random.PCG64(seed))
    B, Hkv, S, D = k_cache.shape
    mb = (S + block_size - 1) // block_size
    n = B * mb + spare
    perm = rng.permutation(n).astype(np.int32)
    table = perm[:B * mb].reshape(B, mb).copy()

    def build(cache):
        pool = np.empty((n, Hkv, block_size, D), dtype=cache.dtype)
        if cache.dtype == np.uint16:        # bf16 patterns: large finite values
            pool[:] = np.uint16(0x4480)     # 1024.0
        else:
            pool[:] = np.float32(1024.0)
        pad = np.zeros((B, Hkv, mb * block_size, D), dtype=cache.dtype)
        pad[:, :, :S] = cache
        for b in range(B):
            for j in range(mb):
                pool[table[b, j]] = pad[b, :, j * block_size:(j + 1) * block_size]
        return pool

    return build(k_cache), build(v_cache), table
