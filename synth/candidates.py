"""Seeded candidate continuations for token-tree construction.

Several small speculative models continuing the same context tend to agree on
the first tokens and diverge later; the draw below reproduces that shape of
input (shared prefixes of random length) without modelling any of the method:
nothing here merges candidates or builds a tree.

Draw order (one ``PCG64(seed)`` stream): per request, root token; then per
candidate k: its length, then -- for k > 0 -- the earlier candidate it shares a
prefix with and the shared length, then its fresh tokens.
"""

from __future__ import annotations

import numpy as np


def make_candidates(seed: int, B: int, K: int, Lmax: int, V: int, min_len: int = 1):
    """Returns (root_tokens int32 [B], seqs int32 [B][K][Lmax], lens int32
    [B][K]).  Candidate k > 0 copies the first s tokens of a uniformly chosen
    earlier candidate (s uniform in [0, Lmax]) and draws the rest uniformly
    from [0, V); lengths are uniform in [min_len, Lmax]; slots past a length
    hold random tokens too (they must be ignored)."""
    rng = np.random.Generator(np.random.PCG64(seed))
    root = np.zeros(B, np.int32)
    seqs = np.zeros((B, K, Lmax), np.int32)
    lens = np.zeros((B, K), np.int32)
    for b in range(B):
        root[b] = rng.integers(0, V)
        for k in range(K):
            lens[b, k] = rng.integers(min_len, Lmax + 1)
            s = 0
            if k > 0:
                src = int(rng.integers(0, k))
                s = int(rng.integers(0, Lmax + 1))
                seqs[b, k, :s] = seqs[b, src, :s]
            seqs[b, k, s:] = rng.integers(0, V, Lmax - s)
    return root, seqs, lens


# The measured construction case: 16 requests, 16 candidates of up to 8 tokens
# each, a 32000-token vocabulary, trees of at most 128 nodes.
TREE_BUILD_CASE = dict(B=16, K=16, Lmax=8, V=32000, cap=128)
