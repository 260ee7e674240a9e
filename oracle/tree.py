"""Token tree structure: validity, root paths, depth, and the ancestor mask.

[SpecInfer-dev §2.1]: every tree node carries a pointer to its parent.
[SpecInfer-news "Token 樹驗證器"]: tree attention lets every node see exactly
the tokens on its own root path, through a constructed mask matrix.

Reading used here: node 0 of each request is the root (the last token the
target already emitted), parent[0] = -1 and 0 <= parent[i] < i.  Node i sees
tree node k iff k lies on the path from i up to the root (i itself included).
"""

from __future__ import annotations

import numpy as np

STATUS_BAD_PARENT = 1
STATUS_BAD_TOKEN = 2
STATUS_NONFINITE = 4
STATUS_PATH_OVERFLOW = 8


def check_tree(node_off, parent) -> int:
    """Status bit 1 if any request's parent array breaks the rules above."""
    status = 0
    B = len(node_off) - 1
    for b in range(B):
        lo, hi = int(node_off[b]), int(node_off[b + 1])
        if hi - lo < 1:
            status |= STATUS_BAD_PARENT
            continue
        if int(parent[lo]) != -1:
            status |= STATUS_BAD_PARENT
        for i in range(1, hi - lo):
            p = int(parent[lo + i])
            if not (0 <= p < i):
                status |= STATUS_BAD_PARENT
    return status


def root_path(parent_local, i: int) -> list:
    """Nodes from i up to the root, by following parent pointers."""
    path = []
    j = int(i)
    while j != -1:
        if len(path) > len(parent_local):
            raise ValueError("parent pointers form a cycle")
        path.append(j)
        j = int(parent_local[j])
    return path


def depth_of(parent_local, i: int) -> int:
    """Number of edges between node i and the root."""
    return len(root_path(parent_local, i)) - 1


def children_of(parent_local, u: int) -> list:
    """Children of node u in ascending local index."""
    return [c for c in range(len(parent_local)) if int(parent_local[c]) == u]


def dense_tree_mask(parent_local) -> np.ndarray:
    """Boolean N x N matrix: [i, k] is True iff k is on i's root path."""
    n = len(parent_local)
    m = np.zeros((n, n), dtype=bool)
    for i in range(n):
        for k in root_path(parent_local, i):
            m[i, k] = True
    return m


def pack_mask_bits(dense: np.ndarray, W: int) -> np.ndarray:
    """Pack each row into W little-endian 64-bit words: bit (k % 64) of word
    (k // 64) is column k."""
    n, ncols = dense.shape
    out = np.zeros((n, W), dtype=np.uint64)
    for i in range(n):
        for k in range(ncols):
            if dense[i, k]:
                out[i, k // 64] |= np.uint64(1) << np.uint64(k % 64)
    return out


def tree_mask(node_off, parent, W: int):
    """Packed ancestor mask [T][W] (uint64) and depth [T] (int32) for every
    node of every request."""
    T = int(node_off[-1])
    mask = np.zeros((T, W), dtype=np.uint64)
    depth = np.zeros(T, dtype=np.int32)
    for b in range(len(node_off) - 1):
        lo, hi = int(node_off[b]), int(node_off[b + 1])
        par = [int(x) for x in parent[lo:hi]]
        dense = dense_tree_mask(par)
        mask[lo:hi] = pack_mask_bits(dense, W)
        for i in range(hi - lo):
            depth[lo + i] = depth_of(par, i)
    return mask, depth
