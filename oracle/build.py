"""Token-tree construction: merging several candidate sequences into one tree.

Sources:
  [SpecInfer-news "研究現狀"] the outputs of several small speculative models
      are merged into one speculated token tree that the target verifies.
  [SpecInfer-dev §2.1, §2.2] the speculation stage builds the token tree from
      several candidate sequences; sharing prefixes avoids repeated work; a
      tree node carries a parent pointer.

Readings used here (the pages fix no layout or order):
  * request b has a root token (the last token the target emitted) and K
    candidate continuations seq[k][0 .. len_k - 1]; the tree's nodes are the
    root and every distinct non-empty prefix of a candidate, the node of
    prefix seq[k][0..j] being the child of the node of seq[k][0..j-1] that
    carries token seq[k][j];
  * nodes are numbered level by level (so parents precede children); within
    a level by their parent's number, then by the smallest candidate index k
    whose prefix it is;
  * a request whose tree would exceed the capacity keeps its first `cap`
    nodes in that order and reports status bit 8 (path overflow); a length
    outside [0, Lmax] counts as 0 and a token outside [0, V) stops that
    candidate there, both reporting bit 2 (bad token).
"""

from __future__ import annotations

import numpy as np

from .tree import STATUS_BAD_TOKEN, STATUS_PATH_OVERFLOW


def build_tree(root_tokens, seqs, lens, V: int, cap: int):
    """Returns dict(n_nodes [B], parent [B][cap], tokens [B][cap], depth [B][cap],
    status); unused slots hold -1."""
    B, K, Lmax = seqs.shape
    n_nodes = np.zeros(B, np.int32)
    parent = np.full((B, cap), -1, np.int32)
    tokens = np.full((B, cap), -1, np.int32)
    depth = np.full((B, cap), -1, np.int32)
    status = 0
    for b in range(B):
        # usable length of each candidate
        use = []
        for k in range(K):
            n = int(lens[b, k])
            if n < 0 or n > Lmax:
                status |= STATUS_BAD_TOKEN
                n = 0
            for j in range(n):
                if not (0 <= int(seqs[b, k, j]) < V):
                    status |= STATUS_BAD_TOKEN
                    n = j
                    break
            use.append(n)
        # the distinct prefixes, level by level
        index = {(): 0}
        order = [((), -1, 0)]      # (prefix, parent number, depth)
        frontier = [()]
        for j in range(Lmax):
            level = {}
            for k in range(K):
                if use[k] > j:
                    pre = tuple(int(x) for x in seqs[b, k, :j + 1])
                    if pre not in level:
                        level[pre] = (index[pre[:-1]], k)     # parent number, first candidate
            for pre, (par, k) in sorted(level.items(), key=lambda kv: kv[1]):
                index[pre] = len(order)
                order.append((pre, par, j + 1))
        if len(order) > cap:
            status |= STATUS_PATH_OVERFLOW
            order = order[:cap]
        n_nodes[b] = len(order)
        for i, (pre, par, d) in enumerate(order):
            parent[b, i] = par
            tokens[b, i] = int(root_tokens[b]) if i == 0 else pre[-1]
            depth[b, i] = d
    return dict(n_nodes=n_nodes, parent=parent, tokens=tokens, depth=depth, status=status)


def pack_trees(n_nodes, parent, tokens):
    """Concatenate padded per-request trees: node_off [B+1], parent [T], tokens [T]."""
    B = len(n_nodes)
    node_off = np.zeros(B + 1, np.int32)
    node_off[1:] = np.cumsum(n_nodes)
    par = np.concatenate([parent[b, :n_nodes[b]] for b in range(B)]).astype(np.int32)
    tok = np.concatenate([tokens[b, :n_nodes[b]] for b in range(B)]).astype(np.int32)
    return node_off, par, tok
