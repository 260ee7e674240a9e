"""Pins for the oracle's KV compaction."""

import numpy as np
import torch
import torch.nn.functional as F

import oracle
from oracle.tree import STATUS_PATH_OVERFLOW
from synth import make_workload, tree_random_attach


def test_hand_worked_overlapping_moves(golden):
    g = golden("compact_small.txt")
    P, S = int(g["prefix"][0]), int(g["slots"][0])
    k = np.arange(S, dtype=np.float32).reshape(1, 1, S, 1)
    v = -k
    nodes = np.array([[int(x) for x in g["accept_nodes"]]], np.int32)
    L = int((nodes[0] >= 0).sum()) - 1
    kn, vn, src, new_len, st = oracle.kv_compact(k, v, np.array([P]), np.array([L]), nodes,
                                                 nodes.shape[1])
    assert st == 0
    assert kn[0, 0, :, 0].tolist() == [float(x) for x in g["after"]]
    assert vn[0, 0, :, 0].tolist() == [-float(x) for x in g["after"]]
    assert src[0].tolist() == [int(x) for x in g["src_slot"]]
    assert int(new_len[0]) == int(g["new_len"][0])
    assert k[0, 0, :, 0].tolist() == list(range(S))             # inputs untouched


def test_random_paths_move_rows_bit_exactly():
    rng = np.random.default_rng(3)
    B, H, S, D, P = 3, 2, 40, 4, 10
    k = rng.integers(0, 2 ** 16, (B, H, S, D)).astype(np.uint16)
    v = rng.integers(0, 2 ** 16, (B, H, S, D)).astype(np.uint16)
    paths = [[0, 3, 7, 20], [0], [0, 1, 2]]
    nodes = np.full((B, 6), -1, np.int32)
    for b, p in enumerate(paths):
        nodes[b, :len(p)] = p
    L = np.array([len(p) - 1 for p in paths], np.int32)
    kn, vn, src, new_len, st = oracle.kv_compact(k, v, np.full(B, P), L, nodes, 6)
    assert st == 0
    for b, p in enumerate(paths):
        for j, n in enumerate(p):
            assert np.array_equal(kn[b, :, P + j], k[b, :, P + n])
            assert np.array_equal(vn[b, :, P + j], v[b, :, P + n])
        untouched = [s for s in range(S) if not (P <= s < P + len(p))]
        assert np.array_equal(kn[b][:, untouched], k[b][:, untouched])
        assert int(new_len[b]) == P + len(p)
        assert src[b, :len(p)].tolist() == [P + n for n in p]


def test_compacted_cache_decodes_like_the_tree():
    """After moving the accepted path into place, ordinary single-query attention of
    the last accepted node over the committed cache equals its tree attention."""
    rng = np.random.default_rng(8)
    n, P, D, H = 16, 12, 8, 2
    parent, _ = tree_random_attach(rng, n, 6)
    q = rng.standard_normal((n, H, D)).astype(np.float32)
    k = rng.standard_normal((1, H, P + n, D)).astype(np.float32)
    v = rng.standard_normal((1, H, P + n, D)).astype(np.float32)
    out, _ = oracle.tree_attention(q, k, v, "f32", H, H, np.array([0, n], np.int32), parent,
                                   np.array([P], np.int32))
    leaf = n - 1
    path = []
    i = leaf
    while i != -1:
        path.append(i)
        i = int(parent[i])
    path = path[::-1]
    nodes = np.full((1, 8), -1, np.int32)
    nodes[0, :len(path)] = path
    kn, vn, _, new_len, _ = oracle.kv_compact(k, v, np.array([P]), np.array([len(path) - 1]),
                                              nodes, 8)
    m = int(new_len[0])
    ref = F.scaled_dot_product_attention(
        torch.from_numpy(q[leaf].astype(np.float64))[:, None, :],
        torch.from_numpy(kn[0, :, :m].astype(np.float64)),
        torch.from_numpy(vn[0, :, :m].astype(np.float64))).numpy()[:, 0, :]
    np.testing.assert_allclose(out[leaf], ref, atol=1e-12)


def test_overflow_and_bad_path_status():
    wl = make_workload("tiny_fp32", 0)
    nodes = np.array([[0, 1, 3, 7]], np.int32)
    _, _, _, new_len, st = oracle.kv_compact(wl.k_cache, wl.v_cache, wl.prefix_len,
                                             np.array([3]), nodes, 3)
    assert st & STATUS_PATH_OVERFLOW and int(new_len[0]) == int(wl.prefix_len[0])
    _, _, _, _, st = oracle.kv_compact(wl.k_cache, wl.v_cache, wl.prefix_len, np.array([1]),
                                       np.array([[0, 99, -1, -1]], np.int32), 4)
    assert st & 1
