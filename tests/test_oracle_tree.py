"""Pins for the oracle's tree structure functions (mask, depth, validity)."""

import itertools

import numpy as np
import pytest

import oracle
from synth import tree_beam_plus_leaves, tree_chain, tree_complete_binary, tree_random_attach


def _words(mask_row):
    return [int(x) for x in mask_row]


def test_hand_worked_small_tree(golden):
    g = golden("tree_mask_small.txt")
    parent = np.array([int(x) for x in g["small.parent"]], dtype=np.int32)
    node_off = np.array([0, len(parent)], dtype=np.int32)
    mask, depth = oracle.tree_mask(node_off, parent, 1)
    assert [int(m) for m in mask[:, 0]] == [int(x) for x in g["small.mask"]]
    assert depth.tolist() == [int(x) for x in g["small.depth"]]


def test_hand_worked_chain70_two_words(golden):
    g = golden("tree_mask_small.txt")
    n = int(g["chain70.chain"][0])
    parent, _ = tree_chain(n)
    mask, depth = oracle.tree_mask(np.array([0, n], np.int32), parent, 2)
    for r in (63, 64, 69):
        assert _words(mask[r]) == [int(x) for x in g[f"chain70.row{r}"]]
    assert int(depth[69]) == int(g["chain70.depth69"][0])


def test_chain_is_lower_triangular():
    n = 40
    parent, _ = tree_chain(n)
    dense = oracle.dense_tree_mask(parent)
    assert np.array_equal(dense, np.tril(np.ones((n, n), dtype=bool)))


def test_complete_binary_heap_closed_form():
    # In heap order (parent of i is (i-1)//2), k is an ancestor-or-self of i iff the
    # binary numeral of k+1 is a prefix of that of i+1.
    n = 63
    parent, _ = tree_complete_binary(n)
    dense = oracle.dense_tree_mask(parent)
    for i in range(n):
        bi = bin(i + 1)[2:]
        for k in range(n):
            bk = bin(k + 1)[2:]
            assert dense[i, k] == bi.startswith(bk), (i, k)
        assert oracle.depth_of(parent, i) == len(bi) - 1


def _reachability(parent):
    """Ancestor-or-self relation as the transitive closure of the child->parent
    adjacency, by repeated boolean matrix products."""
    n = len(parent)
    A = np.zeros((n, n), dtype=np.int64)
    for i in range(1, n):
        A[i, parent[i]] = 1
    R = np.eye(n, dtype=np.int64)
    step = np.eye(n, dtype=np.int64)
    for _ in range(n):
        step = (step @ A > 0).astype(np.int64)
        R = ((R + step) > 0).astype(np.int64)
    return R.astype(bool)


def test_brute_force_all_trees_up_to_6_nodes():
    for n in range(1, 7):
        choices = [range(i) for i in range(1, n)]
        for tail in itertools.product(*choices):
            parent = np.array((-1,) + tail, dtype=np.int32)
            dense = oracle.dense_tree_mask(parent)
            assert np.array_equal(dense, _reachability(parent))
            pm = oracle.pack_mask_bits(dense, 1)
            for i in range(n):
                assert bin(int(pm[i, 0])).count("1") == oracle.depth_of(parent, i) + 1


@pytest.mark.parametrize("seed", [1, 2, 3])
def test_recurrence_matches_definition(seed):
    rng = np.random.default_rng(seed)
    parent, _ = tree_random_attach(rng, 200, 9)
    W = 4
    mask, depth = oracle.tree_mask(np.array([0, 200], np.int32), parent, W)
    rec = np.zeros((200, W), dtype=np.uint64)
    for i in range(200):
        if i:
            rec[i] = rec[parent[i]]
        rec[i, i // 64] |= np.uint64(1) << np.uint64(i % 64)
    assert np.array_equal(rec, mask)
    pop = [sum(bin(int(w)).count("1") for w in mask[i]) for i in range(200)]
    assert pop == (depth + 1).tolist()


def test_synth_shapes_respect_depth_bounds():
    rng = np.random.default_rng(5)
    p, _ = tree_random_attach(rng, 64, 8)
    assert max(oracle.depth_of(p, i) for i in range(64)) <= 8
    p, _ = tree_beam_plus_leaves(rng, 100, 5, 3)
    assert max(oracle.depth_of(p, i) for i in range(100)) <= 3
    assert oracle.check_tree(np.array([0, 100]), p) == 0


def test_check_tree_flags_bad_parents():
    ok = np.array([-1, 0, 1], np.int32)
    assert oracle.check_tree(np.array([0, 3]), ok) == 0
    for bad in ([0, 0, 1], [-1, 1, 1], [-1, 0, 3], [-1, -1, 0], [-1, 0, 2]):
        assert oracle.check_tree(np.array([0, 3]), np.array(bad, np.int32)) == 1
    assert oracle.check_tree(np.array([0, 0]), np.array([], np.int32)) == 1
