"""Pins for the oracle's token-tree construction: a hand-worked merge, brute
force over random candidates (every candidate is a root path, nodes are the
distinct prefixes, the numbering is level order with the stated tie rule),
capacity and bad inputs."""

import numpy as np
import pytest

import oracle
from oracle.tree import STATUS_BAD_TOKEN, STATUS_PATH_OVERFLOW, check_tree, depth_of


def test_hand_worked_merge():
    seqs = np.array([[[1, 2, 3], [1, 2, 4], [1, 5, 0], [6, 0, 0]]], np.int32)
    lens = np.array([[3, 3, 2, 1]], np.int32)
    r = oracle.build_tree(np.array([7]), seqs, lens, V=10, cap=16)
    n = int(r["n_nodes"][0])
    assert n == 7 and r["status"] == 0
    assert r["parent"][0, :n].tolist() == [-1, 0, 0, 1, 1, 3, 3]
    assert r["tokens"][0, :n].tolist() == [7, 1, 6, 2, 5, 3, 4]
    assert r["depth"][0, :n].tolist() == [0, 1, 1, 2, 2, 3, 3]
    assert (r["parent"][0, n:] == -1).all() and (r["tokens"][0, n:] == -1).all()


def _root_path_tokens(parent, tokens, i):
    out = []
    while parent[i] != -1:
        out.append(int(tokens[i]))
        i = int(parent[i])
    return out[::-1]


@pytest.mark.parametrize("seed", range(6))
def test_random_merges_brute_force(seed):
    rng = np.random.default_rng(seed)
    B, K, Lmax, V = 5, int(rng.integers(1, 9)), int(rng.integers(1, 7)), int(rng.integers(2, 6))
    seqs = rng.integers(0, V, (B, K, Lmax)).astype(np.int32)
    lens = rng.integers(0, Lmax + 1, (B, K)).astype(np.int32)
    r = oracle.build_tree(rng.integers(0, V, B), seqs, lens, V, cap=1 + K * Lmax)
    assert r["status"] == 0
    for b in range(B):
        n = int(r["n_nodes"][b])
        par, tok, dep = r["parent"][b, :n], r["tokens"][b, :n], r["depth"][b, :n]
        prefixes = {tuple(seqs[b, k, :j]) for k in range(K) for j in range(1, lens[b, k] + 1)}
        assert n == 1 + len(prefixes)
        assert check_tree(np.array([0, n]), par) == 0
        paths = {tuple(_root_path_tokens(par, tok, i)) for i in range(1, n)}
        assert paths == prefixes                   # every node is one distinct prefix
        for i in range(1, n):
            assert dep[i] == dep[par[i]] + 1
            assert dep[i] == depth_of(list(par), i)
        # level order, parents ascending within a level, ties by first candidate
        key = []
        for i in range(1, n):
            path = _root_path_tokens(par, tok, i)
            first = min(k for k in range(K) if lens[b, k] >= len(path)
                        and list(seqs[b, k, :len(path)]) == path)
            key.append((dep[i], par[i], first))
        assert key == sorted(key)
        sib = {}
        for i in range(1, n):
            assert (par[i], tok[i]) not in sib
            sib[(par[i], tok[i])] = i


def test_capacity_and_bad_inputs():
    seqs = np.array([[[1, 2, 3], [4, 5, 6]]], np.int32)
    r = oracle.build_tree(np.array([0]), seqs, np.array([[3, 3]]), V=10, cap=4)
    assert r["status"] & STATUS_PATH_OVERFLOW and int(r["n_nodes"][0]) == 4
    assert r["parent"][0].tolist() == [-1, 0, 0, 1] and r["tokens"][0].tolist() == [0, 1, 4, 2]
    bad = np.array([[[1, 12, 3], [4, 5, 6]]], np.int32)
    r = oracle.build_tree(np.array([0]), bad, np.array([[3, 9]]), V=10, cap=16)
    assert r["status"] & STATUS_BAD_TOKEN
    assert r["tokens"][0, :int(r["n_nodes"][0])].tolist() == [0, 1]   # stops before 12; len 9 -> 0


def test_pack_concatenates_requests():
    seqs = np.array([[[1, 2]], [[3, 3]]], np.int32)
    r = oracle.build_tree(np.array([9, 8]), seqs, np.array([[2], [1]]), V=5, cap=4)
    off, par, tok = oracle.pack_trees(r["n_nodes"], r["parent"], r["tokens"])
    assert off.tolist() == [0, 3, 5] and par.tolist() == [-1, 0, 1, -1, 0]
    assert tok.tolist() == [9, 1, 2, 8, 3]
