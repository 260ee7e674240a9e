"""GPU parity: merging candidate continuations into token trees (the step
before verification), bit-exact against the oracle through the C ABI; the
packed output feeds the ancestor-mask call."""

import numpy as np
import pytest
import torch

import oracle
from oracle.tree import STATUS_BAD_TOKEN, STATUS_PATH_OVERFLOW
from synth import TREE_BUILD_CASE, make_candidates
from token_tree_verification_st_amd import Tree, st_tree_build, st_tree_mask
from tests.gpu_util import require_gpu, say

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _gpu():
    require_gpu()


def _run(root, seqs, lens, V, cap, packed=True):
    B, K, Lmax = seqs.shape
    d = lambda a: torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).cuda()
    o = {k: torch.full((B * cap,), -7, dtype=torch.int32, device="cuda")
         for k in ("parent", "tokens", "depth", "parent_packed", "tokens_packed")}
    o["n_nodes"] = torch.full((B,), -7, dtype=torch.int32, device="cuda")
    o["node_off"] = torch.full((B + 1,), -7, dtype=torch.int32, device="cuda")
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    kw = dict(node_off=o["node_off"], parent_packed=o["parent_packed"],
              tokens_packed=o["tokens_packed"]) if packed else {}
    st_tree_build(d(root), d(seqs), d(lens), V, cap, o["n_nodes"], o["parent"], o["tokens"],
                  o["depth"], status=status, **kw)
    torch.cuda.synchronize()
    out = {k: v.cpu().numpy() for k, v in o.items()}
    out["status"] = int(status.item())
    return out


def _compare(root, seqs, lens, V, cap, packed=True):
    B = seqs.shape[0]
    g = _run(root, seqs, lens, V, cap, packed)
    r = oracle.build_tree(root, seqs, lens, V, cap)
    assert g["status"] == r["status"]
    assert np.array_equal(g["n_nodes"], r["n_nodes"])
    for k in ("parent", "tokens", "depth"):
        assert np.array_equal(g[k].reshape(B, cap), r[k]), k
    if packed:
        off, par, tok = oracle.pack_trees(r["n_nodes"], r["parent"], r["tokens"])
        T = int(off[-1])
        assert np.array_equal(g["node_off"], off)
        assert np.array_equal(g["parent_packed"][:T], par)
        assert np.array_equal(g["tokens_packed"][:T], tok)
        assert (g["parent_packed"][T:] == -7).all()       # past node_off[B]: untouched
    return g, r


@pytest.mark.parametrize("seed,B,K,Lmax,V", [
    (1, 4, 1, 1, 5), (2, 3, 5, 3, 3), (3, 8, 16, 8, 4), (4, 2, 64, 6, 3), (5, 5, 7, 12, 32000),
    (6, 1, 256, 32, 2), (7, 16, 16, 8, 32000), (8, 3, 255, 2, 2), (9, 2, 33, 40, 3)])
def test_random_candidates_match_oracle(seed, B, K, Lmax, V):
    say(f"tree_build seed={seed} B={B} K={K} Lmax={Lmax} V={V}")
    root, seqs, lens = make_candidates(seed, B, K, Lmax, V, min_len=0)
    cap = min(256, 1 + K * Lmax)
    g, r = _compare(root, seqs, lens, V, cap)
    if K * Lmax + 1 > 256:
        return
    assert g["status"] == 0


def test_measured_case_and_its_masks():
    c = TREE_BUILD_CASE
    say(f"tree_build measured case {c}")
    root, seqs, lens = make_candidates(0, c["B"], c["K"], c["Lmax"], c["V"])
    g, r = _compare(root, seqs, lens, c["V"], c["cap"])
    assert g["status"] == 0
    # the packed trees are st_tree input: their ancestor masks match the oracle's
    off = g["node_off"]
    T = int(off[-1])
    tree = Tree(torch.from_numpy(off).cuda(), torch.from_numpy(g["parent_packed"][:T]).cuda(),
                int(g["n_nodes"].max()), c["Lmax"])
    mask = torch.zeros(T * tree.W, dtype=torch.int64, device="cuda")
    depth = torch.zeros(T, dtype=torch.int32, device="cuda")
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    st_tree_mask(tree, mask, depth, status)
    torch.cuda.synchronize()
    ref_mask, ref_depth = oracle.tree_mask(off, g["parent_packed"][:T], tree.W)
    assert np.array_equal(mask.cpu().numpy().view(np.uint64).reshape(T, tree.W), ref_mask)
    assert np.array_equal(depth.cpu().numpy(),
                          np.concatenate([r["depth"][b, :r["n_nodes"][b]] for b in range(c["B"])]))
    assert int(status.item()) == 0


def test_capacity_truncation():
    root, seqs, lens = make_candidates(11, 4, 32, 8, 50)
    for cap in (1, 2, 17, 64):
        say(f"tree_build cap={cap}")
        g, r = _compare(root, seqs, lens, 50, cap)
        assert g["status"] & STATUS_PATH_OVERFLOW
        assert (g["n_nodes"] <= cap).all() and (g["n_nodes"] == cap).any()


def test_bad_lengths_and_tokens():
    root, seqs, lens = make_candidates(12, 3, 6, 5, 10, min_len=0)
    lens[0, 1] = 6          # longer than Lmax: counts as 0
    lens[1, 2] = -1         # negative: counts as 0
    seqs[2, 3, 2] = 10      # out of range: candidate stops before it
    seqs[2, 4, 0] = -5
    lens[2, 3] = lens[2, 4] = 5
    g, r = _compare(root, seqs, lens, 10, 64)
    assert g["status"] == STATUS_BAD_TOKEN


def test_padded_only_and_max_limits():
    root, seqs, lens = make_candidates(13, 2, 256, 32, 3)
    _compare(root, seqs, lens, 3, 256, packed=False)


def test_host_errors():
    root, seqs, lens = make_candidates(14, 1, 4, 4, 10)
    d = lambda a: torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).cuda()
    z = lambda n: torch.zeros(n, dtype=torch.int32, device="cuda")
    with pytest.raises(RuntimeError):       # capacity above 256 nodes
        st_tree_build(d(root), d(seqs), d(lens), 10, 300, z(1), z(300), z(300), z(300))
    big = np.zeros((1, 257, 1), np.int32)
    with pytest.raises(RuntimeError):       # more than 256 candidates
        st_tree_build(d(root), d(big), z(257), 10, 8, z(1), z(8), z(8), z(8))
    long = np.zeros((1, 2, 4097), np.int32)
    with pytest.raises(RuntimeError):       # K * Lmax above 8192
        st_tree_build(d(root), d(long), z(2), 10, 8, z(1), z(8), z(8), z(8))
    with pytest.raises(ValueError):         # packed outputs go together
        st_tree_build(d(root), d(seqs), d(lens), 10, 8, z(1), z(8), z(8), z(8), node_off=z(2))


def test_built_trees_feed_the_verification_step():
    """Candidates -> st_tree_build -> one-call verification step (mask,
    attention, greedy acceptance, compaction), against the oracle; the target
    is planted to agree with one candidate of each request along its whole
    length, so the accepted path is that candidate."""
    from synth import build_workload
    from token_tree_verification_st_amd import to_device
    from token_tree_verification_st_amd import step as stp

    B, K, Lmax, V = 4, 6, 5, 500
    root, seqs, lens = make_candidates(21, B, K, Lmax, V)
    g = _run(root, seqs, lens, V, 64)
    assert g["status"] == 0
    off = g["node_off"]
    T = int(off[-1])
    par_p, tok_p = g["parent_packed"][:T], g["tokens_packed"][:T]
    trees = []
    for b in range(B):
        n = int(g["n_nodes"][b])
        trees.append((g["parent"][b * 64:b * 64 + n].copy(), g["depth"][b * 64:b * 64 + n].copy()))
    rng = np.random.default_rng(22)
    wl = build_workload("built", rng, dtype="bf16", Hq=4, Hkv=4, D=128, V=V,
                        prefix_lens=[37, 300, 129, 64], trees=trees, max_depth=Lmax)
    assert np.array_equal(wl.node_off, off) and np.array_equal(wl.parent, par_p)
    wl.tokens = tok_p.astype(np.int32).copy()
    # plant: after each node on candidate k's path, the target's argmax is the
    # candidate's next token (the tree holds that child); after its last node,
    # token 7
    want = {}
    for b in range(B):
        k = int(np.argmax(lens[b]))
        node, path = 0, [0]
        lo = int(off[b])
        for j in range(int(lens[b, k])):
            kids = [c for c in range(int(g["n_nodes"][b])) if g["parent"][b * 64 + c] == node]
            node = next(c for c in kids if g["tokens"][b * 64 + c] == seqs[b, k, j])
            path.append(node)
        for u, nxt in zip(path, path[1:] + [None]):
            wl.logits[lo + u, :] = -5.0
            wl.logits[lo + u, int(seqs[b, k, len(path[:path.index(u)])]) if nxt is not None
                      else 7] = 5.0
        want[b] = path
    dw = to_device(wl)
    k0 = wl.k_cache.copy()
    stp.verification_step(dw, stochastic=False)
    torch.cuda.synchronize()
    res = oracle.verify_greedy(wl.node_off, wl.parent, wl.tokens, wl.logits, V, wl.max_depth)
    for key in ("accept_len", "accept_nodes", "out_tokens"):
        assert np.array_equal(dw.buf[key].cpu().numpy(), res[key]), key
    for b in range(B):
        L = int(res["accept_len"][b])
        assert res["accept_nodes"][b, :L + 1].tolist() == want[b]
    kn, vn, src, new_len, st = oracle.kv_compact(k0, wl.v_cache, wl.prefix_len,
                                                 res["accept_len"], res["accept_nodes"],
                                                 wl.max_depth + 1)
    assert np.array_equal(dw.k_cache.cpu().view(torch.int16).numpy().view(np.uint16), kn)
    assert np.array_equal(dw.buf["new_len"].cpu().numpy(), new_len)
    out = dw.buf["out"].float().cpu().numpy().astype(np.float64)
    ref, _ = oracle.tree_attention(wl.q, k0, wl.v_cache, wl.dtype, wl.Hq, wl.Hkv, wl.node_off,
                                   wl.parent, wl.prefix_len)
    assert np.abs(out - ref).max() <= 1e-2
    assert int(dw.buf["status"].item()) == 0


@pytest.mark.parametrize("K", [63, 64, 65, 128])
def test_kernel_width_boundary(K):
    """Around the switch from one wavefront (K <= 64) to 256 threads."""
    root, seqs, lens = make_candidates(30 + K, 3, K, 6, 7)
    _compare(root, seqs, lens, 7, 256)


def test_degenerate_candidate_sets():
    """Identical candidates (one chain), candidates differing in their first
    token only (a star of chains), and no candidate tokens at all (the root
    alone)."""
    B, K, L = 3, 8, 5
    seqs = np.zeros((B, K, L), np.int32)
    lens = np.full((B, K), L, np.int32)
    seqs[0] = np.arange(L)                                    # all the same
    for k in range(K):
        seqs[1, k] = [k] + [9] * (L - 1)                      # first tokens differ
    lens[2] = 0                                               # nothing to merge
    root = np.array([1, 2, 3], np.int32)
    g, r = _compare(root, seqs, lens, 10, 64)
    assert g["n_nodes"].tolist() == [1 + L, 1 + K * L, 1]
    assert g["parent"][:1 + L].tolist() == [-1] + list(range(L))
    assert g["status"] == 0
