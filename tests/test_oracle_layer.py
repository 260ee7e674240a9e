"""Pins for the oracle's one-layer model pieces: rotary embedding against the
complex-number form and its invariants, the projection against explicit sums,
node positions on hand-drawn trees, and the lossless property: greedy tree
verification steps (tree layer, greedy acceptance, compaction) reproduce plain
autoregressive greedy decoding with the same model."""

import numpy as np
import pytest

import oracle
from oracle.attention import decode_values
from synth import model_config, model_weights, tree_random_attach


def _params(seed, cfg):
    w = model_weights(seed, cfg)
    return {k: decode_values(v, "bf16") for k, v in w.items()}


def test_rope_equals_complex_rotation():
    rng = np.random.default_rng(1)
    n, H, D = 5, 3, 16
    x = rng.standard_normal((n, H, D))
    pos = np.array([0, 1, 7, 100, 4095])
    got = oracle.rope(x, pos)
    j = np.arange(D // 2)
    ang = pos[:, None, None] * 10000.0 ** (-2.0 * j / D)[None, None, :]
    z = (x[..., :D // 2] + 1j * x[..., D // 2:]) * np.exp(1j * ang)
    want = np.concatenate([z.real, z.imag], axis=-1)
    np.testing.assert_allclose(got, want, rtol=0, atol=1e-12)


def test_rope_unit_vectors_closed_form():
    D = 8
    for j in range(D // 2):
        x = np.zeros((1, 1, D))
        x[0, 0, j] = 1.0
        p = 3
        theta = p * 10000.0 ** (-2.0 * j / D)
        got = oracle.rope(x, np.array([p]))[0, 0]
        want = np.zeros(D)
        want[j] = np.cos(theta)
        want[j + D // 2] = np.sin(theta)
        np.testing.assert_allclose(got, want, atol=1e-15)
        # the second half of a pair turns the other way round
        x = np.zeros((1, 1, D))
        x[0, 0, j + D // 2] = 1.0
        got = oracle.rope(x, np.array([p]))[0, 0]
        want = np.zeros(D)
        want[j] = -np.sin(theta)
        want[j + D // 2] = np.cos(theta)
        np.testing.assert_allclose(got, want, atol=1e-15)


def test_rope_position_zero_is_identity_and_norms_are_kept():
    rng = np.random.default_rng(2)
    x = rng.standard_normal((4, 2, 32))
    np.testing.assert_array_equal(oracle.rope(x, np.zeros(4, np.int64)), x)
    y = oracle.rope(x, np.array([5, 50, 500, 5000]))
    np.testing.assert_allclose(np.linalg.norm(y, axis=-1), np.linalg.norm(x, axis=-1),
                               rtol=1e-13)


def test_rope_scores_depend_on_relative_position_only():
    rng = np.random.default_rng(3)
    D = 32
    q = rng.standard_normal((1, 1, D))
    k = rng.standard_normal((1, 1, D))
    for m, n in [(7, 3), (100, 0), (12, 40)]:
        base = float(np.sum(oracle.rope(q, np.array([m])) * oracle.rope(k, np.array([n]))))
        for s in (1, 9, 1000):
            sh = float(np.sum(oracle.rope(q, np.array([m + s])) *
                              oracle.rope(k, np.array([n + s]))))
            assert abs(sh - base) < 1e-10


def test_linear_matches_explicit_sums():
    rng = np.random.default_rng(4)
    M, N, K = 3, 5, 7
    x = rng.standard_normal((M, K))
    w = rng.standard_normal((N, K))
    r = rng.standard_normal((M, N))
    y = oracle.linear(x, w, residual=r)
    for m in range(M):
        for n in range(N):
            s = r[m, n]
            for k in range(K):
                s += x[m, k] * w[n, k]
            assert abs(y[m, n] - s) < 1e-12


def test_node_positions_hand_drawn():
    # request 0: chain 0-1-2; request 1: root with children 1, 2 and grandchild 3 under 2
    node_off = np.array([0, 3, 7], np.int32)
    parent = np.array([-1, 0, 1, -1, 0, 0, 2], np.int32)
    pos = oracle.node_positions(node_off, parent, np.array([10, 4], np.int32))
    assert pos.tolist() == [10, 11, 12, 4, 5, 5, 6]


CFG = model_config(V=96, Hq=4, Hkv=2, D=16)


def test_chain_tree_layer_equals_autoregressive_logits():
    """A chain of the prompt's tokens verified with an empty prefix gives every
    position the logits that one-token-at-a-time decoding gives."""
    params = _params(5, CFG)
    rng = np.random.default_rng(5)
    prompt = rng.integers(0, CFG["V"], 9)
    n = len(prompt)
    kc = np.zeros((1, CFG["Hkv"], 16, CFG["D"]))
    out = oracle.tree_layer(params, CFG, prompt, np.array([0, n], np.int32),
                            np.arange(-1, n - 1, dtype=np.int32), np.array([0], np.int32), kc,
                            kc.copy())
    toks, _ = oracle.ar_greedy_decode(params, CFG, prompt, 1)
    assert int(np.argmax(out["logits"][-1])) == int(toks[0])
    for i in range(1, n):
        ar, _ = oracle.ar_greedy_decode(params, CFG, prompt[:i], 1)
        assert int(np.argmax(out["logits"][i - 1])) == int(ar[0])
    # the keys written for the chain are the prefix cache of the same tokens
    pk, pv = oracle.prefix_cache(params, CFG, prompt, 16)
    np.testing.assert_allclose(out["k_cache"], pk, atol=1e-12)
    np.testing.assert_allclose(out["v_cache"], pv, atol=1e-12)


def draft_tree(rng, truth, n_nodes, depth, break_at=None, V=96):
    """Parent array and tokens of a draft tree whose node 1.. path follows
    ``truth`` (the model's own continuation) for ``depth`` levels, changed at
    level ``break_at`` if given; the other nodes attach at random with random
    tokens."""
    parent = [-1]
    tokens = [-1]
    level = [0]
    prev = 0
    for lvl in range(1, depth + 1):
        parent.append(prev)
        tok = int(truth[lvl - 1])
        if break_at is not None and lvl == break_at:
            tok = (tok + 1) % V
        tokens.append(tok)
        level.append(lvl)
        prev = len(parent) - 1
    while len(parent) < n_nodes:
        cand = [i for i in range(len(parent)) if level[i] < depth]
        p = int(rng.choice(cand))
        parent.append(p)
        tokens.append(int(rng.integers(0, V)))
        level.append(level[p] + 1)
    # shuffle non-root labels while keeping parents before children
    order = [0] + sorted(range(1, len(parent)), key=lambda i: (level[i], rng.random()))
    new = {old: k for k, old in enumerate(order)}
    par = [-1] + [new[parent[old]] for old in order[1:]]
    tok = [tokens[old] for old in order]
    return np.array(par, np.int32), np.array(tok, np.int32)


@pytest.mark.parametrize("seed", [0, 1])
def test_tree_verification_reproduces_autoregressive_decoding(seed):
    """[Specular, 主要特性] / [SpecDec §2.2]: greedy verification leaves the
    output identical to the target's own greedy decoding."""
    params = _params(100 + seed, CFG)
    rng = np.random.default_rng(seed)
    prompt = rng.integers(0, CFG["V"], 6)
    n_new = 14
    ar, _ = oracle.ar_greedy_decode(params, CFG, prompt, n_new + 6)
    S_max = 64
    kc, vc = oracle.prefix_cache(params, CFG, prompt[:-1], S_max)
    P = len(prompt) - 1
    root = int(prompt[-1])
    gen = []
    step = 0
    while len(gen) < n_new:
        truth = ar[len(gen):]
        depth = 3
        par, tok = draft_tree(rng, truth, 9, depth, break_at=(2 if step % 3 == 1 else None))
        tok[0] = root
        node_off = np.array([0, len(par)], np.int32)
        out = oracle.tree_layer(params, CFG, tok, node_off, par, np.array([P], np.int32), kc, vc)
        acc = oracle.verify_greedy(node_off, par, tok, out["logits"], CFG["V"], depth)
        assert acc["status"] == 0
        L = int(acc["accept_len"][0])
        kc, vc, _, new_len, st = oracle.kv_compact(out["k_cache"], out["v_cache"],
                                                   np.array([P], np.int32), acc["accept_len"],
                                                   acc["accept_nodes"], depth + 1)
        assert st == 0 and int(new_len[0]) == P + L + 1
        emitted = [int(x) for x in acc["out_tokens"][0, :L + 1]]
        gen += emitted
        P = int(new_len[0])
        root = emitted[-1]
        step += 1
    assert gen[:n_new] == [int(x) for x in ar[:n_new]]
    # the compacted cache holds the keys of the decoded sequence
    seq = np.concatenate([prompt, np.array(gen[:-1], np.int32)])
    pk, pv = oracle.prefix_cache(params, CFG, seq, S_max)
    np.testing.assert_allclose(kc[:, :, :P], pk[:, :, :P], atol=1e-10)
    np.testing.assert_allclose(vc[:, :, :P], pv[:, :, :P], atol=1e-10)
