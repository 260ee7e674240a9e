"""Pins for the oracle's greedy and stochastic acceptance: hand-worked examples,
plain greedy decoding of a toy model, the lossless guarantee as a statistical test,
the closed-form single-draft accept rate, and special cases."""

import zlib

import numpy as np
import pytest
from scipy.stats import chisquare

import oracle
from oracle.tree import STATUS_BAD_TOKEN, STATUS_NONFINITE, STATUS_PATH_OVERFLOW
from synth import make_workload, tree_chain, tree_random_attach


def _ints(g, k):
    return [int(x) for x in g[k]]


# ---------------------------------------------------------------- greedy


def test_greedy_hand_worked(golden):
    g = golden("greedy_small.txt")
    parent = np.array(_ints(g, "parent"), np.int32)
    tokens = np.array(_ints(g, "tokens"), np.int32)
    logits = np.array([[float(x) for x in r] for r in g["logits"]], np.float32)
    res = oracle.verify_greedy(np.array([0, len(parent)]), parent, tokens, logits, 4, 4)
    L = int(g["accept_len"][0])
    assert res["status"] == 0
    assert int(res["accept_len"][0]) == L
    assert res["accept_nodes"][0, :L + 1].tolist() == _ints(g, "accept_nodes")
    assert res["out_tokens"][0, :L + 1].tolist() == _ints(g, "out_tokens")
    assert (res["accept_nodes"][0, L + 1:] == -1).all() and (res["out_tokens"][0, L + 1:] == -1).all()


def _toy_logits(ctx, V, salt=0):
    rng = np.random.default_rng(zlib.crc32(np.asarray(ctx, np.int64).tobytes()) + salt)
    return (rng.standard_normal(V) * 2.0).astype(np.float32)


@pytest.mark.parametrize("seed", range(8))
def test_greedy_reproduces_plain_greedy_decoding(seed):
    """A deterministic toy target whose next-token logits depend on the whole token
    path.  The accepted tokens plus the bonus token must equal what plain
    token-by-token greedy decoding emits, and no child of the last accepted node may
    continue that sequence."""
    rng = np.random.default_rng(seed)
    V = 12
    root_ctx = (int(rng.integers(0, V)),)
    parent, ctxs = [-1], [root_ctx]
    frontier = [0]
    for _depth in range(4):
        nxt = []
        for u in frontier:
            for _ in range(int(rng.integers(0, 4))):
                if rng.random() < 0.5:
                    tok = int(np.argmax(_toy_logits(ctxs[u], V)))
                else:
                    tok = int(rng.integers(0, V))
                parent.append(u)
                ctxs.append(ctxs[u] + (tok,))
                nxt.append(len(parent) - 1)
        frontier = nxt
    n = len(parent)
    tokens = np.array([c[-1] for c in ctxs], np.int32)
    logits = np.stack([_toy_logits(c, V) for c in ctxs])
    res = oracle.verify_greedy(np.array([0, n]), np.array(parent, np.int32), tokens, logits, V, 8)
    L = int(res["accept_len"][0])
    ctx, seq = root_ctx, []
    for _ in range(L + 1):
        tok = int(np.argmax(_toy_logits(ctx, V)))
        seq.append(tok)
        ctx = ctx + (tok,)
    assert res["out_tokens"][0, :L + 1].tolist() == seq
    last = int(res["accept_nodes"][0, L])
    kids = [c for c in range(n) if parent[c] == last]
    assert all(int(tokens[c]) != seq[L] for c in kids)


def test_greedy_tiny_fp32_workload_accepts_planted_path():
    wl = make_workload("tiny_fp32", 0)
    a3 = int(np.argmax(wl.logits[3]))
    assert int(wl.tokens[7]) != a3 and int(wl.tokens[8]) != a3   # no chance hit below node 3
    res = oracle.verify_greedy(wl.node_off, wl.parent, wl.tokens, wl.logits, wl.V, wl.max_depth)
    assert int(res["accept_len"][0]) == 2
    assert res["accept_nodes"][0, :3].tolist() == [0, 1, 3]
    assert int(res["out_tokens"][0, 2]) == a3


def test_greedy_chain_all_or_none_accepted():
    rng = np.random.default_rng(1)
    V, n = 50, 6
    parent, _ = tree_chain(n)
    logits = rng.standard_normal((n, V)).astype(np.float32)
    a = logits.argmax(1)
    tokens = np.zeros(n, np.int32)
    tokens[1:] = a[:-1]
    res = oracle.verify_greedy(np.array([0, n]), parent, tokens, logits, V, 5)
    assert int(res["accept_len"][0]) == 5
    assert res["out_tokens"][0, :6].tolist() == list(a[:-1]) + [int(a[-1])]
    tokens[1:] = (a[:-1] + 1) % V
    res = oracle.verify_greedy(np.array([0, n]), parent, tokens, logits, V, 5)
    assert int(res["accept_len"][0]) == 0
    assert res["out_tokens"][0, 0] == a[0]


def test_greedy_ties_lowest_vocab_index_and_lowest_sibling():
    parent = np.array([-1, 0, 0, 0], np.int32)
    logits = np.zeros((4, 6), np.float32)
    logits[0, [2, 4]] = 3.0                       # tie between 2 and 4 -> 2
    tokens = np.array([0, 4, 2, 2], np.int32)     # nodes 2 and 3 both match -> node 2
    res = oracle.verify_greedy(np.array([0, 4]), parent, tokens, logits, 6, 3)
    assert res["accept_nodes"][0, :2].tolist() == [0, 2]
    assert int(res["out_tokens"][0, 1]) == 0      # row 2 all zero -> index 0


def test_greedy_overflow_and_input_status():
    n = 5
    parent, _ = tree_chain(n)
    logits = np.zeros((n, 3), np.float32)
    tokens = np.zeros(n, np.int32)                # every node matches argmax 0
    res = oracle.verify_greedy(np.array([0, n]), parent, tokens, logits, 3, 2)
    assert res["status"] & STATUS_PATH_OVERFLOW
    assert int(res["accept_len"][0]) == 2 and int(res["out_tokens"][0, 2]) == -1
    bad = tokens.copy()
    bad[3] = 3
    assert oracle.verify_greedy(np.array([0, n]), parent, bad, logits, 3, 8)["status"] & STATUS_BAD_TOKEN
    nf = logits.copy()
    nf[2, 1] = np.inf
    assert oracle.verify_greedy(np.array([0, n]), parent, tokens, nf, 3, 8)["status"] & STATUS_NONFINITE


# ---------------------------------------------------------------- stochastic


def _fixture_case(g, case):
    p = np.array([[float(x) for x in r] for r in g["p"]])
    q = np.array([[float(x) for x in r] for r in g["q"]])
    parent = np.array(_ints(g, "parent"), np.int32)
    tokens = np.array(_ints(g, f"{case}_tokens"), np.int32)
    ua = [float(x) for x in g[f"{case}_u_acc"]]
    us = [float(x) for x in g[f"{case}_u_smp"]]
    return p, q, parent, tokens, ua, us


@pytest.mark.parametrize("case", ["case1", "case2", "case3"])
def test_stochastic_hand_worked(golden, case):
    g = golden("stochastic_small.txt")
    p, q, parent, tokens, ua, us = _fixture_case(g, case)
    res = oracle.verify_stochastic(
        np.array([0, len(parent)]), parent, tokens, np.log(p).astype(np.float32),
        np.log(q).astype(np.float32), 3, 1.0, 0, 0, 4, uniforms=lambda b, i: (ua[i], us[i]))
    L = int(res["accept_len"][0])
    assert res["accept_nodes"][0, :L + 1].tolist() == _ints(g, f"{case}_accept_nodes")
    assert res["out_tokens"][0, :L + 1].tolist() == _ints(g, f"{case}_out_tokens")
    assert res["status"] == 0 and int(res["near_ties"][0]) == 0


def _softmax(x):
    e = np.exp(x - x.max())
    return e / e.sum()


class _ToyPair:
    """Target and draft next-token logits as seeded functions of the token path."""

    def __init__(self, V, salt, noise=1.5):
        self.V, self.salt, self.noise = V, salt, noise

    def logits(self, ctx):
        rng = np.random.default_rng(zlib.crc32(np.asarray(ctx, np.int64).tobytes()) + self.salt)
        t = rng.standard_normal(self.V) * 1.5
        d = t + rng.standard_normal(self.V) * self.noise
        return t.astype(np.float32), d.astype(np.float32)


def _draft_tree(pair, T, root_ctx, widths, rng):
    """Children of every node drawn i.i.d. from the draft at that node."""
    parent, ctxs, frontier = [-1], [root_ctx], [0]
    for w in widths:
        nxt = []
        for u in frontier:
            _, d = pair.logits(ctxs[u])
            qd = _softmax(d.astype(np.float64) / T)
            for tok in rng.choice(pair.V, size=w, p=qd):
                parent.append(u)
                ctxs.append(ctxs[u] + (int(tok),))
                nxt.append(len(parent) - 1)
        frontier = nxt
    tl = np.stack([pair.logits(c)[0] for c in ctxs])
    dl = np.stack([pair.logits(c)[1] for c in ctxs])
    tokens = np.array([c[-1] for c in ctxs], np.int32)
    return np.array(parent, np.int32), tokens, tl, dl


def test_stochastic_output_has_the_target_distribution():
    """Lossless guarantee: over many independent steps, the first emitted token
    follows the target's distribution, and so does the pair of the first two tokens
    (when a step emits only one token, the second is drawn from the target itself, as
    the next step would)."""
    V, T, trials = 5, 0.7, 16000
    pair = _ToyPair(V, salt=3)
    root_ctx = (1,)
    rng = np.random.default_rng(2024)
    first = np.zeros(V, np.int64)
    joint = np.zeros((V, V), np.int64)
    for t in range(trials):
        parent, tokens, tl, dl = _draft_tree(pair, T, root_ctx, (3, 2), rng)
        res = oracle.verify_stochastic(np.array([0, len(parent)]), parent, tokens, tl, dl, V, T,
                                       seed=99, offset=t, max_depth=4)
        L = int(res["accept_len"][0])
        t1 = int(res["out_tokens"][0, 0])
        if L >= 1:
            t2 = int(res["out_tokens"][0, 1])
        else:
            p2 = _softmax(pair.logits(root_ctx + (t1,))[0].astype(np.float64) / T)
            t2 = int(rng.choice(V, p=p2))
        first[t1] += 1
        joint[t1, t2] += 1
    p1 = _softmax(pair.logits(root_ctx)[0].astype(np.float64) / T)
    assert chisquare(first, p1 * trials).pvalue > 1e-3
    pj = np.array([[p1[a] * _softmax(pair.logits(root_ctx + (a,))[0].astype(np.float64) / T)[b]
                    for b in range(V)] for a in range(V)])
    assert chisquare(joint.ravel(), pj.ravel() * trials).pvalue > 1e-3


def test_single_draft_accept_rate_is_one_minus_total_variation():
    V, T, trials = 6, 1.0, 12000
    pair = _ToyPair(V, salt=8, noise=1.0)
    root_ctx = (2,)
    rng = np.random.default_rng(5)
    acc = 0
    for t in range(trials):
        parent, tokens, tl, dl = _draft_tree(pair, T, root_ctx, (1,), rng)
        res = oracle.verify_stochastic(np.array([0, 2]), parent, tokens, tl, dl, V, T,
                                       seed=1, offset=t, max_depth=2)
        acc += int(res["accept_len"][0])
    tl0, dl0 = pair.logits(root_ctx)
    p, q = _softmax(tl0.astype(np.float64)), _softmax(dl0.astype(np.float64))
    expect = np.minimum(p, q).sum()
    std = np.sqrt(expect * (1 - expect) / trials)
    assert abs(acc / trials - expect) < 4 * std


def test_equal_target_and_draft_always_accepts_first_child():
    rng = np.random.default_rng(12)
    n, V = 20, 40
    parent, _ = tree_random_attach(rng, n, 6)
    lg = (rng.standard_normal((n, V)) * 3).astype(np.float32)
    tokens = rng.integers(0, V, n).astype(np.int32)
    res = oracle.verify_stochastic(np.array([0, n]), parent, tokens, lg, lg, V, 0.7, 3, 0, 8)
    u, path = 0, [0]
    while True:
        kids = [c for c in range(n) if parent[c] == u]
        if not kids:
            break
        u = kids[0]
        path.append(u)
    L = int(res["accept_len"][0])
    assert res["accept_nodes"][0, :L + 1].tolist() == path


@pytest.mark.parametrize("seed", range(4))
def test_one_hot_target_reduces_to_greedy(seed):
    rng = np.random.default_rng(seed)
    n, V = 24, 30
    parent, _ = tree_random_attach(rng, n, 5)
    best = rng.integers(0, V, n)
    tl = np.full((n, V), -1000.0, np.float32)
    tl[np.arange(n), best] = 0.0
    dl = (rng.standard_normal((n, V)) * 2).astype(np.float32)
    tokens = rng.integers(0, V, n).astype(np.int32)
    for i in range(1, n):                        # make about half the nodes match
        if rng.random() < 0.5:
            tokens[i] = best[parent[i]]
    st = oracle.verify_stochastic(np.array([0, n]), parent, tokens, tl, dl, V, 1.0, 4, seed, 8)
    gr = oracle.verify_greedy(np.array([0, n]), parent, tokens, tl, V, 8)
    for k in ("accept_len", "accept_nodes", "out_tokens"):
        assert np.array_equal(st[k], gr[k]), k


def test_outcomes_without_ties_are_the_exact_walk():
    """On the named stochastic workloads (no near ties at seed 0) the tie
    enumeration yields one outcome per request: the exact rule's."""
    for name in ("stochastic_chain", "stochastic_tree"):
        wl = make_workload(name, 0)
        sl = slice(0, int(wl.node_off[4]))
        args = (wl.node_off[:5], wl.parent[sl], wl.tokens[sl], wl.logits[sl],
                wl.draft_logits[sl], wl.V, wl.temperature, wl.rng_seed, wl.rng_offset,
                wl.max_depth)
        own = oracle.verify_stochastic(*args)
        outs = oracle.stochastic_outcomes(*args)
        for b in range(4):
            first = outs[b][0]
            L = int(own["accept_len"][b])
            assert first["ties_flipped"] == 0
            assert first["accept_len"] == L
            assert first["accept_nodes"] == own["accept_nodes"][b, :L + 1].tolist()
            assert first["out_tokens"] == own["out_tokens"][b, :L + 1].tolist()
            assert first["near_ties"] == int(own["near_ties"][b])
            ties = own["near_ties"][b] + own["mass_ties"][b] + own["nucleus_ties"][b]
            assert len(outs[b]) == 1 or ties > 0


def _one_node(p, q, tokens, uni, top_p=1.0):
    """A root whose children carry `tokens`, target probabilities p (as
    logits, T = 1) and draft probabilities q, with the given uniforms."""
    n = len(tokens) + 1
    parent = np.array([-1] + [0] * (n - 1), np.int32)
    tok = np.array([0] + list(tokens), np.int32)
    tl = np.log(np.array([p] * n, np.float64))
    dl = np.array([q] * n, np.float64)
    args = (np.array([0, n]), parent, tok, tl, dl, len(p), 1.0, 0, 0, 2)
    kw = dict(uniforms=lambda b, i: uni[i], draft_probs=True, top_p=top_p)
    return oracle.verify_stochastic(*args, **kw), oracle.stochastic_outcomes(*args, **kw)[0]


def test_outcomes_comparison_tie_takes_both_decisions():
    """u q[x] within 1e-7 below r[x]: the exact rule accepts child 1; the
    other decision rejects it, leaves r = max(0, p - q)/0.1 = (1, 0), rejects
    child 2 (token 1, r = 0) and draws token 0 from (1, 0)."""
    p, q = [0.6, 0.4], [0.5, 0.5]
    uni = {1: ((0.6 - 1e-7) / 0.5, 0.3), 2: (0.2, 0.3), 0: (0.5, 0.7)}
    res, outs = _one_node(p, q, [0, 1], uni)
    assert res["accept_nodes"][0, :2].tolist() == [0, 1]
    got = {(o["accept_len"], tuple(o["out_tokens"])) for o in outs}
    assert (1, (0, int(res["out_tokens"][0, 1]))) in got
    assert (0, (0,)) in got
    assert outs[0]["ties_flipped"] == 0 and outs[0]["near_ties"] >= 1


def test_outcomes_draw_on_a_bin_edge_takes_both_bins():
    """A leaf root with r = (0.5, 0.5) and u_smp 1e-7 above one half: the
    threshold passes bin 0's upper edge by 1e-7, so token 1 is drawn and
    token 0 is the other outcome."""
    parent = np.array([-1], np.int32)
    tl = np.log(np.array([[0.5, 0.5]]))
    args = (np.array([0, 1]), parent, np.array([0], np.int32), tl, tl, 2, 1.0, 0, 0, 2)
    kw = dict(uniforms=lambda b, i: (0.5, 0.5 + 1e-7))
    res = oracle.verify_stochastic(*args, **kw)
    outs = oracle.stochastic_outcomes(*args, **kw)[0]
    assert res["out_tokens"][0, 0] == 1 and res["bonus_tie"][0]
    assert sorted(o["out_tokens"][0] for o in outs) == [0, 1]


def test_outcomes_nucleus_tie_takes_both_cuts():
    """Sorted target (0.5, 0.3, 0.2) with top_p 0.8 + 1e-8: the running sum
    0.8 sits at the cut, so the nucleus holds three tokens by the exact rule
    and two (0.625, 0.375) by the other rounding.  A leaf root with
    u_smp = 0.9 draws token 2 from the three-token nucleus and token 1 from
    the two-token one."""
    parent = np.array([-1], np.int32)
    tl = np.log(np.array([[0.5, 0.3, 0.2]]))
    args = (np.array([0, 1]), parent, np.array([0], np.int32), tl, tl, 3, 1.0, 0, 0, 2)
    kw = dict(uniforms=lambda b, i: (0.5, 0.9), top_p=0.8 + 1e-8)
    res = oracle.verify_stochastic(*args, **kw)
    outs = oracle.stochastic_outcomes(*args, **kw)[0]
    assert res["nucleus_ties"][0] == 1 and res["out_tokens"][0, 0] == 2
    assert sorted(o["out_tokens"][0] for o in outs) == [1, 2]


# ---------------------------------------------------------------- nucleus and draft probabilities


def test_nucleus_hand_worked():
    p = np.array([0.05, 0.5, 0.15, 0.3])
    d, tie = oracle.nucleus(p, 0.9)          # running sums 0.5, 0.8, 0.95: three kept
    np.testing.assert_allclose(d, [0.0, 0.5 / 0.95, 0.15 / 0.95, 0.3 / 0.95], atol=1e-15)
    assert not tie
    d, _ = oracle.nucleus(p, 0.75)           # 0.5, 0.8: two kept
    np.testing.assert_allclose(d, [0.0, 0.5 / 0.8, 0.0, 0.3 / 0.8], atol=1e-15)
    d, _ = oracle.nucleus(p, 0.3)            # the top token alone
    np.testing.assert_array_equal(d, [0.0, 1.0, 0.0, 0.0])
    d, _ = oracle.nucleus(p, 1.0)
    np.testing.assert_array_equal(d, p)
    # tokens as likely as the last one needed are all kept
    d, _ = oracle.nucleus(np.array([0.4, 0.2, 0.2, 0.2]), 0.5)
    np.testing.assert_allclose(d, [0.4, 0.2, 0.2, 0.2], atol=1e-15)
    # the cut lands on 0.75: the two-token set holds exactly top_p, and the
    # three-token set is what a rounding of that sum below 0.75 would keep
    vs, tie = oracle.nucleus_variants(np.array([0.5, 0.25, 0.2, 0.05]), 0.75)
    assert tie and len(vs) == 2
    np.testing.assert_allclose(vs[0], [0.5 / 0.75, 0.25 / 0.75, 0.0, 0.0], atol=1e-15)
    np.testing.assert_allclose(vs[1], [0.5 / 0.95, 0.25 / 0.95, 0.2 / 0.95, 0.0], atol=1e-15)
    # a level of equal tokens is kept or dropped whole: with (0.5, 0.25, 0.25)
    # the sets are {0.5} (0.5) and everything (1.0), neither near 0.75
    vs, tie = oracle.nucleus_variants(np.array([0.5, 0.25, 0.25]), 0.75)
    assert not tie and len(vs) == 1


def test_draft_probabilities_equal_draft_logits():
    wl = make_workload("stochastic_tree", 0)
    sl = slice(0, int(wl.node_off[3]))
    T = wl.temperature
    dl = wl.draft_logits[sl].astype(np.float64) / T
    probs = np.exp(dl - dl.max(axis=1, keepdims=True))
    probs /= probs.sum(axis=1, keepdims=True)
    base = (wl.node_off[:4], wl.parent[sl], wl.tokens[sl], wl.logits[sl])
    tail = (wl.V, T, wl.rng_seed, wl.rng_offset, wl.max_depth)
    a = oracle.verify_stochastic(*base, wl.draft_logits[sl], *tail)
    b = oracle.verify_stochastic(*base, probs, *tail, draft_probs=True)
    for k in ("accept_len", "accept_nodes", "out_tokens"):
        assert np.array_equal(a[k], b[k]), k
    bad = probs.copy()
    bad[0, 0] = -0.1
    assert oracle.verify_stochastic(*base, bad, *tail, draft_probs=True)["status"] & STATUS_NONFINITE


def _draft_tree_nucleus(pair, T, root_ctx, widths, rng, top_p):
    parent, ctxs, frontier = [-1], [root_ctx], [0]
    for w in widths:
        nxt = []
        for u in frontier:
            _, d = pair.logits(ctxs[u])
            qd, _ = oracle.nucleus(_softmax(d.astype(np.float64) / T), top_p)
            for tok in rng.choice(pair.V, size=w, p=qd):
                parent.append(u)
                ctxs.append(ctxs[u] + (int(tok),))
                nxt.append(len(parent) - 1)
        frontier = nxt
    tl = np.stack([pair.logits(c)[0] for c in ctxs])
    dl = np.stack([pair.logits(c)[1] for c in ctxs])
    tokens = np.array([c[-1] for c in ctxs], np.int32)
    return np.array(parent, np.int32), tokens, tl, dl


def test_nucleus_output_has_the_filtered_target_distribution():
    """With drafts drawn from the draft's nucleus, the first emitted token
    follows the target's nucleus distribution (and never leaves it)."""
    V, T, top_p, trials = 8, 1.5, 0.8, 12000
    pair = _ToyPair(V, salt=11)             # a nucleus of 4 of the 8 tokens at the root
    root_ctx = (4,)
    rng = np.random.default_rng(77)
    first = np.zeros(V, np.int64)
    for t in range(trials):
        parent, tokens, tl, dl = _draft_tree_nucleus(pair, T, root_ctx, (3, 2), rng, top_p)
        res = oracle.verify_stochastic(np.array([0, len(parent)]), parent, tokens, tl, dl, V, T,
                                       seed=5, offset=t, max_depth=4, top_p=top_p)
        first[int(res["out_tokens"][0, 0])] += 1
    p1, _ = oracle.nucleus(_softmax(pair.logits(root_ctx)[0].astype(np.float64) / T), top_p)
    keep = p1 > 0
    assert keep.sum() < V and first[~keep].sum() == 0
    assert chisquare(first[keep], p1[keep] * trials).pvalue > 1e-3


@pytest.mark.parametrize("seed", range(3))
def test_tiny_nucleus_reduces_to_greedy(seed):
    """A nucleus that keeps only the top target token makes acceptance greedy."""
    rng = np.random.default_rng(seed)
    n, V = 24, 30
    parent, _ = tree_random_attach(rng, n, 5)
    tl = (rng.standard_normal((n, V)) * 2).astype(np.float32)
    dl = (rng.standard_normal((n, V)) * 2).astype(np.float32)
    best = tl.argmax(axis=1)
    tokens = rng.integers(0, V, n).astype(np.int32)
    for i in range(1, n):
        if rng.random() < 0.5:
            tokens[i] = best[parent[i]]
    st = oracle.verify_stochastic(np.array([0, n]), parent, tokens, tl, dl, V, 1.0, 4, seed, 8,
                                  top_p=1e-6)
    gr = oracle.verify_greedy(np.array([0, n]), parent, tokens, tl, V, 8)
    # r is one-hot at the argmax: a child carrying it is accepted whatever q
    # says (u q < 1), any other is rejected, and a rejection leaves r one-hot
    for k in ("accept_len", "accept_nodes", "out_tokens"):
        assert np.array_equal(st[k], gr[k]), k


def test_residual_mass_rule_is_exact():
    """After a rejection the residual max(0, r - q) is renormalised whenever
    it has any mass, however small (the explainer §2.2 residual: anything
    else changes the output distribution), and r is kept only when that mass
    is exactly 0.  Masses in (0, 2e-6] are reported as mass ties."""
    V = 2
    parent = np.array([-1, 0, 0], np.int32)
    # equal one-hot rows: child 1 (token 1, q = 0) is rejected and leaves no
    # residual at all (p <= q everywhere), so r stays p and child 2 (token 0)
    # is accepted
    uni = {1: (0.999, 0.5), 2: (0.9, 0.5), 0: (0.5, 0.5)}
    tl = np.array([[0.0, -1000.0]] * 3, np.float32)     # exp(-1000) is 0 in fp64
    res = oracle.verify_stochastic(np.array([0, 3]), parent, np.array([0, 1, 0], np.int32), tl,
                                   tl, V, 1.0, 0, 0, 2, uniforms=lambda b, i: uni[i])
    assert res["accept_nodes"][0, :2].tolist() == [0, 2]
    assert int(res["mass_ties"][0]) == 0
    # p exceeds q by 5e-7 on token 0.  Child 1 (token 1): u q = 0.49999995 is
    # not below r = 0.4999995, rejected; the residual (5e-7, 0) is
    # renormalised to (1, 0).  Child 2 (token 1): r = 0, rejected; the
    # residual of (1, 0) against q is (0.5, 0) -> (1, 0); the draw gives 0.
    res, outs = _one_node([0.5 + 5e-7, 0.5 - 5e-7], [0.5, 0.5], [1, 1],
                          {1: (0.9999999, 0.5), 2: (0.9, 0.5), 0: (0.5, 0.5)})
    assert int(res["accept_len"][0]) == 0
    assert res["out_tokens"][0, 0] == 0
    assert int(res["mass_ties"][0]) == 1
    # keeping r instead (what rounding to no mass would do) accepts child 2
    assert {(o["accept_len"], tuple(o["out_tokens"])) for o in outs} == {(0, (0,)), (1, (1, 0)),
                                                                          (1, (1, 1))}


def test_residual_mass_is_relative_to_the_current_residual():
    """Two rejections at one node.  p = (.6000605, .3960395, .0039) and
    q = (.6, .396, .004), both children token 2, u_acc .999999, u_smp .9.
    Child 1: u q = .003999996 > .0039, rejected; residual (6.05e-5, 3.95e-5, 0)
    of mass 1e-4 -> r = (.605, .395, 0).  Child 2: r = 0, rejected; residual
    max(0, r - q) = (.005, 0, 0) of mass .005 (of r) -> (1, 0, 0); the draw
    gives token 0.  As a fraction of p that second mass is only 5e-7, which
    must not count as none."""
    p = [0.6000605, 0.3960395, 0.0039]
    q = [0.6, 0.396, 0.004]
    res, outs = _one_node(p, q, [2, 2], {1: (0.999999, 0.9), 2: (0.999999, 0.9), 0: (0.5, 0.9)})
    assert int(res["accept_len"][0]) == 0
    assert res["out_tokens"][0, 0] == 0
    assert int(res["mass_ties"][0]) == 0 and int(res["near_ties"][0]) == 0
    assert len(outs) == 1
