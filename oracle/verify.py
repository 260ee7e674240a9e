"""Acceptance of a verified token tree: greedy and rejection sampling, fp64.

Sources:
  [SpecInfer-dev §2.1] accept the longest verified prefix of the tree.
  [SpecDec §2.2] check candidates left to right; accept a candidate with
      probability min(1, p_main / p_draft); at the first rejection drop the
      later candidates and emit a replacement token from the main model; the
      output then has exactly the main model's distribution.
  [Specular, 主要特性] greedy: the final output equals the original model's.

Readings used here (the pages leave them open):
  * logits row i holds the target's (and draft's) distribution for the
    children of node i;
  * greedy: a[i] = argmax of row i, lowest vocab index on ties; from the root,
    step to the lowest-index child whose token equals a[u]; the replacement
    ("bonus") token is a[u] at the last accepted node;
  * stochastic: p_i = softmax(target_i / T), q_i = softmax(draft_i / T); at
    node u with residual r (initially p_u), test the children in ascending
    index: child c with token x is accepted iff u_acc(c) * q_u[x] < r[x]
    (that is u < min(1, r/q) without a division); after a rejection
    r <- max(0, r - q_u) renormalised, kept as it was if its mass is at most
    1e-6 (a residual of the rounding of nearly equal r and q, which must not
    be renormalised into a distribution: two one-token nuclei on the same
    token leave exactly such a residual); when
    no child is accepted the replacement token is drawn from r by inverse CDF
    with u_smp(u), summing r in ascending vocab order.  The residual draw is
    what makes the equal-distribution guarantee hold;
  * accept_len L counts accepted non-root nodes; out_tokens holds their tokens
    followed by the replacement token, so L + 1 tokens are emitted;
  * if an accepted path would grow past ``max_depth`` nodes below the root the
    walk stops, status bit 8 is set and the replacement token is -1;
  * nucleus sampling (the pages' configuration and tuning table recommend
    top-p 0.9 alongside temperature 0.7): p and q are each restricted to their
    nucleus -- sort descending, take the first rank where the running sum
    reaches top_p of the total, keep every token at least as likely as that
    one -- and renormalised before any test.  Both are filtered because the
    draft tokens were drawn from the filtered draft and the output must follow
    the filtered target;
  * the draft may be given as probabilities (the explainer's
    calculate_accept_prob takes draft probabilities): q is then the row as
    given, normalised, with no temperature.
"""

from __future__ import annotations

import numpy as np

from .philox import uniforms_for_node
from .tree import (STATUS_BAD_TOKEN, STATUS_NONFINITE, STATUS_PATH_OVERFLOW, check_tree,
                   children_of)

NEAR_TIE_EPS = 1e-6


def _input_status(node_off, parent, tokens, V, rows):
    status = check_tree(node_off, parent)
    roots = set(int(x) for x in node_off[:-1])
    T = int(node_off[-1])
    for t in range(T):
        if t not in roots and not (0 <= int(tokens[t]) < V):   # a root's token is not checked
            status |= STATUS_BAD_TOKEN
    for r in rows:
        if r is not None and not np.all(np.isfinite(r)):
            status |= STATUS_NONFINITE
    return status


def verify_greedy(node_off, parent, tokens, logits, V: int, max_depth: int):
    """Returns dict(accept_len [B], accept_nodes [B][max_depth+1],
    out_tokens [B][max_depth+2], status)."""
    B = len(node_off) - 1
    status = _input_status(node_off, parent, tokens, V, [logits])
    accept_len = np.zeros(B, dtype=np.int32)
    accept_nodes = np.full((B, max_depth + 1), -1, dtype=np.int32)
    out_tokens = np.full((B, max_depth + 2), -1, dtype=np.int32)
    for b in range(B):
        lo, hi = int(node_off[b]), int(node_off[b + 1])
        par = [int(x) for x in parent[lo:hi]]
        choice = [int(np.argmax(np.asarray(logits[lo + i], dtype=np.float64)))
                  for i in range(hi - lo)]
        path = [0]
        u = 0
        overflow = False
        while True:
            nxt = None
            for c in children_of(par, u):
                if int(tokens[lo + c]) == choice[u]:
                    nxt = c
                    break
            if nxt is None:
                break
            if len(path) - 1 == max_depth:
                overflow = True
                break
            path.append(nxt)
            u = nxt
        L = len(path) - 1
        accept_len[b] = L
        accept_nodes[b, :L + 1] = path
        out_tokens[b, :L] = [int(tokens[lo + c]) for c in path[1:]]
        out_tokens[b, L] = -1 if overflow else choice[u]
        if overflow:
            status |= STATUS_PATH_OVERFLOW
    return dict(accept_len=accept_len, accept_nodes=accept_nodes, out_tokens=out_tokens,
                status=status)


def softmax_with_temperature(row, temperature: float) -> np.ndarray:
    z = np.asarray(row, dtype=np.float64) / float(temperature)
    e = np.exp(z - z.max())
    return e / e.sum()


def nucleus(prob, top_p: float):
    """prob restricted to its top-p nucleus and renormalised, and whether the
    cut is a near tie (the running sum at the cut, or just before it, within
    NEAR_TIE_EPS of top_p)."""
    prob = np.asarray(prob, dtype=np.float64)
    if top_p >= 1.0:
        return prob, False
    total = float(prob.sum())
    order = np.argsort(-prob, kind="stable")
    csum = np.cumsum(prob[order])
    target = top_p * total
    k = int(np.nonzero(csum >= target)[0][0])
    thr = prob[order[k]]
    kept = np.where(prob >= thr, prob, 0.0)
    tie = abs(csum[k] - target) < NEAR_TIE_EPS * total or \
        (k > 0 and abs(csum[k - 1] - target) < NEAR_TIE_EPS * total)
    return kept / kept.sum(), bool(tie)


def inverse_cdf(r: np.ndarray, u: float):
    """Smallest v whose running sum (ascending v) exceeds u * sum(r); if
    rounding leaves none, the last v with r[v] > 0.  Also reports whether the
    threshold falls within NEAR_TIE_EPS * sum(r) of the chosen bin's edges."""
    total = float(r.sum())
    thr = u * total
    csum = np.cumsum(r)
    hits = np.nonzero(csum > thr)[0]
    if len(hits):
        v = int(hits[0])
    else:
        v = int(np.nonzero(r > 0)[0][-1])
    lo_edge = float(csum[v - 1]) if v > 0 else 0.0
    tie = abs(float(csum[v]) - thr) < NEAR_TIE_EPS * total or \
        (v > 0 and abs(lo_edge - thr) < NEAR_TIE_EPS * total)
    return v, bool(tie)


def verify_stochastic(node_off, parent, tokens, target_logits, draft_logits, V: int,
                      temperature: float, seed: int, offset: int, max_depth: int,
                      follow=None, uniforms=None, top_p: float = 1.0, draft_probs: bool = False):
    """Multi-step rejection sampling down the tree.

    ``follow`` (optional) maps request -> accepted path observed elsewhere.  The
    walk then takes that path's decision wherever it differs from its own and
    records the difference in ``divergences`` with whether its own comparison
    was a near tie (|r[x] - u*q[x]| < 1e-6).

    ``uniforms`` (optional) replaces the Philox draws: a callable
    (request, local_node) -> (u_acc, u_smp), for hand-worked examples.

    ``top_p`` < 1 restricts p and q to their nuclei; ``draft_probs`` takes
    draft_logits as probabilities (rows of q as given).

    Returns dict(accept_len, accept_nodes, out_tokens, near_ties [B], status,
    divergences [B] (list of (node, child, near_tie)), bonus_tie [B],
    nucleus_ties [B] (near-tie nucleus cuts met on the walk), mass_ties [B]
    (residual masses within 2e-6 of zero after a rejection, where the
    no-mass rule below is decided by rounding)).
    """
    B = len(node_off) - 1
    if uniforms is None:
        def uniforms(req, node):
            return uniforms_for_node(seed, offset, req, node)
    status = _input_status(node_off, parent, tokens, V, [target_logits, draft_logits])
    accept_len = np.zeros(B, dtype=np.int32)
    accept_nodes = np.full((B, max_depth + 1), -1, dtype=np.int32)
    out_tokens = np.full((B, max_depth + 2), -1, dtype=np.int32)
    near_ties = np.zeros(B, dtype=np.int32)
    divergences = [[] for _ in range(B)]
    bonus_tie = np.zeros(B, dtype=bool)
    nucleus_ties = np.zeros(B, dtype=np.int32)
    mass_ties = np.zeros(B, dtype=np.int32)
    if draft_probs:
        T = int(node_off[-1])
        for t in range(T):
            row = np.asarray(draft_logits[t], dtype=np.float64)
            if np.any(row < 0) or not row.sum() > 0:
                status |= STATUS_NONFINITE

    def target_dist(b, t):
        d, tie = nucleus(softmax_with_temperature(target_logits[t], temperature), top_p)
        nucleus_ties[b] += int(tie)
        return d

    def draft_dist(b, t):
        if draft_probs:
            row = np.asarray(draft_logits[t], dtype=np.float64)
            row = row / row.sum()
        else:
            row = softmax_with_temperature(draft_logits[t], temperature)
        d, tie = nucleus(row, top_p)
        nucleus_ties[b] += int(tie)
        return d

    for b in range(B):
        lo, hi = int(node_off[b]), int(node_off[b + 1])
        par = [int(x) for x in parent[lo:hi]]
        path = [0]
        u = 0
        r = target_dist(b, lo)
        overflow = False
        forced = None if follow is None else [int(x) for x in follow[b]]
        while True:
            kids = children_of(par, u)
            q_u = draft_dist(b, lo + u) if kids else None
            accepted = None
            for c in kids:
                x = int(tokens[lo + c])
                u_acc, _ = uniforms(b, c)
                lhs = u_acc * q_u[x]
                rhs = r[x]
                tie = abs(rhs - lhs) < NEAR_TIE_EPS
                near_ties[b] += int(tie)
                take = lhs < rhs
                if forced is not None:
                    k = len(path)
                    want = k < len(forced) and forced[k] == c
                    if want != take:
                        divergences[b].append((u, c, bool(tie)))
                        take = want
                if take:
                    accepted = c
                    break
                resid = np.maximum(0.0, r - q_u)
                mass = resid.sum()
                if mass > NEAR_TIE_EPS:
                    r = resid / mass
                if 0.0 < mass <= 2 * NEAR_TIE_EPS:
                    mass_ties[b] += 1
            if accepted is None:
                break
            if len(path) - 1 == max_depth:
                overflow = True
                break
            path.append(accepted)
            u = accepted
            r = target_dist(b, lo + u)
        L = len(path) - 1
        accept_len[b] = L
        accept_nodes[b, :L + 1] = path
        out_tokens[b, :L] = [int(tokens[lo + c]) for c in path[1:]]
        if overflow:
            status |= STATUS_PATH_OVERFLOW
            out_tokens[b, L] = -1
        else:
            _, u_smp = uniforms(b, u)
            v, tie = inverse_cdf(r, u_smp)
            out_tokens[b, L] = v
            bonus_tie[b] = tie
            near_ties[b] += int(tie)
    return dict(accept_len=accept_len, accept_nodes=accept_nodes, out_tokens=out_tokens,
                near_ties=near_ties, status=status, divergences=divergences,
                bonus_tie=bonus_tie, nucleus_ties=nucleus_ties, mass_ties=mass_ties)
