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
    r <- max(0, r - q_u) renormalised whenever that residual has any mass,
    and kept as it was only when its mass is exactly 0 (r <= q_u everywhere:
    the rejected token's distribution is then unchanged); when no child is
    accepted the replacement token is drawn from r by inverse CDF with
    u_smp(u), summing r in ascending vocab order.  The residual draw is what
    makes the equal-distribution guarantee hold;
  * near ties: a comparison |r[x] - u q[x]| < 1e-6, a residual mass in
    (0, 2e-6], a nucleus cut whose running sum lies within 1e-6 of top_p and a
    draw within 1e-6 of a bin edge are decided by rounding in any finite
    precision; stochastic_outcomes lists what each may lead to;
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


def _at_or_above(prob, thr):
    """prob restricted to the entries at least thr, renormalised."""
    kept = np.where(prob >= thr, prob, 0.0)
    return kept / kept.sum()


def nucleus_variants(prob, top_p: float):
    """prob restricted to its top-p nucleus and renormalised (first entry):
    sorted descending, the first rank whose running sum reaches top_p of the
    total sets the cut, and every token at least as likely as that rank's is
    kept.  Whether a set of tokens holds top_p of the mass is decided by its
    sum, and the candidate sets are the value levels: all tokens at or above
    some probability.  When the level chosen holds a mass within NEAR_TIE_EPS
    of top_p, the next lower level (one more level of tokens) follows as a
    variant; when the next higher level does, that level follows.  Also
    returns whether the cut is a near tie."""
    prob = np.asarray(prob, dtype=np.float64)
    if top_p >= 1.0:
        return [prob], False
    total = float(prob.sum())
    sp = prob[np.argsort(-prob, kind="stable")]
    csum = np.cumsum(sp)
    target = top_p * total
    k = int(np.nonzero(csum >= target)[0][0])
    start = int(np.nonzero(sp == sp[k])[0][0])       # the level of rank k, in rank order
    end = int(np.nonzero(sp == sp[k])[0][-1])
    out = [_at_or_above(prob, sp[k])]
    near_at = abs(csum[end] - target) < NEAR_TIE_EPS * total
    near_before = start > 0 and abs(csum[start - 1] - target) < NEAR_TIE_EPS * total
    if near_before:
        out.append(_at_or_above(prob, sp[start - 1]))
    if near_at and end + 1 < len(sp) and sp[end + 1] > 0:
        out.append(_at_or_above(prob, sp[end + 1]))
    return out, bool(near_at or near_before)


def nucleus(prob, top_p: float):
    """prob restricted to its top-p nucleus and renormalised, and whether the
    cut is a near tie (the running sum at the cut, or just before it, within
    NEAR_TIE_EPS of top_p)."""
    variants, tie = nucleus_variants(prob, top_p)
    return variants[0], tie


def inverse_cdf_variants(r: np.ndarray, u: float):
    """Smallest v whose running sum (ascending v) exceeds u * sum(r); if
    rounding leaves none, the last v with r[v] > 0 (first entry of the list).
    When the threshold falls within NEAR_TIE_EPS * sum(r) of that bin's lower
    edge, the previous bin with mass follows; within it of the upper edge, the
    next one.  Also returns whether the draw is a near tie."""
    total = float(r.sum())
    thr = u * total
    csum = np.cumsum(r)
    hits = np.nonzero(csum > thr)[0]
    if len(hits):
        v = int(hits[0])
    else:
        v = int(np.nonzero(r > 0)[0][-1])
    lo_edge = float(csum[v - 1]) if v > 0 else 0.0
    near_hi = abs(float(csum[v]) - thr) < NEAR_TIE_EPS * total
    near_lo = v > 0 and abs(lo_edge - thr) < NEAR_TIE_EPS * total
    out = [v]
    if near_lo:
        before = np.nonzero(r[:v] > 0)[0]
        if len(before):
            out.append(int(before[-1]))
    if near_hi:
        after = np.nonzero(r[v + 1:] > 0)[0]
        if len(after):
            out.append(v + 1 + int(after[0]))
    return out, bool(near_hi or near_lo)


def inverse_cdf(r: np.ndarray, u: float):
    """Smallest v whose running sum (ascending v) exceeds u * sum(r); if
    rounding leaves none, the last v with r[v] > 0.  Also reports whether the
    threshold falls within NEAR_TIE_EPS * sum(r) of the chosen bin's edges."""
    variants, tie = inverse_cdf_variants(r, u)
    return variants[0], tie


class _Choices:
    """The decisions a walk takes at its near ties.  The k-th near tie met
    takes option script[k] (0 = the exact rule's own decision) when the
    script reaches that far, else option 0; the number of options of every
    tie met is recorded, so that all combinations can be enumerated."""

    def __init__(self, script=()):
        self.script = list(script)
        self.options = []

    def pick(self, n_options: int) -> int:
        k = len(self.options)
        self.options.append(int(n_options))
        return self.script[k] if k < len(self.script) else 0


def _stochastic_walk(b, lo, hi, parent, tokens, V, target_dist, draft_dist, uniforms,
                     max_depth, choices):
    """Rejection sampling down request b's tree (nodes lo..hi-1).

    target_dist(t) / draft_dist(t) return the list of the row's possible
    distributions (first entry: the exact one; more only at a near-tie nucleus
    cut).  Every near tie consults ``choices``.  Returns the walk's outcome."""
    par = [int(x) for x in parent[lo:hi]]
    path = [0]
    u = 0
    tally = dict(near_ties=0, nucleus_ties=0, mass_ties=0, comparison_ties=0, bonus_tie=False)

    def dist(fn, t):
        variants = fn(t)
        if len(variants) > 1:
            tally["nucleus_ties"] += 1
            return variants[choices.pick(len(variants))]
        return variants[0]

    r = dist(target_dist, lo)
    overflow = False
    while True:
        kids = children_of(par, u)
        q_u = dist(draft_dist, lo + u) if kids else None
        accepted = None
        for c in kids:
            x = int(tokens[lo + c])
            u_acc, _ = uniforms(b, c)
            lhs = u_acc * q_u[x]
            rhs = r[x]
            take = lhs < rhs
            if abs(rhs - lhs) < NEAR_TIE_EPS:            # decided by rounding either way
                tally["near_ties"] += 1
                tally["comparison_ties"] += 1
                if choices.pick(2):
                    take = not take
            if take:
                accepted = c
                break
            # r <- max(0, r - q_u) renormalised; with no mass left r stays as it was
            resid = np.maximum(0.0, r - q_u)
            mass = resid.sum()
            renorm = mass > 0.0
            if 0.0 < mass <= 2 * NEAR_TIE_EPS:           # no mass up to rounding
                tally["mass_ties"] += 1
                if choices.pick(2):
                    renorm = False
            if renorm:
                r = resid / mass
        if accepted is None:
            break
        if len(path) - 1 == max_depth:
            overflow = True
            break
        path.append(accepted)
        u = accepted
        r = dist(target_dist, lo + u)
    L = len(path) - 1
    out_tokens = [int(tokens[lo + c]) for c in path[1:]]
    if overflow:
        out_tokens.append(-1)
    else:
        _, u_smp = uniforms(b, u)
        variants, tie = inverse_cdf_variants(r, u_smp)
        tally["bonus_tie"] = tie
        tally["near_ties"] += int(tie)
        out_tokens.append(variants[choices.pick(len(variants))] if len(variants) > 1
                          else variants[0])
    return dict(accept_len=L, accept_nodes=path, out_tokens=out_tokens, overflow=overflow,
                **tally)


def _stochastic_setup(node_off, parent, tokens, target_logits, draft_logits, V, temperature,
                      seed, offset, uniforms, top_p, draft_probs):
    if uniforms is None:
        def uniforms(req, node):
            return uniforms_for_node(seed, offset, req, node)
    status = _input_status(node_off, parent, tokens, V, [target_logits, draft_logits])
    if draft_probs:
        for t in range(int(node_off[-1])):
            row = np.asarray(draft_logits[t], dtype=np.float64)
            if np.any(row < 0) or not row.sum() > 0:
                status |= STATUS_NONFINITE

    def target_dist(t):
        return nucleus_variants(softmax_with_temperature(target_logits[t], temperature), top_p)[0]

    def draft_dist(t):
        if draft_probs:
            row = np.asarray(draft_logits[t], dtype=np.float64)
            row = row / row.sum()
        else:
            row = softmax_with_temperature(draft_logits[t], temperature)
        return nucleus_variants(row, top_p)[0]

    return uniforms, status, target_dist, draft_dist


def verify_stochastic(node_off, parent, tokens, target_logits, draft_logits, V: int,
                      temperature: float, seed: int, offset: int, max_depth: int,
                      uniforms=None, top_p: float = 1.0, draft_probs: bool = False):
    """Multi-step rejection sampling down the tree, by the exact rule.

    ``uniforms`` (optional) replaces the Philox draws: a callable
    (request, local_node) -> (u_acc, u_smp), for hand-worked examples.

    ``top_p`` < 1 restricts p and q to their nuclei; ``draft_probs`` takes
    draft_logits as probabilities (rows of q as given).

    Returns dict(accept_len, accept_nodes, out_tokens, near_ties [B], status,
    bonus_tie [B], nucleus_ties [B] (near-tie nucleus cuts met on the walk),
    mass_ties [B] (residual masses in (0, 2e-6] after a rejection, which the
    exact rule renormalises but which rounding could have left at zero)).
    """
    B = len(node_off) - 1
    uniforms, status, target_dist, draft_dist = _stochastic_setup(
        node_off, parent, tokens, target_logits, draft_logits, V, temperature, seed, offset,
        uniforms, top_p, draft_probs)
    accept_len = np.zeros(B, dtype=np.int32)
    accept_nodes = np.full((B, max_depth + 1), -1, dtype=np.int32)
    out_tokens = np.full((B, max_depth + 2), -1, dtype=np.int32)
    near_ties = np.zeros(B, dtype=np.int32)
    bonus_tie = np.zeros(B, dtype=bool)
    nucleus_ties = np.zeros(B, dtype=np.int32)
    mass_ties = np.zeros(B, dtype=np.int32)
    for b in range(B):
        lo, hi = int(node_off[b]), int(node_off[b + 1])
        w = _stochastic_walk(b, lo, hi, parent, tokens, V, target_dist, draft_dist, uniforms,
                             max_depth, _Choices())
        L = w["accept_len"]
        accept_len[b] = L
        accept_nodes[b, :L + 1] = w["accept_nodes"]
        out_tokens[b, :L + 1] = w["out_tokens"]
        near_ties[b] = w["near_ties"]
        bonus_tie[b] = w["bonus_tie"]
        nucleus_ties[b] = w["nucleus_ties"]
        mass_ties[b] = w["mass_ties"]
        if w["overflow"]:
            status |= STATUS_PATH_OVERFLOW
    return dict(accept_len=accept_len, accept_nodes=accept_nodes, out_tokens=out_tokens,
                near_ties=near_ties, status=status, bonus_tie=bonus_tie,
                nucleus_ties=nucleus_ties, mass_ties=mass_ties)


def stochastic_outcomes(node_off, parent, tokens, target_logits, draft_logits, V: int,
                        temperature: float, seed: int, offset: int, max_depth: int,
                        uniforms=None, top_p: float = 1.0, draft_probs: bool = False,
                        limit: int = 256):
    """Every outcome of the walk of each request when each near tie it meets
    may go either way: a comparison within NEAR_TIE_EPS (accept or reject), a
    residual mass in (0, 2e-6] (renormalised or none), a nucleus cut near top_p
    (one rank smaller or larger) and a draw on a bin edge (the neighbouring
    bin).  Between ties every decision is the exact rule's.

    Returns a list over requests; entry b is a list of dicts (accept_len,
    accept_nodes, out_tokens, near_ties, ties_flipped), the first being the
    exact rule's own outcome (ties_flipped 0).  At most ``limit`` outcomes per
    request are enumerated (more raises)."""
    B = len(node_off) - 1
    uniforms, _, target_dist, draft_dist = _stochastic_setup(
        node_off, parent, tokens, target_logits, draft_logits, V, temperature, seed, offset,
        uniforms, top_p, draft_probs)
    result = []
    for b in range(B):
        lo, hi = int(node_off[b]), int(node_off[b + 1])
        outs = []
        pending = [[]]
        while pending:
            script = pending.pop()
            ch = _Choices(script)
            w = _stochastic_walk(b, lo, hi, parent, tokens, V, target_dist, draft_dist,
                                 uniforms, max_depth, ch)
            outs.append(dict(accept_len=w["accept_len"], accept_nodes=list(w["accept_nodes"]),
                             out_tokens=list(w["out_tokens"]), near_ties=w["near_ties"],
                             ties_flipped=sum(1 for s in script if s)))
            if len(outs) > limit:
                raise RuntimeError(f"request {b}: more than {limit} near-tie outcomes")
            # every later tie (beyond the script) may take each of its other options
            for k in range(len(script), len(ch.options)):
                for opt in range(1, ch.options[k]):
                    pending.append(script + [0] * (k - len(script)) + [opt])
        result.append(outs)
    return result
