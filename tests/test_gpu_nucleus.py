"""GPU parity of stochastic acceptance with nucleus (top-p) sampling and with
the draft given as probabilities (st_verify_stochastic_ex) against the oracle.
Every request is compared exactly with the outcomes the oracle's walk can
reach when its near ties (a comparison within 1e-6, a residual mass in
(0, 2e-6], a draw on a bin edge, a nucleus cut whose mass lies within 1e-6 of
top_p) go either way; no request is skipped."""

import numpy as np
import pytest
import torch

import oracle
from synth import build_workload, make_workload, tree_random_attach
from token_tree_verification_st_amd import to_device
from token_tree_verification_st_amd import step as stp
from tests.gpu_util import device_paths, require_gpu, say, status_of, stochastic_parity

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _gpu():
    require_gpu()


def _probs(wl):
    z = wl.draft_logits.astype(np.float64) / wl.temperature
    p = np.exp(z - z.max(axis=1, keepdims=True))
    return (p / p.sum(axis=1, keepdims=True)).astype(np.float32)


def _check(wl, top_p, probs=False, dw=None):
    """Runs st_verify_stochastic_ex and compares every request with the
    oracle's outcomes; returns (accept_len, requests decided at a tie the
    other way)."""
    dw = dw or to_device(wl)
    draft_host = _probs(wl) if probs else wl.draft_logits
    draft = torch.from_numpy(draft_host).cuda() if probs else None
    stp.run_verify(dw, stochastic=True, top_p=top_p, draft=draft)
    torch.cuda.synchronize()
    al, _, _ = device_paths(dw)
    followed = stochastic_parity(wl, dw, draft_host=draft_host, top_p=top_p, probs=probs,
                                 label=f"top_p {top_p} probs {probs} offset {wl.rng_offset}")
    assert status_of(dw) == 0
    return al, followed


@pytest.mark.parametrize("name", ["stochastic_tree", "stochastic_chain"])
@pytest.mark.parametrize("top_p,probs", [(0.9, False), (1.0, True), (0.9, True), (0.5, False)])
def test_nucleus_named_workloads(name, top_p, probs):
    wl = make_workload(name, 0)
    al, followed = _check(wl, top_p, probs)
    say(f"{name} top_p={top_p} probs={probs}: accept_len {al.tolist()[:8]}... "
        f"requests decided at a tie the other way {followed} of {wl.B}")


@pytest.mark.parametrize("seed", range(3))
def test_nucleus_many_offsets_small_vocab(seed):
    rng = np.random.default_rng(300 + seed)
    B = 8
    trees = [tree_random_attach(rng, int(rng.integers(1, 40)), 6) for _ in range(B)]
    wl = build_workload("nuc", rng, dtype="bf16", Hq=1, Hkv=1, D=64, V=int(rng.integers(3, 60)),
                        prefix_lens=[1] * B, trees=trees, max_depth=6, token_rule="draft_sample",
                        logit_sigma=2.0, draft_noise_sigma=1.0, temperature=0.7 + 0.3 * seed)
    dw = to_device(wl)
    for off in range(12):
        wl.rng_offset = off
        dw.rng_offset = off
        _check(wl, (0.9, 0.6, 0.3)[off % 3], probs=bool(off & 1), dw=dw)


def test_ex_with_plain_options_equals_plain_entry_point():
    from token_tree_verification_st_amd import st_verify_stochastic_ex
    wl = make_workload("stochastic_tree", 1)
    dw = to_device(wl)
    stp.run_verify(dw, stochastic=True)
    torch.cuda.synchronize()
    plain = [x.copy() for x in device_paths(dw)]
    b = dw.buf
    for k in ("accept_len", "accept_nodes", "out_tokens"):
        b[k].fill_(-7)
    st_verify_stochastic_ex(dw.tree, dw.tokens, dw.logits, dw.draft_logits, dw.temperature,
                            dw.rng_seed, dw.rng_offset, b["accept_len"], b["accept_nodes"],
                            b["out_tokens"], b["verify_ws"], b["near_ties"], b["status"],
                            top_p=1.0, draft_is_probs=False)
    torch.cuda.synchronize()
    for x, y in zip(plain, device_paths(dw)):
        assert np.array_equal(x, y)


def test_rejects_bad_arguments_and_flags_negative_probabilities():
    wl = make_workload("stochastic_chain", 0)
    dw = to_device(wl)
    for top_p in (0.0, -0.5, 1.5, float("nan")):
        with pytest.raises(RuntimeError):
            stp.run_verify(dw, stochastic=True, top_p=top_p,
                           draft=torch.from_numpy(_probs(wl)).cuda())
    bad = _probs(wl)
    bad[0, 3] = -1e-3
    dw.buf["status"].zero_()
    stp.run_verify(dw, stochastic=True, top_p=0.9, draft=torch.from_numpy(bad).cuda())
    torch.cuda.synchronize()
    assert status_of(dw) & 4


@pytest.mark.parametrize("name", ["stochastic_tree", "stochastic_chain"])
@pytest.mark.parametrize("top_p,probs", [(0.9, False), (1.0, True), (0.6, True)])
def test_one_call_step_ex_equals_separate_calls(name, top_p, probs):
    """st_verification_step_ex gives what mask -> attention ->
    st_verify_stochastic_ex -> compaction give, bit for bit, and its
    acceptance follows the oracle up to near ties."""
    wl = make_workload(name, 0)
    a, b = to_device(wl), to_device(wl)
    draft = torch.from_numpy(_probs(wl)).cuda() if probs else None
    stp.verification_step(a, stochastic=True, fused=False, top_p=top_p, draft=draft)
    stp.verification_step(b, stochastic=True, fused=True, top_p=top_p, draft=draft)
    torch.cuda.synchronize()
    for k in ("accept_len", "accept_nodes", "out_tokens", "near_ties", "src_slot", "new_len",
              "status"):
        assert torch.equal(a.buf[k], b.buf[k]), k
    assert torch.equal(a.buf["out"], b.buf["out"]) and torch.equal(a.buf["lse"], b.buf["lse"])
    assert torch.equal(a.k_cache, b.k_cache) and torch.equal(a.v_cache, b.v_cache)
    # the separate path's acceptance against the oracle (fresh copies of the
    # workload: the step compacted a's caches, which acceptance does not read)
    _check(wl, top_p, probs)
    say(f"{name} top_p={top_p} probs={probs}: one-call step ex equals separate calls, "
        f"accept_len {b.buf['accept_len'].tolist()[:4]}")


def test_one_call_step_ex_plain_options_and_bad_arguments():
    from token_tree_verification_st_amd import st_verification_step_ex
    wl = make_workload("stochastic_tree", 2)
    a, b = to_device(wl), to_device(wl)
    stp.run_step(a, stochastic=True)
    bb = b.buf
    args = (b.tree, b.q, b.k_cache, b.v_cache, b.prefix_len, b.max_prefix, bb["out"], bb["lse"],
            b.tokens, b.logits, bb["accept_len"], bb["accept_nodes"], bb["out_tokens"],
            bb["src_slot"], bb["new_len"], bb["step_ws"], b.draft_logits)
    kw = dict(temperature=b.temperature, seed=b.rng_seed, offset=b.rng_offset,
              near_ties=bb["near_ties"], status=bb["status"])
    st_verification_step_ex(*args, **kw, top_p=1.0, draft_is_probs=False)
    torch.cuda.synchronize()
    for k in ("accept_len", "accept_nodes", "out_tokens", "near_ties", "new_len", "out"):
        assert torch.equal(a.buf[k], b.buf[k]), k
    assert torch.equal(a.k_cache, b.k_cache)
    for top_p in (0.0, -0.5, 1.5, float("nan")):
        with pytest.raises(RuntimeError):
            st_verification_step_ex(*args, **kw, top_p=top_p)


def _levels(rng, T, V, n):
    """Logits on n integer levels 0, -1, ..., -(n-1): thousands of exactly
    tied weights on every level."""
    return -rng.integers(0, n, size=(T, V)).astype(np.float32)


@pytest.mark.parametrize("pattern,top_p", [("plateaus", 0.9), ("flat", 0.90001),
                                           ("near_total", 0.99999), ("spike", 0.9),
                                           ("plateaus_draft_probs", 0.7), ("wide", 0.9)])
def test_nucleus_search_paths(pattern, top_p):
    """Rows that drive the nucleus search down each of its paths at full
    vocabulary: plateaus (thousands of weights tied at the cut, so the bounds
    never hold few enough entries to gather), a flat row (every token kept),
    a nucleus holding all but 1e-5 of the mass (the search may end at its
    starting bound), one dominant token (a one-token nucleus), and logits of
    spread 2.5 (a few hundred weights in the 1/8-binade bin of the cut: the
    larger sorting network)."""
    rng = np.random.default_rng(500 + len(pattern))
    B = 4
    trees = [tree_random_attach(rng, 24, 5) for _ in range(B)]
    # near_total at 4000 tokens: the running sums near the cut then move by
    # about 2.5e-4 a token, so few nodes land in the oracle's 1e-6 tie band
    wl = build_workload("paths", rng, dtype="bf16", Hq=1, Hkv=1, D=64,
                        V=4000 if pattern == "near_total" else 32000,
                        prefix_lens=[1] * B, trees=trees, max_depth=5, token_rule="uniform",
                        logit_sigma=1.0, draft_noise_sigma=0.5, temperature=1.0)
    T, V = wl.logits.shape
    if pattern.startswith("plateaus"):
        wl.logits[:] = _levels(rng, T, V, 6)
        wl.draft_logits[:] = _levels(rng, T, V, 4)
    elif pattern == "flat":
        wl.logits[:] = 0.0
        wl.draft_logits[:] = 0.0
    elif pattern == "wide":
        wl.logits[:] = rng.normal(0.0, 2.5, (T, V)).astype(np.float32)
        wl.draft_logits[:] = rng.normal(0.0, 2.5, (T, V)).astype(np.float32)
    elif pattern == "near_total":
        wl.logits[:] = rng.normal(0.0, 0.5, (T, V)).astype(np.float32)
        wl.draft_logits[:] = rng.normal(0.0, 0.5, (T, V)).astype(np.float32)
    else:   # spike: the node's own token dominates both rows
        wl.logits[:] = rng.normal(0.0, 1.0, (T, V)).astype(np.float32)
        wl.draft_logits[:] = rng.normal(0.0, 1.0, (T, V)).astype(np.float32)
        hot = rng.integers(0, V, size=T)
        wl.logits[np.arange(T), hot] += 30.0
        wl.draft_logits[np.arange(T), hot] += 30.0
    al, followed = _check(wl, top_p, probs=pattern.endswith("draft_probs"))
    say(f"{pattern} top_p={top_p}: accept_len {al.tolist()}, requests decided at a tie the "
        f"other way {followed} of {B}")


def test_second_rejection_residual_mass_is_relative():
    """Two rejections at one node (the explainer §2.2 residual, applied
    twice).  p = (.6000605, .3960395, .0039), q = (.6, .396, .004) given as
    probabilities, both children token 2, uniforms that reject child 1 and
    draw above .605 at the root.  After child 1 the residual is
    (.605, .395, 0); child 2 (r = 0 on its token) is rejected and leaves
    max(0, r - q) = (.005, 0, 0), half a percent of the current residual
    (5e-7 of p): it is renormalised to (1, 0, 0), so the draw gives token 0.
    Measuring that mass against p instead would keep (.605, .395, 0) and draw
    token 1."""
    from tests.test_gpu_verify_compact import _star_tree
    p = np.array([0.6000605, 0.3960395, 0.0039])
    q = np.array([0.6, 0.396, 0.004])
    rng = np.random.default_rng(8)
    wl = build_workload("tworej", rng, dtype="bf16", Hq=1, Hkv=1, D=64, V=3, prefix_lens=[1],
                        trees=[_star_tree(3)], max_depth=2, token_rule="uniform",
                        draft_noise_sigma=1.0, temperature=1.0)
    wl.tokens[:] = [0, 2, 2]
    wl.logits[:] = np.log(p).astype(np.float32)
    probs = np.tile(q.astype(np.float32), (3, 1))
    wl.draft_logits[:] = probs
    off = next(o for o in range(100000)
               if oracle.uniforms_for_node(0, o, 0, 1)[0] > 0.98
               and oracle.uniforms_for_node(0, o, 0, 0)[1] > 0.65)
    wl.rng_seed, wl.rng_offset = 0, off
    dw = to_device(wl)
    stp.run_verify(dw, stochastic=True, top_p=1.0, draft=torch.from_numpy(probs).cuda())
    torch.cuda.synchronize()
    assert stochastic_parity(wl, dw, draft_host=probs, probs=True) == 0
    al, an, ot = device_paths(dw)
    assert int(al[0]) == 0 and int(ot[0, 0]) == 0 and status_of(dw) == 0
    say(f"two rejections at offset {off}: token {int(ot[0, 0])}")
