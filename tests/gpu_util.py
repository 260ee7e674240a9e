"""Helpers for the GPU parity tests: run the HIP path through the C ABI on a
seeded workload and compare with the oracle on the same host bytes."""

import contextlib
import sys

import numpy as np
import pytest
import torch

import oracle
from token_tree_verification_st_amd import load_library, to_device
from token_tree_verification_st_amd.binding import st_testing_set_plan
from token_tree_verification_st_amd import step as stp

BF16_TOL = 1e-2   # max-abs error, bf16 inputs with fp32 accumulation
F32_TOL = 1e-5    # max-abs error, fp32 inputs


def require_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    load_library()  # raises if libst.so is missing


@contextlib.contextmanager
def plan_override(**fields):
    """Planner overrides (st_testing_plan fields) for the calls inside the
    block, workspace queries included."""
    st_testing_set_plan(fields)
    try:
        yield
    finally:
        st_testing_set_plan(None)


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def status_of(dw) -> int:
    return int(dw.buf["status"].item())


def gpu_mask(dw):
    stp.run_mask(dw)
    torch.cuda.synchronize()
    W = dw.tree.W
    mask = dw.buf["mask"].cpu().numpy().view(np.uint64).reshape(dw.T, W)
    return mask, dw.buf["depth"].cpu().numpy()


def attention_errors(wl, dw, nodes=None, heads=None, derive_mask=False):
    """Run mask + attention on the GPU (or attention alone, deriving the
    ancestor masks in the kernel); return (max-abs out error, max-abs lse
    error) against the oracle over the given (or all) rows."""
    if derive_mask:
        stp.run_attention(dw, derive_mask=True)
    else:
        stp.run_mask(dw)
        stp.run_attention(dw)
    torch.cuda.synchronize()
    out = dw.buf["out"].float().cpu().numpy().astype(np.float64)
    lse = dw.buf["lse"].cpu().numpy().astype(np.float64)
    ref, ref_lse = oracle.tree_attention(wl.q, wl.k_cache, wl.v_cache, wl.dtype, wl.Hq, wl.Hkv,
                                         wl.node_off, wl.parent, wl.prefix_len, nodes=nodes,
                                         heads=heads)
    sel = ~np.isnan(ref_lse)
    assert sel.any()
    assert np.isfinite(out[sel]).all()
    err = np.abs(out[sel] - ref[sel]).max()
    lerr = np.abs(lse[sel] - ref_lse[sel]).max()
    return float(err), float(lerr)


def device_paths(dw):
    al = dw.buf["accept_len"].cpu().numpy()
    an = dw.buf["accept_nodes"].cpu().numpy()
    ot = dw.buf["out_tokens"].cpu().numpy()
    return al, an, ot


def stochastic_parity(wl, dw, draft_host=None, top_p=1.0, probs=False, label=""):
    """The GPU's stochastic acceptance (already run on dw) against the
    oracle, request by request and exactly: accept_len, the accepted nodes,
    the emitted tokens (bonus included), the -1 padding and the near-tie
    count must equal one of the outcomes the oracle's walk can reach when the
    near ties it meets go either way (the first outcome is the exact rule's;
    every decision between ties is the exact rule's).  Returns how many
    requests matched only an outcome with a tie decided the other way."""
    al, an, ot = device_paths(dw)
    ties_gpu = dw.buf["near_ties"].cpu().numpy()
    draft = wl.draft_logits if draft_host is None else draft_host
    outs = oracle.stochastic_outcomes(wl.node_off, wl.parent, wl.tokens, wl.logits, draft, wl.V,
                                      wl.temperature, wl.rng_seed, wl.rng_offset, wl.max_depth,
                                      top_p=top_p, draft_probs=probs)
    followed = 0
    for b in range(wl.B):
        L = int(al[b])
        assert (an[b, L + 1:] == -1).all() and (ot[b, L + 1:] == -1).all(), f"request {b}"
        got = (L, an[b, :L + 1].tolist(), ot[b, :L + 1].tolist(), int(ties_gpu[b]))
        match = [o for o in outs[b]
                 if (o["accept_len"], o["accept_nodes"], o["out_tokens"], o["near_ties"]) == got]
        assert match, (f"{label} request {b}: GPU (L, path, tokens, near ties) {got} is none of "
                       f"the oracle's {[(o['accept_len'], o['accept_nodes'], o['out_tokens'], o['near_ties']) for o in outs[b]]}")
        followed += min(o["ties_flipped"] for o in match) > 0
    return followed
