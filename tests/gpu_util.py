"""Helpers for the GPU parity tests: run the HIP path through the C ABI on a
seeded workload and compare with the oracle on the same host bytes."""

import sys

import numpy as np
import pytest
import torch

import oracle
from token_tree_verification_st_amd import load_library, to_device
from token_tree_verification_st_amd import step as stp

BF16_TOL = 1e-2   # max-abs error, bf16 inputs with fp32 accumulation
F32_TOL = 1e-5    # max-abs error, fp32 inputs


def require_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    load_library()  # raises if libst.so is missing


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


def sample_rows(wl, per_req=4, heads=3, seed=0):
    """A few nodes per request (root, last, random) and a few q-heads."""
    rng = np.random.default_rng(seed)
    nodes = []
    for b in range(wl.B):
        lo, hi = int(wl.node_off[b]), int(wl.node_off[b + 1])
        pick = {lo, hi - 1}
        while len(pick) < min(per_req, hi - lo):
            pick.add(int(rng.integers(lo, hi)))
        nodes += sorted(pick)
    hs = sorted({0, wl.Hq - 1} | {int(x) for x in rng.integers(0, wl.Hq, heads)})
    return nodes, hs


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
