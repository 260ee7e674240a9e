"""The one-call step without a workspace argument (st_verification_step_noalloc,
for callers that cannot allocate): its outputs equal st_verification_step's
on the same inputs, bit for bit, on consecutive calls whose second is smaller,
and a step that needs more than the static buffer is refused."""

import numpy as np
import pytest
import torch

from synth import build_workload, make_workload, tree_random_attach
from token_tree_verification_st_amd import binding as bd
from token_tree_verification_st_amd import to_device
from token_tree_verification_st_amd import step as stp
from tests.gpu_util import require_gpu, say

pytestmark = pytest.mark.gpu

OUTS = ("out", "lse", "accept_len", "accept_nodes", "out_tokens", "near_ties", "src_slot",
        "new_len", "status")


@pytest.fixture(autouse=True)
def _gpu():
    require_gpu()


def _noalloc(dw, stochastic):
    b = dw.buf
    bd.st_verification_step_noalloc(
        dw.tree, dw.q, dw.k_cache, dw.v_cache, dw.prefix_len, dw.max_prefix, b["out"], b["lse"],
        dw.tokens, dw.logits, b["accept_len"], b["accept_nodes"], b["out_tokens"],
        b["src_slot"], b["new_len"], draft_logits=dw.draft_logits if stochastic else None,
        temperature=dw.temperature, seed=dw.rng_seed, offset=dw.rng_offset,
        near_ties=b["near_ties"] if stochastic else None, status=b["status"])


def test_noalloc_step_equals_step_on_consecutive_calls():
    """llama7b (4 MiB of split partials in the static buffer), the ragged
    batch (39 MiB: splits sized per request, room for up to 4 a request), then
    the smaller stochastic tree batch, the fp32 tiny tree and llama7b again,
    each against the workspace entry point on a fresh copy of the same
    inputs."""
    for name in ("llama7b", "ragged_batch", "stochastic_tree", "tiny_fp32", "llama7b"):
        wl = make_workload(name, 0)
        stochastic = wl.draft_logits is not None
        ref, got = to_device(wl), to_device(wl)
        stp.run_step(ref, stochastic)
        for k in OUTS:       # outputs start from garbage, so nothing stale can pass
            if got.buf[k].dtype.is_floating_point:
                got.buf[k].fill_(float("nan"))
            elif k != "status":
                got.buf[k].fill_(-7)
        _noalloc(got, stochastic)
        torch.cuda.synchronize()
        for k in OUTS:
            if k == "near_ties" and not stochastic:
                continue
            assert torch.equal(ref.buf[k], got.buf[k]), f"{name}: {k}"
        assert torch.equal(ref.k_cache, got.k_cache) and torch.equal(ref.v_cache, got.v_cache)
        say(f"noalloc step {name}: equal to the workspace step, accept_len "
            f"{got.buf['accept_len'].tolist()[:4]}")


def test_noalloc_step_refuses_a_step_larger_than_its_buffer():
    """3 requests of 256 nodes x 64 heads (D 128): 49152 rows whose split
    partials (room for 4 splits a row) exceed the 64 MiB buffer."""
    rng = np.random.default_rng(5)
    trees = [tree_random_attach(rng, 256, 6) for _ in range(3)]
    wl = build_workload("big", rng, dtype="bf16", Hq=64, Hkv=64, D=128, V=64,
                        prefix_lens=[512] * 3, trees=trees, max_depth=255, token_rule="uniform")
    dw = to_device(wl)
    b = dw.buf
    step = bd._step_struct(dw.tree, dw.q, dw.k_cache, dw.v_cache, dw.prefix_len, dw.max_prefix,
                           b["out"], b["lse"], dw.tokens, dw.logits, None, 1.0, 0, 0,
                           b["accept_len"], b["accept_nodes"], b["out_tokens"], None,
                           b["src_slot"], b["new_len"], None)
    assert bd.st_verification_step_workspace(dw.tree, step) > 64 << 20
    with pytest.raises(RuntimeError, match="workspace"):
        _noalloc(dw, False)
