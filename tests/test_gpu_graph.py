"""The benchmark replays the verification step from a captured HIP graph.  Each
replay must equal the eager result, with eager work and synchronisations between
replays (the step records no memset nodes)."""

import numpy as np
import pytest
import torch

from synth import make_workload
from token_tree_verification_st_amd import to_device
from token_tree_verification_st_amd import step as stp
from tests.gpu_util import require_gpu, say

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("name,stochastic,top_p,probs",
                         [("tiny_fp32", False, 1.0, False), ("ragged_batch", False, 1.0, False),
                          ("stochastic_chain", True, 1.0, False),
                          ("stochastic_tree", True, 0.9, True)])
def test_graph_replays_equal_eager(name, stochastic, top_p, probs):
    require_gpu()
    wl = make_workload(name, 0)
    dw = to_device(wl)
    draft = None
    if probs:   # the draft as probabilities (one-call step with the sampling options)
        z = wl.draft_logits.astype(np.float64) / wl.temperature
        pr = np.exp(z - z.max(axis=1, keepdims=True))
        draft = torch.from_numpy((pr / pr.sum(axis=1, keepdims=True)).astype(np.float32)).cuda()
    opts = dict(stochastic=stochastic, top_p=top_p, draft=draft)
    k0, v0 = dw.k_cache.clone(), dw.v_cache.clone()
    keys = ["mask", "depth", "out", "lse", "accept_len", "accept_nodes", "out_tokens", "src_slot",
            "new_len"]
    stp.verification_step(dw, **opts)
    torch.cuda.synchronize()
    eager = {k: dw.buf[k].clone() for k in keys}
    k_eager, v_eager = dw.k_cache.clone(), dw.v_cache.clone()

    g = torch.cuda.CUDAGraph()
    dw.k_cache.copy_(k0)
    dw.v_cache.copy_(v0)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        stp.verification_step(dw, **opts)
    for rep in range(4):
        for k in keys:                      # eager work between replays
            dw.buf[k].zero_()
        dw.k_cache.copy_(k0)
        dw.v_cache.copy_(v0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for k in keys:
            assert torch.equal(dw.buf[k], eager[k]), f"replay {rep}: {k} differs"
        assert torch.equal(dw.k_cache, k_eager) and torch.equal(dw.v_cache, v_eager)
        _ = (dw.buf["out"].float() * 2).sum().item()   # unrelated eager kernels
    assert int(dw.buf["status"].item()) == 0
    say(f"{name} top_p={top_p} probs={probs}: 4 graph replays equal the eager step")


def test_stream_read_helper():
    """The read-ceiling helper runs over any 16-byte multiple, leaves its sink
    alone on ordinary data, and refuses a size that is not a multiple of 16."""
    import ctypes
    from token_tree_verification_st_amd import load_library, st_stream_read
    require_gpu()
    for n in (4, 1000, 1 << 22, (1 << 24) + 12):
        src = torch.ones(n, dtype=torch.int32, device="cuda")
        sink = torch.zeros(64, dtype=torch.int32, device="cuda")
        st_stream_read(src, sink)
        torch.cuda.synchronize()
        assert int(sink.abs().sum().item()) == 0
    src = torch.ones(10, dtype=torch.int32, device="cuda")
    rc = load_library().st_stream_read(ctypes.c_void_p(src.data_ptr()), 40, ctypes.c_void_p(
        sink.data_ptr()), 64, None)
    assert rc == -1
