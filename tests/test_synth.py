"""The seeded input generator: determinism and the documented shapes."""

import numpy as np
import pytest

import oracle
from synth import WORKLOADS, make_workload


@pytest.mark.parametrize("name", ["tiny_fp32", "llama7b", "ragged_batch", "stochastic_chain"])
def test_seeded_and_deterministic(name):
    a, b = make_workload(name, 0), make_workload(name, 0)
    for f in ("parent", "tokens", "q", "node_off", "prefix_len"):
        assert np.array_equal(getattr(a, f), getattr(b, f))
    c = make_workload(name, 1)
    assert not np.array_equal(a.q, c.q)


def test_documented_shapes():
    wl = make_workload("llama7b")
    assert (wl.B, wl.Hq, wl.Hkv, wl.D, wl.V, wl.T) == (1, 32, 32, 128, 32000, 64)
    assert wl.q.dtype == np.uint16 and wl.k_cache.shape == (1, 32, 4096 + 64, 128)
    wl = make_workload("ragged_batch")
    assert wl.B == 8 and all(512 <= p <= 4096 for p in wl.prefix_len)
    assert all(16 <= n <= 128 for n in wl.sizes)
    assert oracle.check_tree(wl.node_off, wl.parent) == 0
    wl = make_workload("stochastic_tree")
    assert wl.B == 16 and wl.T == 512 and wl.temperature == 0.7
    assert set(WORKLOADS) == {"tiny_fp32", "llama7b", "ragged_batch", "llama70b_gqa",
                              "stochastic_tree", "stochastic_chain"}
