"""GPU parity: ancestor mask (bit-exact) and tree attention (max-abs error) of the
HIP path against the oracle, through the C ABI."""


import numpy as np
import pytest
import torch

import oracle
from synth import (build_workload, make_workload, tree_beam_plus_leaves, tree_chain,
                   tree_complete_binary, tree_random_attach)
from token_tree_verification_st_amd import to_device
from tests.gpu_util import BF16_TOL, F32_TOL, attention_errors, gpu_mask, plan_override, \
    require_gpu, \
    say, status_of

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _gpu():
    require_gpu()


# ---------------------------------------------------------------- mask


@pytest.mark.parametrize("name", ["tiny_fp32", "llama7b", "ragged_batch", "stochastic_tree",
                                  "stochastic_chain"])
def test_mask_named_workloads(name):
    wl = make_workload(name, 0)
    dw = to_device(wl)
    mask, depth = gpu_mask(dw)
    ref, ref_depth = oracle.tree_mask(wl.node_off, wl.parent, dw.tree.W)
    assert np.array_equal(mask, ref)
    assert np.array_equal(depth, ref_depth)
    assert status_of(dw) == 0


def test_mask_random_trees_all_word_counts():
    rng = np.random.default_rng(1)
    trees, sizes = [], [1, 2, 63, 64, 65, 127, 128, 129, 200, 256]
    for n in sizes:
        trees.append(tree_random_attach(rng, n, int(rng.integers(1, 40))))
    trees.append(tree_chain(256))
    trees.append(tree_complete_binary(255))
    wl = build_workload("masks", rng, dtype="bf16", Hq=1, Hkv=1, D=64, V=0,
                        prefix_lens=[0] * len(trees), trees=trees, max_depth=255)
    dw = to_device(wl)
    mask, depth = gpu_mask(dw)
    ref, ref_depth = oracle.tree_mask(wl.node_off, wl.parent, 4)
    assert dw.tree.W == 4
    assert np.array_equal(mask, ref) and np.array_equal(depth, ref_depth)


def test_mask_bad_parent_sets_status():
    rng = np.random.default_rng(2)
    wl = build_workload("bad", rng, dtype="bf16", Hq=1, Hkv=1, D=64, V=0, prefix_lens=[0, 0],
                        trees=[tree_chain(5), tree_chain(4)], max_depth=4)
    wl.parent[3] = 3          # request 0, node 3 points at itself
    dw = to_device(wl)
    gpu_mask(dw)
    assert status_of(dw) & 1


# ---------------------------------------------------------------- attention


def test_attention_tiny_fp32_full():
    wl = make_workload("tiny_fp32", 0)
    err, lerr = attention_errors(wl, to_device(wl))
    say(f"tiny_fp32 max-abs {err:.2e} lse {lerr:.2e}")
    assert err <= F32_TOL and lerr <= F32_TOL


def _small_case(seed, dtype="bf16", D=128, Hq=4, Hkv=4, B=3, pmax=700, nmax=90, q_sigma=1.0,
                poison=False):
    rng = np.random.default_rng(seed)
    prefix = [int(rng.integers(0, pmax)) for _ in range(B)]
    trees = [tree_random_attach(rng, int(rng.integers(1, nmax + 1)), 7) for _ in range(B)]
    return build_workload(f"small{seed}", rng, dtype=dtype, Hq=Hq, Hkv=Hkv, D=D, V=0,
                          prefix_lens=prefix, trees=trees, max_depth=7, q_sigma=q_sigma,
                          poison_unused=poison)


@pytest.mark.parametrize("seed,D,Hq,Hkv", [(1, 128, 4, 4), (2, 64, 4, 4), (3, 128, 8, 2),
                                           (4, 64, 6, 3), (5, 128, 16, 1)])
def test_attention_bf16_small_full(seed, D, Hq, Hkv):
    wl = _small_case(seed, D=D, Hq=Hq, Hkv=Hkv)
    err, lerr = attention_errors(wl, to_device(wl))
    say(f"seed {seed} D {D} Hq {Hq} Hkv {Hkv}: max-abs {err:.2e} lse {lerr:.2e}")
    assert err <= BF16_TOL and lerr <= 1e-3


@pytest.mark.parametrize("split_keys", [64, 128, 320])
def test_attention_forced_splits_and_combine(split_keys):
    for dtype in ("bf16", "f32"):
        wl = _small_case(10 + split_keys, dtype=dtype, D=64 if dtype == "f32" else 128)
        with plan_override(attn_split_keys=split_keys):
            err, lerr = attention_errors(wl, to_device(wl))
        say(f"split {split_keys} {dtype}: max-abs {err:.2e} lse {lerr:.2e}")
        tol = F32_TOL if dtype == "f32" else BF16_TOL
        assert err <= tol and lerr <= (F32_TOL if dtype == "f32" else 1e-3)


# bf16 kernel variants by plan shape: (64-row groups per workgroup, 16-row
# blocks per wavefront) = (1,1) (1,2) (1,4) (2,4) (4,4) for shapes 0..4, then two
# workgroups per CU: (2,2) (4,2) for shapes 5, 6
@pytest.mark.parametrize("derive", [False, True])
@pytest.mark.parametrize("shape", [0, 1, 2, 3, 4, 5, 6])
def test_attention_every_kernel_shape(shape, derive):
    """derive: no mask is passed, the kernel builds it from the parent array."""
    for i, (D, Hq, Hkv, nmax) in enumerate([(128, 4, 4, 90), (64, 6, 3, 40), (128, 16, 2, 25)]):
        wl = _small_case(70 + i, D=D, Hq=Hq, Hkv=Hkv, nmax=nmax)
        with plan_override(attn_shape=shape):
            err, lerr = attention_errors(wl, to_device(wl), derive_mask=derive)
        say(f"shape {shape} D {D} Hq {Hq} Hkv {Hkv}: max-abs {err:.2e} lse {lerr:.2e}")
        assert err <= BF16_TOL and lerr <= 1e-3
    # forced short splits: some key groups get no chunk, tails are partial chunks
    wl = _small_case(79, D=128, Hq=8, Hkv=2, nmax=70)
    with plan_override(attn_shape=shape, attn_split_keys=80):
        err, lerr = attention_errors(wl, to_device(wl), derive_mask=derive)
    say(f"shape {shape} split 80: max-abs {err:.2e} lse {lerr:.2e}")
    assert err <= BF16_TOL and lerr <= 1e-3


def test_attention_derived_mask_fp32_and_edges():
    """The in-kernel ancestor masks on the fp32 path and on the edge trees:
    a single node with no prefix, a 256-node tree (four mask words), a chain."""
    wl = make_workload("tiny_fp32", 0)
    err, lerr = attention_errors(wl, to_device(wl), derive_mask=True)
    assert err <= F32_TOL and lerr <= F32_TOL
    wl = _small_case(33, dtype="f32", D=64)
    err, _ = attention_errors(wl, to_device(wl), derive_mask=True)
    assert err <= F32_TOL
    rng = np.random.default_rng(42)
    trees = [tree_chain(1), tree_random_attach(rng, 17, 5), tree_random_attach(rng, 256, 30),
             tree_chain(64), tree_chain(256)]
    for dtype in ("bf16", "f32"):
        wl = build_workload("edges_d", rng, dtype=dtype, Hq=4, Hkv=2, D=128 if dtype == "bf16" else 64,
                            V=0, prefix_lens=[0, 128, 63, 1, 40], trees=trees, max_depth=255)
        dw = to_device(wl)
        err, lerr = attention_errors(wl, dw, derive_mask=True)
        say(f"derived edges {dtype}: max-abs {err:.2e} lse {lerr:.2e}")
        assert err <= (BF16_TOL if dtype == "bf16" else F32_TOL) and status_of(dw) == 0


def test_attention_derived_mask_bad_parent_sets_status():
    from token_tree_verification_st_amd import step
    for dtype in ("bf16", "f32"):
        rng = np.random.default_rng(3)
        wl = build_workload("badp", rng, dtype=dtype, Hq=2, Hkv=2, D=64, V=0, prefix_lens=[5, 7],
                            trees=[tree_chain(6), tree_chain(9)], max_depth=8)
        wl.parent[wl.node_off[1] + 4] = 6   # request 1, node 4 points forward
        dw = to_device(wl)
        step.run_attention(dw, derive_mask=True)
        torch.cuda.synchronize()
        assert status_of(dw) & 1


def test_attention_workspace_reused_across_calls():
    """One workspace serves calls with different trees and split counts."""
    ws = torch.empty(64 << 20, dtype=torch.uint8, device="cuda")
    for i, sk in enumerate([96, 64, 200, 96]):
        wl = _small_case(90 + i, D=128, Hq=4, Hkv=2, nmax=60)
        dw = to_device(wl)
        dw.buf["attn_ws"] = ws
        for _ in range(2):
            with plan_override(attn_split_keys=sk):
                err, lerr = attention_errors(wl, dw)
            assert err <= BF16_TOL and lerr <= 1e-3
        assert status_of(dw) == 0


# Split plans for batches: one split size for all requests (1), or splits sized
# per request on the device (2, the planner's choice for 2..64 requests), with
# the planner's workgroup target, a small one (many splits, up to the cap) and
# a large one; the batches mix long and short requests.
@pytest.mark.parametrize("target", [0, 24, 4096])
@pytest.mark.parametrize("balance", [1, 2])
def test_attention_split_plans(balance, target):
    cases = [(128, 4, 4, 5, 1500, 90), (64, 8, 2, 9, 900, 40), (128, 16, 2, 3, 2000, 25),
             (128, 4, 4, 1, 1200, 60)]
    for i, (D, Hq, Hkv, B, pmax, nmax) in enumerate(cases):
        wl = _small_case(90 + i, D=D, Hq=Hq, Hkv=Hkv, B=B, pmax=pmax, nmax=nmax)
        with plan_override(attn_balance=balance, attn_target_wg=target):
            err, lerr = attention_errors(wl, to_device(wl), derive_mask=i % 2 == 1)
        say(f"balance {balance} target {target} case {i} (B {B}, prefixes "
            f"{wl.prefix_len.tolist()}): max-abs {err:.2e} lse {lerr:.2e}")
        assert err <= BF16_TOL and lerr <= 1e-3


@pytest.mark.parametrize("B", [64, 65])
def test_attention_split_plans_batch_limits(B):
    """64 requests (every lane of the device plan holds one) and 65 (one split
    size for the batch), mixed lengths, few heads so that splits happen."""
    wl = _small_case(300 + B, D=64, Hq=2, Hkv=1, B=B, pmax=1200, nmax=20)
    err, lerr = attention_errors(wl, to_device(wl), derive_mask=True)
    say(f"B {B}: max-abs {err:.2e} lse {lerr:.2e}")
    assert err <= BF16_TOL and lerr <= 1e-3


def test_attention_split_plans_agree():
    """The two split plans of one ragged batch give outputs within the bf16
    rounding of each other, and both set the bad-prefix status for a request
    whose prefix exceeds max_prefix."""
    from token_tree_verification_st_amd import step
    wl = _small_case(97, B=6, pmax=1800, nmax=70)
    outs = []
    for balance in (1, 2):
        with plan_override(attn_balance=balance, attn_target_wg=40):
            dw = to_device(wl)
            step.run_mask(dw)
            step.run_attention(dw)
            torch.cuda.synchronize()
            assert status_of(dw) == 0
            outs.append(dw.buf["out"].float().cpu())
            bad = to_device(wl, max_prefix=int(wl.prefix_len.max()) - 1)
            step.run_mask(bad)
            step.run_attention(bad)
            torch.cuda.synchronize()
            assert status_of(bad) & 16
    diff = float((outs[0] - outs[1]).abs().max())
    say(f"uniform vs per-request splits: max-abs {diff:.2e}")
    assert diff <= 2 * BF16_TOL


def test_attention_peaked_softmax_exercises_rescaling():
    wl = _small_case(21, q_sigma=8.0, pmax=1500)
    err, lerr = attention_errors(wl, to_device(wl))
    say(f"peaked: max-abs {err:.2e} lse {lerr:.2e}")
    assert err <= BF16_TOL


def test_attention_never_reads_unused_slots():
    for dtype in ("bf16", "f32"):
        wl = _small_case(31, dtype=dtype, D=128 if dtype == "bf16" else 64, poison=True)
        err, _ = attention_errors(wl, to_device(wl))
        assert err <= (BF16_TOL if dtype == "bf16" else F32_TOL)


def test_attention_edge_sizes():
    rng = np.random.default_rng(41)
    # single node and empty prefix; prefix that ends exactly on a tile; 256-node tree
    trees = [tree_chain(1), tree_random_attach(rng, 17, 5), tree_random_attach(rng, 256, 30),
             tree_chain(64)]
    wl = build_workload("edges", rng, dtype="bf16", Hq=4, Hkv=2, D=128, V=0,
                        prefix_lens=[0, 128, 63, 1], trees=trees, max_depth=255)
    err, lerr = attention_errors(wl, to_device(wl))
    say(f"edges: max-abs {err:.2e} lse {lerr:.2e}")
    assert err <= BF16_TOL and lerr <= 1e-3


def test_attention_bad_prefix_sets_status():
    wl = _small_case(51)
    dw = to_device(wl, max_prefix=int(wl.prefix_len.max()) - 1)
    from token_tree_verification_st_amd import step
    step.run_mask(dw)
    step.run_attention(dw)
    torch.cuda.synchronize()
    assert status_of(dw) & 16


@pytest.mark.parametrize("name", ["llama7b", "ragged_batch", "llama70b_gqa", "stochastic_tree",
                                  "stochastic_chain"])
def test_attention_full_size_every_row(name):
    """Every (node, q-head) of the named workloads at full size, in the launch
    configuration the benchmark times, against the oracle."""
    wl = make_workload(name, 0)
    err, lerr = attention_errors(wl, to_device(wl),
                                 derive_mask=name in ("llama7b", "stochastic_tree"))
    say(f"{name}: all {wl.T} nodes x {wl.Hq} heads, max-abs {err:.2e} lse {lerr:.2e}")
    assert err <= BF16_TOL and lerr <= 1e-3


def test_attention_host_errors():
    from token_tree_verification_st_amd import binding
    wl = _small_case(61)
    dw = to_device(wl)
    lib = binding.load_library()
    # unsupported head size
    assert lib.st_tree_attention_workspace(dw.tree.ref, 4, 4, 96, 1, 100) == 0
    q96 = torch.zeros(dw.T, 4, 96, dtype=torch.bfloat16, device="cuda")
    rc = lib.st_tree_attention(dw.tree.ref, 4, 4, 96, 1, 0.1, q96.data_ptr(),
                               dw.k_cache.data_ptr(), dw.v_cache.data_ptr(), dw.S_max,
                               dw.prefix_len.data_ptr(), dw.max_prefix, dw.buf["mask"].data_ptr(),
                               q96.data_ptr(), None, None, 0, None, None)
    assert rc == -2
    need = lib.st_tree_attention_workspace(dw.tree.ref, 4, 4, 128, 1, dw.max_prefix)
    if need:
        rc = lib.st_tree_attention(dw.tree.ref, 4, 4, 128, 1, 0.1, dw.q.data_ptr(),
                                   dw.k_cache.data_ptr(), dw.v_cache.data_ptr(), dw.S_max,
                                   dw.prefix_len.data_ptr(), dw.max_prefix,
                                   dw.buf["mask"].data_ptr(), dw.buf["out"].data_ptr(), None,
                                   dw.buf["attn_ws"].data_ptr(), need - 1, None, None)
        assert rc == -3


@pytest.mark.parametrize("shape", [-1, 0, 1, 2, 5, 6])
@pytest.mark.parametrize("D", [128, 64])
def test_attention_first_chunk_before_sizes(shape, D):
    """One split size for the batch (the plan under which each wavefront's
    first chunk is loaded before the request sizes arrive), 64-key splits: a
    short request has a split whose second key group's first chunk straddles
    its key end (loaded again, clamped) and splits past its keys (their
    workgroups leave early), over cache slots past every request's keys that
    hold NaN.  Every row matches the oracle."""
    rng = np.random.default_rng(77 + D)
    trees = [tree_random_attach(rng, 20, 6), tree_random_attach(rng, 40, 8),
             tree_chain(9)]
    wl = build_workload("early_chunk", rng, dtype="bf16", Hq=4, Hkv=2, D=D, V=0,
                        prefix_lens=[100, 3000, 1703], trees=trees, max_depth=39,
                        poison_unused=True)
    with plan_override(attn_balance=1, attn_split_keys=64, attn_shape=shape):
        err, lerr = attention_errors(wl, to_device(wl))
    say(f"shape {shape} D {D}: max-abs {err:.2e} lse {lerr:.2e}")
    assert err <= BF16_TOL and lerr <= 1e-3
