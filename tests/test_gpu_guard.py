"""Out-of-range writes: every output, workspace and in-place cache of every
entry point sits between two guard bands of sentinel bytes inside one
allocation, and every input is checked unchanged.  The header promises that
every write stays inside the documented output ranges (the caller owns the
memory; the library writes only where it is told)."""

import numpy as np
import pytest
import torch

from synth import build_workload, make_workload, tree_chain, tree_random_attach
from synth.paged import make_paged
from token_tree_verification_st_amd import binding as bd
from token_tree_verification_st_amd import to_device
from tests.gpu_util import require_gpu, say, status_of

pytestmark = pytest.mark.gpu

GUARD = 4096          # bytes on each side (keeps every view 256-byte aligned)
SENTINEL = 0xA5


@pytest.fixture(autouse=True)
def _gpu():
    require_gpu()


class Guards:
    """Guarded copies of tensors, and checks of the bands and the inputs."""

    def __init__(self):
        self.bands = []     # (name, raw allocation, payload bytes)
        self.inputs = []    # (name, guarded tensor, pristine copy)

    def wrap(self, name, t, nbytes=None):
        """A guarded tensor with t's shape, dtype and contents; with nbytes,
        a uint8 buffer of exactly that many bytes (a workspace)."""
        if nbytes is not None:
            t = torch.empty(int(nbytes), dtype=torch.uint8, device="cuda")
        n = t.numel() * t.element_size()
        raw = torch.full((GUARD + n + GUARD,), SENTINEL, dtype=torch.uint8, device="cuda")
        mid = raw[GUARD:GUARD + n].view(t.dtype).view(t.shape)
        if nbytes is None:
            mid.copy_(t)
        self.bands.append((name, raw, n))
        return mid

    def wrap_input(self, name, t):
        g = self.wrap(name, t)
        self.inputs.append((name, g, t.clone()))
        return g

    def check(self, what):
        torch.cuda.synchronize()
        for name, raw, n in self.bands:
            head, tail = raw[:GUARD], raw[GUARD + n:]
            assert bool((head == SENTINEL).all()), f"{what}: write before {name}"
            assert bool((tail == SENTINEL).all()), f"{what}: write after {name}"
        for name, g, ref in self.inputs:
            assert torch.equal(g.view(torch.uint8) if g.dtype == torch.bool else g, ref), \
                f"{what}: input {name} changed"


def _guarded_tree(G, tree):
    return bd.Tree(G.wrap_input("node_off", tree.node_off), G.wrap_input("parent", tree.parent),
                   tree.max_nodes, tree.max_depth)


def _guarded(wl):
    """The workload on the device with every tensor guarded (caches as
    outputs: compaction writes them in place)."""
    dw = to_device(wl)
    G = Guards()
    dw.tree = _guarded_tree(G, dw.tree)
    for k in ("tokens", "prefix_len", "q", "logits", "draft_logits"):
        v = getattr(dw, k)
        if v is not None:
            setattr(dw, k, G.wrap_input(k, v))
    dw.k_cache = G.wrap("k_cache", dw.k_cache)
    dw.v_cache = G.wrap("v_cache", dw.v_cache)
    for k in list(dw.buf):
        if not k.endswith("_ws"):
            dw.buf[k] = G.wrap(k, dw.buf[k])
    return dw, G


def _edges_workload(dtype):
    """A single node with no prefix, a prefix ending on a tile, a 256-node
    tree (four mask words) and a 64-chain, with a small vocabulary."""
    rng = np.random.default_rng(41)
    trees = [tree_chain(1), tree_random_attach(rng, 17, 5), tree_random_attach(rng, 256, 30),
             tree_chain(64)]
    return build_workload("edges", rng, dtype=dtype, Hq=4, Hkv=2,
                          D=128 if dtype == "bf16" else 64, V=50, prefix_lens=[0, 128, 63, 1],
                          trees=trees, max_depth=255, token_rule="plant_leaf_path",
                          logit_sigma=2.0, draft_noise_sigma=1.0, temperature=0.7)


WORKLOADS = ["tiny_fp32", "llama7b", "ragged_batch", "stochastic_tree", "stochastic_chain",
             "edges_bf16", "edges_f32"]


def _workload(name):
    return _edges_workload(name[6:]) if name.startswith("edges_") else make_workload(name, 0)


@pytest.mark.parametrize("name", WORKLOADS)
def test_separate_calls_write_only_their_outputs(name):
    wl = _workload(name)
    stochastic = wl.draft_logits is not None
    say(f"guards: separate calls on {name}")
    dw, G = _guarded(wl)
    b, t = dw.buf, dw.tree
    bd.st_tree_mask(t, b["mask"], b["depth"], b["status"])
    G.check("st_tree_mask")
    aws = G.wrap("attn_ws", None, bd.st_tree_attention_workspace(t, dw.Hq, dw.Hkv, dw.D, dw.dtype,
                                                                 dw.max_prefix))
    for mask in (b["mask"], None):
        bd.st_tree_attention(t, dw.q, dw.k_cache, dw.v_cache, dw.prefix_len, dw.max_prefix, mask,
                             b["out"], b["lse"], aws, status=b["status"])
        G.check(f"st_tree_attention (mask {'given' if mask is not None else 'derived'})")
    if stochastic:
        ws = G.wrap("verify_ws", None, bd.st_verify_stochastic_workspace(t, dw.V))
        bd.st_verify_stochastic(t, dw.tokens, dw.logits, dw.draft_logits, dw.temperature,
                                dw.rng_seed, dw.rng_offset, b["accept_len"], b["accept_nodes"],
                                b["out_tokens"], ws, b["near_ties"], b["status"])
        G.check("st_verify_stochastic")
        bd.st_verify_stochastic_ex(t, dw.tokens, dw.logits, dw.draft_logits, dw.temperature,
                                   dw.rng_seed, dw.rng_offset, b["accept_len"],
                                   b["accept_nodes"], b["out_tokens"], ws, b["near_ties"],
                                   b["status"], top_p=0.9)
        G.check("st_verify_stochastic_ex")
    else:
        ws = G.wrap("verify_ws", None, bd.st_verify_greedy_workspace(t, dw.V))
        bd.st_verify_greedy(t, dw.tokens, dw.logits, b["accept_len"], b["accept_nodes"],
                            b["out_tokens"], ws, b["status"])
        G.check("st_verify_greedy")
    k0, v0 = dw.k_cache.clone(), dw.v_cache.clone()
    bd.st_kv_compact(dw.k_cache, dw.v_cache, dw.prefix_len, b["accept_len"], b["accept_nodes"],
                     b["src_slot"], b["new_len"], b["status"])
    G.check("st_kv_compact")
    _rows_outside_paths_unchanged(dw, k0, v0)
    assert status_of(dw) & ~8 == 0    # a 64-chain may overflow max_depth on purpose


def _rows_outside_paths_unchanged(dw, k0, v0):
    """Compaction writes rows P .. P + L of each request only."""
    al = dw.buf["accept_len"].cpu().numpy()
    P = dw.prefix_len.cpu().numpy()
    S = dw.k_cache.shape[2]
    for b in range(dw.B):
        keep = torch.ones(S, dtype=torch.bool, device="cuda")
        keep[int(P[b]):int(P[b]) + int(al[b]) + 1] = False
        for c, c0 in ((dw.k_cache, k0), (dw.v_cache, v0)):
            assert torch.equal(c[b][:, keep], c0[b][:, keep]), f"request {b}: rows off the path"


def _step_ws(G, dw, stochastic, draft=None, block_table=None):
    b = dw.buf
    st = bd._step_struct(dw.tree, dw.q, dw.k_cache, dw.v_cache, dw.prefix_len, dw.max_prefix,
                         b["out"], b["lse"], dw.tokens, dw.logits,
                         (draft if draft is not None else dw.draft_logits) if stochastic else None,
                         dw.temperature, dw.rng_seed, dw.rng_offset, b["accept_len"],
                         b["accept_nodes"], b["out_tokens"], b["near_ties"], b["src_slot"],
                         b["new_len"], None, block_table=block_table)
    return G.wrap("step_ws", None, bd.st_verification_step_workspace(dw.tree, st))


@pytest.mark.parametrize("name", WORKLOADS)
def test_one_call_step_writes_only_its_outputs(name):
    wl = _workload(name)
    stochastic = wl.draft_logits is not None
    say(f"guards: one-call step on {name}")
    dw, G = _guarded(wl)
    b = dw.buf
    k0, v0 = dw.k_cache.clone(), dw.v_cache.clone()
    ws = _step_ws(G, dw, stochastic)
    bd.st_verification_step(dw.tree, dw.q, dw.k_cache, dw.v_cache, dw.prefix_len, dw.max_prefix,
                            b["out"], b["lse"], dw.tokens, dw.logits, b["accept_len"],
                            b["accept_nodes"], b["out_tokens"], b["src_slot"], b["new_len"], ws,
                            draft_logits=dw.draft_logits if stochastic else None,
                            temperature=dw.temperature, seed=dw.rng_seed, offset=dw.rng_offset,
                            near_ties=b["near_ties"] if stochastic else None, status=b["status"])
    G.check("st_verification_step")
    _rows_outside_paths_unchanged(dw, k0, v0)
    if stochastic:
        dw2, G2 = _guarded(wl)
        b2 = dw2.buf
        ws2 = _step_ws(G2, dw2, True)
        bd.st_verification_step_ex(dw2.tree, dw2.q, dw2.k_cache, dw2.v_cache, dw2.prefix_len,
                                   dw2.max_prefix, b2["out"], b2["lse"], dw2.tokens, dw2.logits,
                                   b2["accept_len"], b2["accept_nodes"], b2["out_tokens"],
                                   b2["src_slot"], b2["new_len"], ws2, dw2.draft_logits,
                                   temperature=dw2.temperature, seed=dw2.rng_seed,
                                   offset=dw2.rng_offset, near_ties=b2["near_ties"],
                                   status=b2["status"], top_p=0.9)
        G2.check("st_verification_step_ex")


def test_attention_70b_gqa_writes_only_its_outputs():
    wl = make_workload("llama70b_gqa", 0)
    dw, G = _guarded(wl)
    b, t = dw.buf, dw.tree
    aws = G.wrap("attn_ws", None, bd.st_tree_attention_workspace(t, dw.Hq, dw.Hkv, dw.D, dw.dtype,
                                                                 dw.max_prefix))
    bd.st_tree_attention(t, dw.q, dw.k_cache, dw.v_cache, dw.prefix_len, dw.max_prefix, None,
                         b["out"], b["lse"], aws, status=b["status"])
    G.check("st_tree_attention llama70b_gqa")
    assert status_of(dw) == 0


@pytest.mark.parametrize("name,bs", [("llama7b", 64), ("ragged_batch", 32), ("tiny_fp32", 32),
                                     ("stochastic_tree", 128)])
def test_paged_calls_write_only_their_outputs(name, bs):
    wl = make_workload(name, 0)
    stochastic = wl.draft_logits is not None
    say(f"guards: paged calls on {name}, block {bs}")
    kp_h, vp_h, bt_h = make_paged(3, wl.k_cache, wl.v_cache, bs)
    dt = torch.float32 if wl.dtype == "f32" else torch.bfloat16

    def pool(h):
        x = torch.from_numpy(h.view(np.int16) if wl.dtype == "bf16" else h)
        return x.cuda().view(dt) if wl.dtype == "bf16" else x.cuda()

    for leg in ("separate", "step"):
        dw, G = _guarded(wl)
        b, t = dw.buf, dw.tree
        kp, vp = G.wrap("k_pool", pool(kp_h)), G.wrap("v_pool", pool(vp_h))
        bt = G.wrap_input("block_table", torch.from_numpy(bt_h).cuda())
        if leg == "separate":
            aws = G.wrap("attn_ws", None, bd.st_tree_attention_workspace(
                t, dw.Hq, dw.Hkv, dw.D, dw.dtype, dw.max_prefix))
            bd.st_tree_attention_paged(t, dw.q, kp, vp, bt, dw.prefix_len, dw.max_prefix, None,
                                       b["out"], b["lse"], aws, status=b["status"])
            G.check("st_tree_attention_paged")
            ws = G.wrap("verify_ws", None, bd.st_verify_greedy_workspace(t, dw.V))
            bd.st_verify_greedy(t, dw.tokens, dw.logits, b["accept_len"], b["accept_nodes"],
                                b["out_tokens"], ws, b["status"])
            bd.st_kv_compact_paged(kp, vp, bt, dw.prefix_len, b["accept_len"],
                                   b["accept_nodes"], b["src_slot"], b["new_len"], b["status"])
            G.check("st_kv_compact_paged")
        else:
            st = bd._step_struct(t, dw.q, kp, vp, dw.prefix_len, dw.max_prefix, b["out"],
                                 b["lse"], dw.tokens, dw.logits,
                                 dw.draft_logits if stochastic else None, dw.temperature,
                                 dw.rng_seed, dw.rng_offset, b["accept_len"], b["accept_nodes"],
                                 b["out_tokens"], b["near_ties"], b["src_slot"], b["new_len"],
                                 None, block_table=bt)
            ws = G.wrap("step_ws", None, bd.st_verification_step_workspace(t, st))
            bd.st_verification_step_paged(t, dw.q, kp, vp, bt, dw.prefix_len, dw.max_prefix,
                                          b["out"], b["lse"], dw.tokens, dw.logits,
                                          b["accept_len"], b["accept_nodes"], b["out_tokens"],
                                          b["src_slot"], b["new_len"], ws,
                                          draft_logits=dw.draft_logits if stochastic else None,
                                          temperature=dw.temperature, seed=dw.rng_seed,
                                          offset=dw.rng_offset,
                                          near_ties=b["near_ties"] if stochastic else None,
                                          status=b["status"])
            G.check("st_verification_step_paged")
        assert status_of(dw) == 0
