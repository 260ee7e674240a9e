"""Seeded synthetic workloads shaped like the token-tree verification setups the
pages discuss (LLaMA-7B and LLaMA-2-70B attention layers, a 32000-token vocab,
trees of width 5 and depth 3, temperature 0.7).

Only random draws and bookkeeping of the tree *construction* live here; nothing
in this file evaluates a step of the verification method.

Draw order for one workload (all from one ``PCG64(seed)`` stream):
  1. per request, in request order: prefix length, tree size, parent array
  2. queries ``[T][Hq][D]``
  3. key cache ``[B][Hkv][S_max][D]`` (every slot, used or not)
  4. value cache, same shape
  5. target logits ``[T][V]``
  6. draft-logit noise ``[T][V]`` (stochastic workloads only)
  7. draft tokens ``[T]`` (rule depends on the workload)
"""

from __future__ import annotations

from dataclasses import dataclass, field
from typing import Callable, Dict, List, Optional, Sequence

import numpy as np


# ---------------------------------------------------------------------------
# value encoding


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (round to nearest, ties to even) and
    return the 16-bit patterns as uint16.  Inputs are finite."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    b = x.view(np.uint32)
    out = np.empty(x.shape, dtype=np.uint16)
    flat_b = b.reshape(-1)
    flat_o = out.reshape(-1)
    step = 1 << 24
    for s in range(0, flat_b.size, step):
        c = flat_b[s:s + step]
        r = ((c >> np.uint32(16)) & np.uint32(1)) + np.uint32(0x7FFF)
        flat_o[s:s + step] = ((c + r) >> np.uint32(16)).astype(np.uint16)
    return out


BF16_NAN = np.uint16(0x7FC0)


# ---------------------------------------------------------------------------
# tree shapes: each returns (parent, level) where parent[0] = -1 and
# parent[i] < i; ``level`` is the construction level used to honour the
# shape's depth bound.


def tree_complete_binary(n: int):
    parent = np.array([-1] + [(i - 1) // 2 for i in range(1, n)], dtype=np.int32)
    level = np.array([int(np.floor(np.log2(i + 1))) for i in range(n)], dtype=np.int32)
    return parent, level


def tree_chain(n: int):
    parent = np.arange(-1, n - 1, dtype=np.int32)
    level = np.arange(n, dtype=np.int32)
    return parent, level


def tree_random_attach(rng: np.random.Generator, n: int, max_depth: int):
    """Node i attaches to a uniformly chosen earlier node whose level is below
    ``max_depth``, so no node ends deeper than ``max_depth``."""
    parent = np.full(n, -1, dtype=np.int32)
    level = np.zeros(n, dtype=np.int32)
    open_nodes: List[int] = [0] if max_depth > 0 else []
    for i in range(1, n):
        p = open_nodes[int(rng.integers(0, len(open_nodes)))]
        parent[i] = p
        level[i] = level[p] + 1
        if level[i] < max_depth:
            open_nodes.append(i)
    return parent, level


def tree_beam_plus_leaves(rng: np.random.Generator, n: int, width: int = 5, levels: int = 3):
    """A root, then ``levels`` expansion levels of ``width`` nodes each (every
    node hangs off a uniformly chosen node of the previous level), then
    ``n - 1 - width*levels`` extra leaves hanging off uniformly chosen nodes
    above the last level."""
    base = 1 + width * levels
    assert n >= base
    parent = np.full(n, -1, dtype=np.int32)
    level = np.zeros(n, dtype=np.int32)
    prev = [0]
    idx = 1
    for lv in range(1, levels + 1):
        cur = []
        for _ in range(width):
            p = prev[int(rng.integers(0, len(prev)))]
            parent[idx] = p
            level[idx] = lv
            cur.append(idx)
            idx += 1
        prev = cur
    upper = [i for i in range(base) if level[i] < levels]
    for i in range(base, n):
        p = upper[int(rng.integers(0, len(upper)))]
        parent[i] = p
        level[i] = level[p] + 1
    return parent, level


# ---------------------------------------------------------------------------
# workload container


@dataclass
class Workload:
    name: str
    dtype: str                    # "f32" or "bf16": dtype of q / k / v
    B: int
    Hq: int
    Hkv: int
    D: int
    V: int                        # vocab (0: no acceptance step)
    node_off: np.ndarray          # int32 [B+1]
    parent: np.ndarray            # int32 [T], request-local indices, root = -1
    tokens: np.ndarray            # int32 [T]
    prefix_len: np.ndarray        # int32 [B]
    S_max: int
    q: np.ndarray                 # [T][Hq][D] float32, or uint16 bf16 patterns
    k_cache: np.ndarray           # [B][Hkv][S_max][D]
    v_cache: np.ndarray
    logits: Optional[np.ndarray]  # float32 [T][V]
    draft_logits: Optional[np.ndarray]
    temperature: float
    seed: int
    rng_seed: int                 # counter-RNG key for stochastic acceptance
    rng_offset: int
    max_depth: int                # bound on node depth guaranteed by the shape
    steps: Sequence[str] = field(default_factory=tuple)
    note: str = ""

    @property
    def T(self) -> int:
        return int(self.node_off[-1])

    @property
    def sizes(self) -> np.ndarray:
        return np.diff(self.node_off).astype(np.int32)

    @property
    def max_nodes(self) -> int:
        return int(self.sizes.max())

    @property
    def elem_bytes(self) -> int:
        return 4 if self.dtype == "f32" else 2


def _normal(rng, shape, sigma, dtype_name):
    x = rng.standard_normal(shape, dtype=np.float32)
    if sigma != 1.0:
        x *= np.float32(sigma)
    return x if dtype_name == "f32" else f32_to_bf16_bits(x)


def build_workload(
    name: str,
    rng: np.random.Generator,
    *,
    dtype: str,
    Hq: int,
    Hkv: int,
    D: int,
    V: int,
    prefix_lens: Sequence[int],
    trees: Sequence[tuple],
    max_depth: int,
    token_rule: str = "uniform",
    logit_sigma: float = 3.0,
    draft_noise_sigma: Optional[float] = None,
    temperature: float = 1.0,
    q_sigma: float = 1.0,
    kv_sigma: float = 1.0,
    poison_unused: bool = False,
    seed: int = 0,
    rng_seed: int = 0,
    rng_offset: int = 0,
    steps: Sequence[str] = (),
    note: str = "",
) -> Workload:
    """Draw the value arrays for already-drawn tree shapes.

    ``trees`` holds one ``(parent, level)`` pair per request.  Token rules:
      * ``uniform``: every draft token uniform in [0, V)
      * ``argmax_top2``: nodes on levels 1 and 2 carry the argmax of their
        parent's target logits, deeper nodes and the root are uniform
      * ``plant_leaf_path``: uniform, then one uniformly chosen leaf's root path
        is overwritten with each parent's target argmax
      * ``draft_sample``: each node's token is drawn from softmax(draft/T) of
        its parent with the Gumbel-max trick, independently per node
    """
    B = len(trees)
    assert len(prefix_lens) == B
    sizes = [len(t[0]) for t in trees]
    node_off = np.zeros(B + 1, dtype=np.int32)
    node_off[1:] = np.cumsum(sizes)
    T = int(node_off[-1])
    parent = np.concatenate([t[0] for t in trees]).astype(np.int32)
    level = np.concatenate([t[1] for t in trees]).astype(np.int32)
    prefix_len = np.asarray(prefix_lens, dtype=np.int32)
    S_max = int(max(p + n for p, n in zip(prefix_lens, sizes)))

    q = _normal(rng, (T, Hq, D), q_sigma, dtype)
    k_cache = _normal(rng, (B, Hkv, S_max, D), kv_sigma, dtype)
    v_cache = _normal(rng, (B, Hkv, S_max, D), kv_sigma, dtype)
    if poison_unused:
        bad = np.float32(np.nan) if dtype == "f32" else BF16_NAN
        for b in range(B):
            used = int(prefix_len[b]) + sizes[b]
            k_cache[b, :, used:, :] = bad
            v_cache[b, :, used:, :] = bad

    logits = draft = None
    if V > 0:
        logits = rng.standard_normal((T, V), dtype=np.float32)
        logits *= np.float32(logit_sigma)
        if draft_noise_sigma is not None:
            noise = rng.standard_normal((T, V), dtype=np.float32)
            draft = logits + noise * np.float32(draft_noise_sigma)

    tokens = np.zeros(T, dtype=np.int32)
    if V > 0:
        if token_rule == "uniform":
            tokens[:] = rng.integers(0, V, size=T)
        elif token_rule == "argmax_top2":
            tokens[:] = rng.integers(0, V, size=T)
            for b in range(B):
                o = int(node_off[b])
                for i in range(1, sizes[b]):
                    if level[o + i] in (1, 2):
                        tokens[o + i] = int(np.argmax(logits[o + parent[o + i]]))
        elif token_rule == "plant_leaf_path":
            tokens[:] = rng.integers(0, V, size=T)
            for b in range(B):
                o = int(node_off[b])
                par = parent[o:o + sizes[b]]
                has_child = np.zeros(sizes[b], dtype=bool)
                has_child[par[1:]] = True
                leaves = np.nonzero(~has_child)[0]
                leaf = int(leaves[int(rng.integers(0, len(leaves)))])
                j = leaf
                while j > 0:
                    tokens[o + j] = int(np.argmax(logits[o + par[j]]))
                    j = int(par[j])
        elif token_rule == "draft_sample":
            assert draft is not None
            for t in range(T):
                b = int(np.searchsorted(node_off, t, side="right")) - 1
                i = t - int(node_off[b])
                if i == 0:
                    tokens[t] = int(rng.integers(0, V))
                    continue
                row = draft[int(node_off[b]) + int(parent[t])].astype(np.float64) / temperature
                tokens[t] = int(np.argmax(row + rng.gumbel(size=V)))
        else:
            raise ValueError(token_rule)

    return Workload(
        name=name, dtype=dtype, B=B, Hq=Hq, Hkv=Hkv, D=D, V=V, node_off=node_off,
        parent=parent, tokens=tokens, prefix_len=prefix_len, S_max=S_max, q=q,
        k_cache=k_cache, v_cache=v_cache, logits=logits, draft_logits=draft,
        temperature=float(temperature), seed=seed, rng_seed=rng_seed,
        rng_offset=rng_offset, max_depth=max_depth, steps=tuple(steps), note=note,
    )


# ---------------------------------------------------------------------------
# the named workloads


def _tiny_fp32(seed: int, **kw) -> Workload:
    rng = np.random.default_rng(seed)
    trees = [tree_complete_binary(15)]
    return build_workload(
        "tiny_fp32", rng, dtype="f32", Hq=4, Hkv=4, D=64, V=1000, prefix_lens=[128],
        trees=trees, max_depth=3, token_rule="argmax_top2", logit_sigma=2.0, seed=seed,
        steps=("mask", "attention", "greedy", "compact"),
        note="1 request, 4 heads, D=64, prefix 128, complete binary tree of 15 nodes, fp32", **kw)


def _llama7b(seed: int, **kw) -> Workload:
    rng = np.random.default_rng(seed)
    trees = [tree_random_attach(rng, 64, 8)]
    return build_workload(
        "llama7b", rng, dtype="bf16", Hq=32, Hkv=32, D=128, V=32000, prefix_lens=[4096],
        trees=trees, max_depth=8, token_rule="uniform", logit_sigma=3.0, seed=seed,
        steps=("mask", "attention", "greedy", "compact"),
        note="LLaMA-7B-shaped layer: 32/32 heads, D=128, prefix 4096, 64-node tree, V=32000", **kw)


def _ragged(seed: int, **kw) -> Workload:
    rng = np.random.default_rng(seed)
    prefix, trees = [], []
    for _ in range(8):
        prefix.append(int(rng.integers(512, 4097)))
        n = int(rng.integers(16, 129))
        trees.append(tree_beam_plus_leaves(rng, n, 5, 3))
    return build_workload(
        "ragged_batch", rng, dtype="bf16", Hq=32, Hkv=32, D=128, V=32000, prefix_lens=prefix,
        trees=trees, max_depth=3, token_rule="plant_leaf_path", logit_sigma=3.0, seed=seed,
        steps=("mask", "attention", "greedy", "compact"),
        note="8 requests, prefixes U[512,4096], trees of 16-128 nodes (width 5, depth 3 + leaves)",
        **kw)


def _llama70b(seed: int, **kw) -> Workload:
    rng = np.random.default_rng(seed)
    trees = [tree_random_attach(rng, 64, 6) for _ in range(4)]
    return build_workload(
        "llama70b_gqa", rng, dtype="bf16", Hq=64, Hkv=8, D=128, V=0, prefix_lens=[32768] * 4,
        trees=trees, max_depth=6, seed=seed, steps=("mask", "attention"),
        note="LLaMA-2-70B-shaped GQA layer: 64 q / 8 kv heads, 4 requests, prefix 32768, 64 nodes",
        **kw)


def _stochastic(seed: int, chain: bool, **kw) -> Workload:
    rng = np.random.default_rng(seed)
    if chain:
        trees = [tree_chain(6) for _ in range(16)]
        depth = 5
    else:
        trees = [tree_random_attach(rng, 32, 8) for _ in range(16)]
        depth = 8
    return build_workload(
        "stochastic_chain" if chain else "stochastic_tree", rng, dtype="bf16", Hq=32, Hkv=32,
        D=128, V=32000, prefix_lens=[2048] * 16, trees=trees, max_depth=depth,
        token_rule="draft_sample", logit_sigma=3.0, draft_noise_sigma=1.0, temperature=0.7,
        seed=seed, rng_seed=0, rng_offset=0,
        steps=("mask", "attention", "stochastic", "compact"),
        note=("16 requests, 32 heads, prefix 2048, " + ("K=5 chains" if chain else "32-node trees")
              + ", draft = target + N(0,1), T=0.7"), **kw)


WORKLOADS: Dict[str, Callable[..., Workload]] = {
    "tiny_fp32": _tiny_fp32,
    "llama7b": _llama7b,
    "ragged_batch": _ragged,
    "llama70b_gqa": _llama70b,
    "stochastic_tree": lambda seed, **kw: _stochastic(seed, False, **kw),
    "stochastic_chain": lambda seed, **kw: _stochastic(seed, True, **kw),
}


def make_workload(name: str, seed: int = 0, **kw) -> Workload:
    return WORKLOADS[name](seed, **kw)
