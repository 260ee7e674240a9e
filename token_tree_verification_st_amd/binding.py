"""Thin ctypes binding of libst.so.

Each ``st_*`` function has the name of the C entry point it calls and only
marshals arguments: torch tensors become device pointers, the stream is
torch's current stream, and a negative return code raises.  Every step of the
verification path runs in the library's HIP kernels; there is no fallback.
"""

from __future__ import annotations

import ctypes
import math
import os
from dataclasses import dataclass
from typing import Optional

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libst.so")

ST_F32, ST_BF16 = 0, 1
ST_MAX_NODES = 256
STATUS_BITS = {1: "bad parent", 2: "bad token", 4: "non-finite logit", 8: "path overflow",
               16: "bad prefix length", 32: "block-table entry out of range"}


class StTree(ctypes.Structure):
    _fields_ = [
        ("B", ctypes.c_int32),
        ("total_nodes", ctypes.c_int32),
        ("max_nodes", ctypes.c_int32),
        ("max_depth", ctypes.c_int32),
        ("node_off", ctypes.c_void_p),
        ("parent", ctypes.c_void_p),
    ]


class StStep(ctypes.Structure):
    """Mirror of st_step (include/st.h), field for field."""
    _fields_ = [
        ("Hq", ctypes.c_int32), ("Hkv", ctypes.c_int32), ("D", ctypes.c_int32),
        ("dtype", ctypes.c_int), ("scale", ctypes.c_float),
        ("q", ctypes.c_void_p), ("k_cache", ctypes.c_void_p), ("v_cache", ctypes.c_void_p),
        ("S_max", ctypes.c_int32), ("prefix_len", ctypes.c_void_p), ("max_prefix", ctypes.c_int32),
        ("out", ctypes.c_void_p), ("lse", ctypes.c_void_p),
        ("V", ctypes.c_int32), ("tokens", ctypes.c_void_p), ("logits", ctypes.c_void_p),
        ("draft_logits", ctypes.c_void_p), ("temperature", ctypes.c_float),
        ("seed", ctypes.c_uint64), ("offset", ctypes.c_uint64),
        ("accept_len", ctypes.c_void_p), ("accept_nodes", ctypes.c_void_p),
        ("out_tokens", ctypes.c_void_p), ("near_ties", ctypes.c_void_p),
        ("src_slot", ctypes.c_void_p), ("new_len", ctypes.c_void_p),
    ]


class StTestingPlan(ctypes.Structure):
    """Mirror of st_testing_plan (include/st_testing.h)."""
    _fields_ = [("attn_shape", ctypes.c_int32), ("attn_target_wg", ctypes.c_int32),
                ("attn_split_keys", ctypes.c_int32), ("linear_ksplit", ctypes.c_int32),
                ("linear_stages", ctypes.c_int32), ("attn_balance", ctypes.c_int32),
                ("step_serial", ctypes.c_int32)]


_lib = None
_c = ctypes


def _declare(lib):
    P = _c.c_void_p
    I = _c.c_int
    S = _c.c_size_t
    TP = _c.POINTER(StTree)
    sig = {
        "st_mask_words": (I, [I]),
        "st_tree_mask": (I, [TP, P, P, P, P]),
        "st_tree_attention_workspace": (S, [TP, I, I, I, I, I]),
        "st_tree_attention": (I, [TP, I, I, I, I, _c.c_float, P, P, P, I, P, I, P, P, P, P, S, P,
                                  P]),
        "st_verify_greedy_workspace": (S, [TP, I]),
        "st_verify_greedy": (I, [TP, I, P, P, P, P, P, P, S, P, P]),
        "st_verify_stochastic_workspace": (S, [TP, I]),
        "st_verify_stochastic": (I, [TP, I, P, P, P, _c.c_float, _c.c_uint64, _c.c_uint64, P, P,
                                     P, P, P, S, P, P]),
        "st_verify_stochastic_ex": (I, [TP, I, P, P, P, I, _c.c_float, _c.c_float, _c.c_uint64,
                                        _c.c_uint64, P, P, P, P, P, S, P, P]),
        "st_kv_compact": (I, [I, I, I, I, P, P, I, P, P, P, I, P, P, P, P]),
        "st_status_str": (_c.c_char_p, [I]),
        "st_verification_step_workspace": (S, [TP, _c.POINTER(StStep)]),
        "st_verification_step": (I, [TP, _c.POINTER(StStep), P, S, P, P]),
        "st_embed": (I, [I, I, I, P, P, P, P, P]),
        "st_tree_rope_append": (I, [TP, I, I, I, _c.c_float, P, P, I, I, P, P, P, P, P]),
        "st_linear_workspace": (S, [I, I, I]),
        "st_linear": (I, [I, I, I, P, P, P, P, I, P, S, P]),
        "st_tree_build": (I, [I, I, I, I, I, P, P, P, P, P, P, P, P, P, P, P, P]),
        "st_tree_attention_paged": (I, [TP, I, I, I, I, _c.c_float, P, P, P, I, I, P, I, P, I, P,
                                        P, P, P, S, P, P]),
        "st_kv_compact_paged": (I, [I, I, I, I, P, P, I, I, P, I, P, P, P, I, P, P, P, P]),
        "st_stream_read": (I, [P, S, P, I, P]),
        "st_verification_step_paged": (I, [TP, _c.POINTER(StStep), I, I, P, I, P, S, P, P]),
        "st_verification_step_ex": (I, [TP, _c.POINTER(StStep), I, _c.c_float, P, S, P, P]),
        "st_testing_set_plan": (I, [_c.POINTER(StTestingPlan)]),
        "st_verification_step_noalloc": (I, [TP, _c.POINTER(StStep), P, P]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    return lib


def load_library(path: str = LIB_PATH):
    """Load libst.so; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(path):
            raise RuntimeError(
                f"{path} is missing: build it with `python -m token_tree_verification_st_amd.build`")
        _lib = _declare(ctypes.CDLL(path))
    return _lib


def _check(rc: int, what: str):
    if rc != 0:
        msg = load_library().st_status_str(rc).decode()
        raise RuntimeError(f"{what} failed: {msg} ({rc})")


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _dev(t: torch.Tensor, name: str, dtype=None, numel=None):
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if numel is not None and t.numel() < numel:
        raise ValueError(f"{name} holds {t.numel()} elements, needs {numel}")
    return t


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def decode_status(word: int) -> list:
    return [txt for bit, txt in STATUS_BITS.items() if word & bit]


@dataclass
class Tree:
    """A batch of token trees on the device (request-local parent indices)."""

    node_off: torch.Tensor    # int32 [B+1]
    parent: torch.Tensor      # int32 [T]
    max_nodes: int
    max_depth: int

    def __post_init__(self):
        _dev(self.node_off, "node_off", torch.int32)
        _dev(self.parent, "parent", torch.int32)
        if not (1 <= self.max_nodes <= ST_MAX_NODES):
            raise ValueError(f"max_nodes must be in [1, {ST_MAX_NODES}]")
        self.B = self.node_off.numel() - 1
        self.T = self.parent.numel()
        self.c = StTree(self.B, self.T, self.max_nodes, self.max_depth,
                        self.node_off.data_ptr(), self.parent.data_ptr())

    @property
    def ref(self):
        return ctypes.byref(self.c)

    @property
    def W(self) -> int:
        return (self.max_nodes + 63) // 64


def st_mask_words(max_nodes: int) -> int:
    return load_library().st_mask_words(max_nodes)


def st_tree_mask(tree: Tree, mask: torch.Tensor, depth: torch.Tensor, status=None):
    _dev(mask, "mask", torch.int64, tree.T * tree.W)
    _dev(depth, "depth", torch.int32, tree.T)
    _check(load_library().st_tree_mask(tree.ref, _ptr(mask), _ptr(depth), _ptr(status),
                                       _stream()), "st_tree_mask")


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return ST_F32
    if t.dtype == torch.bfloat16:
        return ST_BF16
    raise ValueError(f"unsupported dtype {t.dtype}")


def st_tree_attention_workspace(tree: Tree, Hq: int, Hkv: int, D: int, dtype: torch.dtype,
                                max_prefix: int) -> int:
    code = ST_F32 if dtype == torch.float32 else ST_BF16
    return load_library().st_tree_attention_workspace(tree.ref, Hq, Hkv, D, code, max_prefix)


def st_tree_attention(tree: Tree, q, k_cache, v_cache, prefix_len, max_prefix: int, mask, out,
                      lse=None, workspace=None, scale: Optional[float] = None, status=None):
    """q [T][Hq][D]; caches [B][Hkv][S_max][D]; out like q; lse fp32 [T][Hq] or None;
    mask [T*W] int64 from st_tree_mask, or None to derive the masks from the tree."""
    T, Hq, D = q.shape
    B, Hkv, S_max, D2 = k_cache.shape
    if D2 != D or tuple(v_cache.shape) != tuple(k_cache.shape) or T != tree.T or B != tree.B:
        raise ValueError("shape mismatch between q, caches and tree")
    for name, t in (("q", q), ("k_cache", k_cache), ("v_cache", v_cache), ("out", out)):
        _dev(t, name, q.dtype)
    if out.shape != q.shape:
        raise ValueError("out must have q's shape")
    _dev(prefix_len, "prefix_len", torch.int32, B)
    if mask is not None:
        _dev(mask, "mask", torch.int64, tree.T * tree.W)
    if lse is not None:
        _dev(lse, "lse", torch.float32, T * Hq)
    need = st_tree_attention_workspace(tree, Hq, Hkv, D, q.dtype, max_prefix)
    if need and (workspace is None or workspace.numel() * workspace.element_size() < need):
        raise ValueError(f"workspace needs {need} bytes")
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    scale = 1.0 / math.sqrt(D) if scale is None else float(scale)
    _check(load_library().st_tree_attention(
        tree.ref, Hq, Hkv, D, _dtype_code(q), scale, _ptr(q), _ptr(k_cache), _ptr(v_cache), S_max,
        _ptr(prefix_len), max_prefix, _ptr(mask), _ptr(out), _ptr(lse), _ptr(workspace), ws_bytes,
        _ptr(status), _stream()), "st_tree_attention")


def st_tree_attention_paged(tree: Tree, q, k_pool, v_pool, block_table, prefix_len,
                            max_prefix: int, mask, out, lse=None, workspace=None,
                            scale: Optional[float] = None, status=None):
    """Tree attention over a paged pool: k_pool / v_pool [n_blocks][Hkv][block][D],
    block_table int32 [B][max_blocks]; other arguments as st_tree_attention."""
    T, Hq, D = q.shape
    n_blocks, Hkv, bs, D2 = k_pool.shape
    B, max_blocks = block_table.shape
    if D2 != D or tuple(v_pool.shape) != tuple(k_pool.shape) or T != tree.T or B != tree.B:
        raise ValueError("shape mismatch between q, pools, block table and tree")
    for name, t in (("q", q), ("k_pool", k_pool), ("v_pool", v_pool), ("out", out)):
        _dev(t, name, q.dtype)
    if out.shape != q.shape:
        raise ValueError("out must have q's shape")
    _dev(block_table, "block_table", torch.int32)
    _dev(prefix_len, "prefix_len", torch.int32, B)
    if mask is not None:
        _dev(mask, "mask", torch.int64, tree.T * tree.W)
    if lse is not None:
        _dev(lse, "lse", torch.float32, T * Hq)
    need = st_tree_attention_workspace(tree, Hq, Hkv, D, q.dtype, max_prefix)
    if need and (workspace is None or workspace.numel() * workspace.element_size() < need):
        raise ValueError(f"workspace needs {need} bytes")
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    scale = 1.0 / math.sqrt(D) if scale is None else float(scale)
    _check(load_library().st_tree_attention_paged(
        tree.ref, Hq, Hkv, D, _dtype_code(q), scale, _ptr(q), _ptr(k_pool), _ptr(v_pool),
        n_blocks, bs, _ptr(block_table), max_blocks, _ptr(prefix_len), max_prefix, _ptr(mask),
        _ptr(out), _ptr(lse), _ptr(workspace), ws_bytes, _ptr(status), _stream()),
        "st_tree_attention_paged")


def st_verify_greedy_workspace(tree: Tree, V: int) -> int:
    return load_library().st_verify_greedy_workspace(tree.ref, V)


def _path_outputs(tree: Tree, accept_len, accept_nodes, out_tokens):
    _dev(accept_len, "accept_len", torch.int32, tree.B)
    _dev(accept_nodes, "accept_nodes", torch.int32, tree.B * (tree.max_depth + 1))
    _dev(out_tokens, "out_tokens", torch.int32, tree.B * (tree.max_depth + 2))


def st_verify_greedy(tree: Tree, tokens, logits, accept_len, accept_nodes, out_tokens,
                     workspace, status=None):
    T, V = logits.shape
    _dev(tokens, "tokens", torch.int32, tree.T)
    _dev(logits, "logits", torch.float32)
    _path_outputs(tree, accept_len, accept_nodes, out_tokens)
    ws_bytes = workspace.numel() * workspace.element_size()
    _check(load_library().st_verify_greedy(
        tree.ref, V, _ptr(tokens), _ptr(logits), _ptr(accept_len), _ptr(accept_nodes),
        _ptr(out_tokens), _ptr(workspace), ws_bytes, _ptr(status), _stream()), "st_verify_greedy")


def st_verify_stochastic_workspace(tree: Tree, V: int) -> int:
    return load_library().st_verify_stochastic_workspace(tree.ref, V)


def st_verify_stochastic(tree: Tree, tokens, target_logits, draft_logits, temperature: float,
                         seed: int, offset: int, accept_len, accept_nodes, out_tokens, workspace,
                         near_ties=None, status=None):
    T, V = target_logits.shape
    _dev(tokens, "tokens", torch.int32, tree.T)
    _dev(target_logits, "target_logits", torch.float32)
    _dev(draft_logits, "draft_logits", torch.float32)
    if draft_logits.shape != target_logits.shape:
        raise ValueError("draft_logits must match target_logits")
    _path_outputs(tree, accept_len, accept_nodes, out_tokens)
    if near_ties is not None:
        _dev(near_ties, "near_ties", torch.int32, tree.B)
    ws_bytes = workspace.numel() * workspace.element_size()
    _check(load_library().st_verify_stochastic(
        tree.ref, V, _ptr(tokens), _ptr(target_logits), _ptr(draft_logits), float(temperature),
        int(seed), int(offset), _ptr(accept_len), _ptr(accept_nodes), _ptr(out_tokens),
        _ptr(near_ties), _ptr(workspace), ws_bytes, _ptr(status), _stream()),
        "st_verify_stochastic")


def st_verify_stochastic_ex(tree: Tree, tokens, target_logits, draft, temperature: float,
                            seed: int, offset: int, accept_len, accept_nodes, out_tokens,
                            workspace, near_ties=None, status=None, top_p: float = 1.0,
                            draft_is_probs: bool = False):
    """st_verify_stochastic with nucleus sampling (top_p < 1) and/or the draft
    given as probabilities."""
    T, V = target_logits.shape
    _dev(tokens, "tokens", torch.int32, tree.T)
    _dev(target_logits, "target_logits", torch.float32)
    _dev(draft, "draft", torch.float32)
    if draft.shape != target_logits.shape:
        raise ValueError("draft must match target_logits")
    _path_outputs(tree, accept_len, accept_nodes, out_tokens)
    if near_ties is not None:
        _dev(near_ties, "near_ties", torch.int32, tree.B)
    ws_bytes = workspace.numel() * workspace.element_size()
    _check(load_library().st_verify_stochastic_ex(
        tree.ref, V, _ptr(tokens), _ptr(target_logits), _ptr(draft), int(bool(draft_is_probs)),
        float(temperature), float(top_p), int(seed), int(offset), _ptr(accept_len),
        _ptr(accept_nodes), _ptr(out_tokens), _ptr(near_ties), _ptr(workspace), ws_bytes,
        _ptr(status), _stream()), "st_verify_stochastic_ex")


def st_tree_build(root_tokens, seqs, lens, V: int, cap: int, n_nodes, parent, tokens, depth,
                  node_off=None, parent_packed=None, tokens_packed=None, status=None):
    """Merge candidates seqs [B][K][Lmax] (lengths lens [B][K]) into one
    token tree per request: padded outputs [B][cap] and n_nodes [B]; with
    node_off [B+1] / parent_packed / tokens_packed [B*cap] also the
    concatenated st_tree layout."""
    B, K, Lmax = seqs.shape
    _dev(root_tokens, "root_tokens", torch.int32, B)
    _dev(seqs, "seqs", torch.int32)
    _dev(lens, "lens", torch.int32, B * K)
    _dev(n_nodes, "n_nodes", torch.int32, B)
    for name, t in (("parent", parent), ("tokens", tokens), ("depth", depth)):
        _dev(t, name, torch.int32, B * cap)
    packed = [node_off, parent_packed, tokens_packed]
    if any(t is not None for t in packed):
        if any(t is None for t in packed):
            raise ValueError("node_off, parent_packed and tokens_packed go together")
        _dev(node_off, "node_off", torch.int32, B + 1)
        _dev(parent_packed, "parent_packed", torch.int32, B * cap)
        _dev(tokens_packed, "tokens_packed", torch.int32, B * cap)
    _check(load_library().st_tree_build(
        B, K, Lmax, int(V), int(cap), _ptr(root_tokens), _ptr(seqs), _ptr(lens), _ptr(n_nodes),
        _ptr(parent), _ptr(tokens), _ptr(depth), _ptr(node_off), _ptr(parent_packed),
        _ptr(tokens_packed), _ptr(status), _stream()), "st_tree_build")


def st_stream_read(src: torch.Tensor, sink: torch.Tensor):
    """One read-only pass over src (the practical HBM read ceiling); sink is an
    int32 scratch tensor (its length bounds the launch width)."""
    _dev(src, "src")
    _dev(sink, "sink", torch.int32)
    nbytes = src.numel() * src.element_size()
    _check(load_library().st_stream_read(_ptr(src), nbytes - nbytes % 16, _ptr(sink),
                                         sink.numel(), _stream()), "st_stream_read")


def st_kv_compact_paged(k_pool, v_pool, block_table, prefix_len, accept_len, accept_nodes,
                        src_slot, new_len, status=None):
    """st_kv_compact on a paged pool [n_blocks][Hkv][block][D] (updated in
    place) through block_table int32 [B][max_blocks]."""
    n_blocks, Hkv, bs, D = k_pool.shape
    B, max_blocks = block_table.shape
    _dev(k_pool, "k_pool")
    _dev(v_pool, "v_pool", k_pool.dtype)
    if tuple(v_pool.shape) != tuple(k_pool.shape):
        raise ValueError("v_pool must match k_pool")
    _dev(block_table, "block_table", torch.int32)
    max_path = accept_nodes.shape[-1]
    _dev(prefix_len, "prefix_len", torch.int32, B)
    _dev(accept_len, "accept_len", torch.int32, B)
    _dev(accept_nodes, "accept_nodes", torch.int32, B * max_path)
    _dev(src_slot, "src_slot", torch.int32, B * max_path)
    _dev(new_len, "new_len", torch.int32, B)
    _check(load_library().st_kv_compact_paged(
        B, Hkv, D, _dtype_code(k_pool), _ptr(k_pool), _ptr(v_pool), n_blocks, bs,
        _ptr(block_table), max_blocks, _ptr(prefix_len), _ptr(accept_len), _ptr(accept_nodes),
        max_path, _ptr(src_slot), _ptr(new_len), _ptr(status), _stream()), "st_kv_compact_paged")


def st_kv_compact(k_cache, v_cache, prefix_len, accept_len, accept_nodes, src_slot, new_len,
                  status=None):
    """k_cache / v_cache [B][Hkv][S_max][D], updated in place."""
    B, Hkv, S_max, D = k_cache.shape
    _dev(k_cache, "k_cache")
    _dev(v_cache, "v_cache", k_cache.dtype)
    max_path = accept_nodes.shape[-1]
    _dev(prefix_len, "prefix_len", torch.int32, B)
    _dev(accept_len, "accept_len", torch.int32, B)
    _dev(accept_nodes, "accept_nodes", torch.int32, B * max_path)
    _dev(src_slot, "src_slot", torch.int32, B * max_path)
    _dev(new_len, "new_len", torch.int32, B)
    _check(load_library().st_kv_compact(
        B, Hkv, D, _dtype_code(k_cache), _ptr(k_cache), _ptr(v_cache), S_max, _ptr(prefix_len),
        _ptr(accept_len), _ptr(accept_nodes), max_path, _ptr(src_slot), _ptr(new_len),
        _ptr(status), _stream()), "st_kv_compact")


def _step_struct(tree: Tree, q, k_cache, v_cache, prefix_len, max_prefix: int, out, lse,
                 tokens, logits, draft_logits, temperature: float, seed: int, offset: int,
                 accept_len, accept_nodes, out_tokens, near_ties, src_slot, new_len,
                 scale: Optional[float], block_table=None) -> StStep:
    T, Hq, D = q.shape
    if block_table is None:
        B, Hkv, S_max, D2 = k_cache.shape
    else:                        # paged pools [n_blocks][Hkv][block][D]
        _, Hkv, bs, D2 = k_cache.shape
        B, max_blocks = block_table.shape
        S_max = max_blocks * bs
    if D2 != D or tuple(v_cache.shape) != tuple(k_cache.shape) or T != tree.T or B != tree.B:
        raise ValueError("shape mismatch between q, caches and tree")
    for name, t in (("q", q), ("k_cache", k_cache), ("v_cache", v_cache), ("out", out)):
        _dev(t, name, q.dtype)
    if out.shape != q.shape:
        raise ValueError("out must have q's shape")
    _dev(prefix_len, "prefix_len", torch.int32, B)
    if lse is not None:
        _dev(lse, "lse", torch.float32, T * Hq)
    V = logits.shape[-1]
    _dev(tokens, "tokens", torch.int32, T)
    _dev(logits, "logits", torch.float32, T * V)
    if draft_logits is not None:
        _dev(draft_logits, "draft_logits", torch.float32, T * V)
    _path_outputs(tree, accept_len, accept_nodes, out_tokens)
    _dev(src_slot, "src_slot", torch.int32, B * (tree.max_depth + 1))
    _dev(new_len, "new_len", torch.int32, B)
    if near_ties is not None:
        _dev(near_ties, "near_ties", torch.int32, B)
    scale = 1.0 / math.sqrt(D) if scale is None else float(scale)
    return StStep(Hq, Hkv, D, _dtype_code(q), scale, q.data_ptr(), k_cache.data_ptr(),
                  v_cache.data_ptr(), S_max, prefix_len.data_ptr(), max_prefix, out.data_ptr(),
                  0 if lse is None else lse.data_ptr(), V, tokens.data_ptr(), logits.data_ptr(),
                  0 if draft_logits is None else draft_logits.data_ptr(), float(temperature),
                  int(seed), int(offset), accept_len.data_ptr(), accept_nodes.data_ptr(),
                  out_tokens.data_ptr(), 0 if near_ties is None else near_ties.data_ptr(),
                  src_slot.data_ptr(), new_len.data_ptr())


def st_verification_step_workspace(tree: Tree, step: StStep) -> int:
    return load_library().st_verification_step_workspace(tree.ref, ctypes.byref(step))


def st_verification_step(tree: Tree, q, k_cache, v_cache, prefix_len, max_prefix: int, out, lse,
                         tokens, logits, accept_len, accept_nodes, out_tokens, src_slot, new_len,
                         workspace, draft_logits=None, temperature: float = 1.0, seed: int = 0,
                         offset: int = 0, near_ties=None, scale: Optional[float] = None,
                         status=None):
    """Acceptance, attention and compaction of one layer in one call (greedy
    when draft_logits is None, else stochastic).  The caches are compacted in
    place."""
    step = _step_struct(tree, q, k_cache, v_cache, prefix_len, max_prefix, out, lse, tokens,
                        logits, draft_logits, temperature, seed, offset, accept_len, accept_nodes,
                        out_tokens, near_ties, src_slot, new_len, scale)
    need = st_verification_step_workspace(tree, step)
    if need == 0:
        raise ValueError("st_verification_step: invalid arguments")
    if workspace is None or workspace.numel() * workspace.element_size() < need:
        raise ValueError(f"workspace needs {need} bytes")
    _check(load_library().st_verification_step(
        tree.ref, ctypes.byref(step), _ptr(workspace), workspace.numel() * workspace.element_size(),
        _ptr(status), _stream()), "st_verification_step")


def st_verification_step_noalloc(tree: Tree, q, k_cache, v_cache, prefix_len, max_prefix: int,
                                 out, lse, tokens, logits, accept_len, accept_nodes, out_tokens,
                                 src_slot, new_len, draft_logits=None, temperature: float = 1.0,
                                 seed: int = 0, offset: int = 0, near_ties=None,
                                 scale: Optional[float] = None, status=None):
    """st_verification_step without a workspace argument: the library's
    static per-GPU buffer serves as the workspace (no allocation)."""
    step = _step_struct(tree, q, k_cache, v_cache, prefix_len, max_prefix, out, lse, tokens,
                        logits, draft_logits, temperature, seed, offset, accept_len, accept_nodes,
                        out_tokens, near_ties, src_slot, new_len, scale)
    _check(load_library().st_verification_step_noalloc(tree.ref, ctypes.byref(step),
                                                       _ptr(status), _stream()),
           "st_verification_step_noalloc")


def st_verification_step_ex(tree: Tree, q, k_cache, v_cache, prefix_len, max_prefix: int, out,
                            lse, tokens, logits, accept_len, accept_nodes, out_tokens, src_slot,
                            new_len, workspace, draft, temperature: float = 1.0, seed: int = 0,
                            offset: int = 0, near_ties=None, scale: Optional[float] = None,
                            status=None, top_p: float = 1.0, draft_is_probs: bool = False):
    """st_verification_step with stochastic acceptance under nucleus
    filtering (top_p < 1) and/or the draft given as probabilities."""
    if draft is None:
        raise ValueError("st_verification_step_ex: draft is required")
    step = _step_struct(tree, q, k_cache, v_cache, prefix_len, max_prefix, out, lse, tokens,
                        logits, draft, temperature, seed, offset, accept_len, accept_nodes,
                        out_tokens, near_ties, src_slot, new_len, scale)
    need = st_verification_step_workspace(tree, step)
    if need == 0:
        raise ValueError("st_verification_step_ex: invalid arguments")
    if workspace is None or workspace.numel() * workspace.element_size() < need:
        raise ValueError(f"workspace needs {need} bytes")
    _check(load_library().st_verification_step_ex(
        tree.ref, ctypes.byref(step), int(bool(draft_is_probs)), float(top_p), _ptr(workspace),
        workspace.numel() * workspace.element_size(), _ptr(status), _stream()),
        "st_verification_step_ex")


def st_verification_step_paged(tree: Tree, q, k_pool, v_pool, block_table, prefix_len,
                               max_prefix: int, out, lse, tokens, logits, accept_len,
                               accept_nodes, out_tokens, src_slot, new_len, workspace,
                               draft_logits=None, temperature: float = 1.0, seed: int = 0,
                               offset: int = 0, near_ties=None, scale: Optional[float] = None,
                               status=None):
    """st_verification_step over paged pools [n_blocks][Hkv][block][D] through
    block_table int32 [B][max_blocks]; the pools are compacted in place."""
    _dev(block_table, "block_table", torch.int32)
    if tuple(v_pool.shape) != tuple(k_pool.shape):
        raise ValueError("v_pool must match k_pool")
    step = _step_struct(tree, q, k_pool, v_pool, prefix_len, max_prefix, out, lse, tokens,
                        logits, draft_logits, temperature, seed, offset, accept_len, accept_nodes,
                        out_tokens, near_ties, src_slot, new_len, scale, block_table=block_table)
    need = st_verification_step_workspace(tree, step)
    if need == 0:
        raise ValueError("st_verification_step_paged: invalid arguments")
    if workspace is None or workspace.numel() * workspace.element_size() < need:
        raise ValueError(f"workspace needs {need} bytes")
    n_blocks, _, bs, _ = k_pool.shape
    _check(load_library().st_verification_step_paged(
        tree.ref, ctypes.byref(step), n_blocks, bs, _ptr(block_table), block_table.shape[1],
        _ptr(workspace), workspace.numel() * workspace.element_size(), _ptr(status), _stream()),
        "st_verification_step_paged")


def st_embed(tokens, table, out, status=None):
    """out[t] = table[tokens[t]] (bf16 rows)."""
    V, d = table.shape
    T = tokens.numel()
    _dev(tokens, "tokens", torch.int32)
    _dev(table, "table", torch.bfloat16)
    _dev(out, "out", torch.bfloat16, T * d)
    _check(load_library().st_embed(T, d, V, _ptr(tokens), _ptr(table), _ptr(out), _ptr(status),
                                   _stream()), "st_embed")


def st_tree_rope_append(tree: Tree, qkv, Hq: int, Hkv: int, prefix_len, max_prefix: int,
                        q_out, k_cache, v_cache, theta: float = 10000.0, status=None):
    """qkv [T][(Hq + 2 Hkv) D] bf16 -> q_out [T][Hq][D]; rotated keys and values
    written at slots prefix_len[b] + i of k_cache / v_cache [B][Hkv][S_max][D]."""
    B, Hkv2, S_max, D = k_cache.shape
    if Hkv2 != Hkv or tuple(v_cache.shape) != tuple(k_cache.shape) or B != tree.B:
        raise ValueError("cache shapes do not match the tree and heads")
    _dev(qkv, "qkv", torch.bfloat16, tree.T * (Hq + 2 * Hkv) * D)
    _dev(q_out, "q_out", torch.bfloat16, tree.T * Hq * D)
    _dev(k_cache, "k_cache", torch.bfloat16)
    _dev(v_cache, "v_cache", torch.bfloat16)
    _dev(prefix_len, "prefix_len", torch.int32, B)
    _check(load_library().st_tree_rope_append(
        tree.ref, Hq, Hkv, D, float(theta), _ptr(qkv), _ptr(prefix_len), max_prefix, S_max,
        _ptr(q_out), _ptr(k_cache), _ptr(v_cache), _ptr(status), _stream()),
        "st_tree_rope_append")


def st_linear_workspace(M: int, N: int, K: int) -> int:
    return load_library().st_linear_workspace(M, N, K)


def st_linear(x, w, y, residual=None, workspace=None):
    """y[M][N] = x[M][K] . w[N][K]^T (+ residual), bf16 inputs, y bf16 or fp32."""
    M, K = x.shape
    N, K2 = w.shape
    if K2 != K or tuple(y.shape) != (M, N):
        raise ValueError("shape mismatch between x, w and y")
    _dev(x, "x", torch.bfloat16)
    _dev(w, "w", torch.bfloat16)
    _dev(y, "y")
    if residual is not None:
        _dev(residual, "residual", torch.bfloat16, M * N)
    need = st_linear_workspace(M, N, K)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    if need and ws_bytes < need:
        raise ValueError(f"workspace needs {need} bytes")
    _check(load_library().st_linear(
        M, N, K, _ptr(x), _ptr(w), _ptr(residual), _ptr(y), _dtype_code(y), _ptr(workspace),
        ws_bytes, _stream()), "st_linear")


def st_status_str(code: int) -> str:
    return load_library().st_status_str(code).decode()


def st_testing_set_plan(plan: Optional[dict]):
    """Test-only (include/st_testing.h): install planner overrides for every
    later call in the process, given as st_testing_plan fields; None restores
    the planners' own choices."""
    if plan is None:
        _check(load_library().st_testing_set_plan(None), "st_testing_set_plan")
        return
    p = StTestingPlan(attn_shape=-1)
    for k, v in plan.items():
        setattr(p, k, int(v))
    _check(load_library().st_testing_set_plan(ctypes.byref(p)), "st_testing_set_plan")
