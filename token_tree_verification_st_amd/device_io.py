"""Upload a host-side workload (numpy arrays) to device tensors and allocate
the outputs and workspaces of one verification step.  Plumbing only."""

from __future__ import annotations

from dataclasses import dataclass, field
from typing import Dict, Optional

import numpy as np
import torch

from .binding import (Tree, st_tree_attention_workspace, st_verify_greedy_workspace,
                      st_verify_stochastic_workspace)


def _t(x: np.ndarray, device, dtype=None) -> torch.Tensor:
    t = torch.from_numpy(np.ascontiguousarray(x))
    if dtype is not None:
        t = t.view(dtype)
    return t.to(device)


@dataclass
class DeviceWorkload:
    tree: Tree
    dtype: torch.dtype
    B: int
    T: int
    Hq: int
    Hkv: int
    D: int
    V: int
    S_max: int
    max_prefix: int
    temperature: float
    rng_seed: int
    rng_offset: int
    tokens: torch.Tensor
    prefix_len: torch.Tensor
    q: torch.Tensor
    k_cache: torch.Tensor
    v_cache: torch.Tensor
    logits: Optional[torch.Tensor]
    draft_logits: Optional[torch.Tensor]
    buf: Dict[str, torch.Tensor] = field(default_factory=dict)


def to_device(wl, device="cuda", max_prefix: Optional[int] = None) -> DeviceWorkload:
    """``wl`` has the fields of synth.Workload.  bf16 arrays hold raw 16-bit
    patterns and are reinterpreted, not converted."""
    dt = torch.float32 if wl.dtype == "f32" else torch.bfloat16
    raw = None if wl.dtype == "f32" else torch.int16
    conv = (lambda a: _t(a, device)) if raw is None else \
        (lambda a: _t(a.view(np.int16), device, dt))
    tree = Tree(_t(wl.node_off.astype(np.int32), device), _t(wl.parent.astype(np.int32), device),
                int(wl.max_nodes), int(wl.max_depth))
    mp = int(wl.prefix_len.max()) if max_prefix is None else int(max_prefix)
    dw = DeviceWorkload(
        tree=tree, dtype=dt, B=wl.B, T=wl.T, Hq=wl.Hq, Hkv=wl.Hkv, D=wl.D, V=wl.V,
        S_max=wl.S_max, max_prefix=mp, temperature=wl.temperature, rng_seed=wl.rng_seed,
        rng_offset=wl.rng_offset, tokens=_t(wl.tokens.astype(np.int32), device),
        prefix_len=_t(wl.prefix_len.astype(np.int32), device), q=conv(wl.q),
        k_cache=conv(wl.k_cache), v_cache=conv(wl.v_cache),
        logits=None if wl.logits is None else _t(wl.logits, device),
        draft_logits=None if wl.draft_logits is None else _t(wl.draft_logits, device))
    alloc_outputs(dw, device)
    return dw


def alloc_outputs(dw: DeviceWorkload, device="cuda"):
    tree = dw.tree
    mp = tree.max_depth + 1
    b = dw.buf
    b["mask"] = torch.zeros(dw.T * tree.W, dtype=torch.int64, device=device)
    b["depth"] = torch.zeros(dw.T, dtype=torch.int32, device=device)
    b["out"] = torch.empty_like(dw.q)
    b["lse"] = torch.empty(dw.T, dw.Hq, dtype=torch.float32, device=device)
    ws = st_tree_attention_workspace(tree, dw.Hq, dw.Hkv, dw.D, dw.dtype, dw.max_prefix)
    b["attn_ws"] = torch.empty(max(ws, 256), dtype=torch.uint8, device=device)
    b["accept_len"] = torch.zeros(dw.B, dtype=torch.int32, device=device)
    b["accept_nodes"] = torch.zeros(dw.B, mp, dtype=torch.int32, device=device)
    b["out_tokens"] = torch.zeros(dw.B, mp + 1, dtype=torch.int32, device=device)
    b["near_ties"] = torch.zeros(dw.B, dtype=torch.int32, device=device)
    if dw.V > 0:
        ws = max(st_verify_greedy_workspace(tree, dw.V), st_verify_stochastic_workspace(tree, dw.V))
        b["verify_ws"] = torch.empty(max(ws, 256), dtype=torch.uint8, device=device)
        # the one-call step: acceptance workspace (256-aligned), then attention's
        b["step_ws"] = torch.empty((ws + 255) // 256 * 256 + b["attn_ws"].numel(),
                                   dtype=torch.uint8, device=device)
    b["src_slot"] = torch.zeros(dw.B, mp, dtype=torch.int32, device=device)
    b["new_len"] = torch.zeros(dw.B, dtype=torch.int32, device=device)
    b["status"] = torch.zeros(1, dtype=torch.int32, device=device)
