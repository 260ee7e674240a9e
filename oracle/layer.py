"""One attention layer of a target model run over a token tree, and plain
autoregressive greedy decoding with the same model, in fp64.

Sources:
  [SpecInfer-news "研究現狀"] incremental decoding: the keys and values of the
      tokens already decoded are cached and reused.
  [SpecInfer-news "Token 樹驗證器"] all tree paths are verified in one pass of
      the target, through the tree attention mask.
  [SpecDec §3.2] the candidates are scored by a single forward pass.
  [Specular, 主要特性] greedy verification leaves the output identical to the
      original model's.

The pages fix no architecture.  Readings used here (a minimal model that has
every piece the verification pass touches):
  * hidden size d = Hq * D; one attention layer with a residual, then the
    vocabulary projection:
        x = E[token];  [q | k | v] = x Wqkv^T;  q, k <- rope(q, k, pos)
        a = attention(q, cache)  (tree mask, scale 1/sqrt(D), GQA h -> h // G)
        h = x + a Wo^T;  logits = h Wlm^T
  * rotary position embedding in the "rotate half" form: dims j and j + D/2
    form pair j, rotated by pos * theta^(-2j/D) (theta = 10000);
  * a tree node's position is P_b + depth: the index its token has in the
    sequence of its root path, so a path's keys are those of the same tokens
    decoded one by one;
  * node i's new key and value go to cache slot P_b + i before attention.
The functions here take weights as fp64 arrays; the tests pass the same bf16
values that the device path uses, decoded exactly.
"""

from __future__ import annotations

import numpy as np

from .attention import tree_attention
from .tree import depth_of

ROPE_THETA = 10000.0


def linear(x, w, residual=None):
    """x [M][K] times w [N][K] transposed, plus ``residual`` [M][N] if given."""
    y = np.asarray(x, np.float64) @ np.asarray(w, np.float64).T
    if residual is not None:
        y = y + np.asarray(residual, np.float64)
    return y


def rope_angles(pos, D: int, theta: float = ROPE_THETA):
    """Angles [len(pos)][D/2]: pos * theta^(-2j/D)."""
    j = np.arange(D // 2, dtype=np.float64)
    inv_freq = theta ** (-2.0 * j / D)
    return np.asarray(pos, np.float64)[:, None] * inv_freq[None, :]


def rope(x, pos, theta: float = ROPE_THETA):
    """Rotate x [n][H][D] at positions pos [n]: pair (j, j + D/2) turns by the
    pair's angle."""
    x = np.asarray(x, np.float64)
    D = x.shape[-1]
    ang = rope_angles(pos, D, theta)[:, None, :]          # [n][1][D/2]
    c, s = np.cos(ang), np.sin(ang)
    x1, x2 = x[..., :D // 2], x[..., D // 2:]
    return np.concatenate([x1 * c - x2 * s, x2 * c + x1 * s], axis=-1)


def node_positions(node_off, parent, prefix_len):
    """P_b + depth of every node [T]."""
    T = int(node_off[-1])
    pos = np.zeros(T, dtype=np.int64)
    for b in range(len(node_off) - 1):
        lo, hi = int(node_off[b]), int(node_off[b + 1])
        par = [int(x) for x in parent[lo:hi]]
        for i in range(hi - lo):
            pos[lo + i] = int(prefix_len[b]) + depth_of(par, i)
    return pos


def qkv_rope(params, cfg, x, pos):
    """Projections of hidden rows x [n][d] at positions pos: q [n][Hq][D]
    and k, v [n][Hkv][D], q and k rotated."""
    Hq, Hkv, D = cfg["Hq"], cfg["Hkv"], cfg["D"]
    qkv = linear(x, params["Wqkv"])
    n = qkv.shape[0]
    q = qkv[:, :Hq * D].reshape(n, Hq, D)
    k = qkv[:, Hq * D:(Hq + Hkv) * D].reshape(n, Hkv, D)
    v = qkv[:, (Hq + Hkv) * D:].reshape(n, Hkv, D)
    theta = cfg.get("theta", ROPE_THETA)
    return rope(q, pos, theta), rope(k, pos, theta), v


def tree_layer(params, cfg, tokens, node_off, parent, prefix_len, k_cache, v_cache):
    """The layer over every request's tree.  k_cache, v_cache [B][Hkv][S][D]
    hold the prefixes; copies with the tree keys and values appended at slots
    P_b + i are returned with the logits [T][V] and the intermediates."""
    Hq, D = cfg["Hq"], cfg["D"]
    T = int(node_off[-1])
    x = np.asarray(params["E"], np.float64)[np.asarray(tokens, np.int64)]
    pos = node_positions(node_off, parent, prefix_len)
    q, k, v = qkv_rope(params, cfg, x, pos)
    kc = np.array(k_cache, dtype=np.float64, copy=True)
    vc = np.array(v_cache, dtype=np.float64, copy=True)
    for b in range(len(node_off) - 1):
        lo, hi = int(node_off[b]), int(node_off[b + 1])
        P = int(prefix_len[b])
        kc[b, :, P:P + hi - lo, :] = k[lo:hi].transpose(1, 0, 2)
        vc[b, :, P:P + hi - lo, :] = v[lo:hi].transpose(1, 0, 2)
    att, _ = tree_attention(q, kc, vc, "f64", Hq, cfg["Hkv"], node_off, parent, prefix_len)
    a = att.reshape(T, Hq * D)
    h = linear(a, params["Wo"], residual=x)
    logits = linear(h, params["Wlm"])
    return dict(logits=logits, q=q, k=k, v=v, attn=a, h=h, k_cache=kc, v_cache=vc, pos=pos)


def prefix_cache(params, cfg, tokens, S_max: int):
    """Keys and values [1][Hkv][S_max][D] of a token sequence at positions
    0..n-1 (slots past n are zero)."""
    Hkv, D = cfg["Hkv"], cfg["D"]
    x = np.asarray(params["E"], np.float64)[np.asarray(tokens, np.int64)]
    _, k, v = qkv_rope(params, cfg, x, np.arange(len(tokens)))
    kc = np.zeros((1, Hkv, S_max, D))
    vc = np.zeros((1, Hkv, S_max, D))
    kc[0, :, :len(tokens)] = k.transpose(1, 0, 2)
    vc[0, :, :len(tokens)] = v.transpose(1, 0, 2)
    return kc, vc


def ar_greedy_decode(params, cfg, prompt, n_new: int):
    """Plain autoregressive greedy decoding: every new token attends causally
    to all earlier ones, one position at a time, with no tree and no mask.
    Returns (tokens [n_new], margins [n_new]): the margin is the gap between
    the largest and second largest logit of each step."""
    Hq, Hkv, D = cfg["Hq"], cfg["Hkv"], cfg["D"]
    G = Hq // Hkv
    E = np.asarray(params["E"], np.float64)
    theta = cfg.get("theta", ROPE_THETA)
    seq = [int(t) for t in prompt]
    keys, vals = [], []          # per position: [Hkv][D]
    out, margins = [], []
    for step in range(len(prompt) - 1 + n_new):
        p = step
        x = E[seq[p]][None, :]
        qkv = x @ np.asarray(params["Wqkv"], np.float64).T
        q = qkv[:, :Hq * D].reshape(1, Hq, D)
        k = qkv[:, Hq * D:(Hq + Hkv) * D].reshape(1, Hkv, D)
        v = qkv[:, (Hq + Hkv) * D:].reshape(1, Hkv, D)
        ang = p * theta ** (-2.0 * np.arange(D // 2) / D)
        c, s = np.cos(ang), np.sin(ang)

        def rot(z):
            z1, z2 = z[..., :D // 2], z[..., D // 2:]
            return np.concatenate([z1 * c - z2 * s, z2 * c + z1 * s], axis=-1)

        q, k = rot(q)[0], rot(k)[0]
        keys.append(k)
        vals.append(v[0])
        K = np.stack(keys, axis=1)   # [Hkv][p+1][D]
        Vv = np.stack(vals, axis=1)
        a = np.zeros((Hq, D))
        for h in range(Hq):
            sc = K[h // G] @ q[h] / np.sqrt(D)
            w = np.exp(sc - sc.max())
            a[h] = (w / w.sum()) @ Vv[h // G]
        hdn = x[0] + a.reshape(-1) @ np.asarray(params["Wo"], np.float64).T
        logits = hdn @ np.asarray(params["Wlm"], np.float64).T
        if p >= len(prompt) - 1:
            order = np.argsort(-logits, kind="stable")
            nxt = int(np.argmax(logits))
            out.append(nxt)
            margins.append(float(logits[order[0]] - logits[order[1]]))
            seq.append(nxt)
    return np.array(out, dtype=np.int32), np.array(margins)
