"""Pins for the oracle's tree attention: hand-worked values, causal decoding,
sequence-by-sequence decoding of each root path, relabelling, GQA, closed forms.
Library routine used as an independent reference: torch's scaled_dot_product_attention
in float64 on the CPU."""

import numpy as np
import pytest
import torch
import torch.nn.functional as F
from scipy.special import logsumexp

import oracle
from synth import build_workload, f32_to_bf16_bits, tree_chain, tree_random_attach


def _rows(g, key):
    return np.array([[float(x) for x in r] for r in g[key]])


def _path(parent, i):
    out = []
    while i != -1:
        out.append(i)
        i = int(parent[i])
    return out[::-1]


def _single(parent, prefix, D, q, k, v, dtype="f32", Hq=1, Hkv=1):
    n = len(parent)
    node_off = np.array([0, n], np.int32)
    return oracle.tree_attention(q, k, v, dtype, Hq, Hkv, node_off, np.asarray(parent, np.int32),
                                 np.array([prefix], np.int32))


def test_hand_worked_uniform_weights(golden):
    g = golden("attention_small.txt")
    parent = [int(x) for x in g["parent"]]
    P = int(g["prefix"][0])
    v = _rows(g, "v").astype(np.float32)[None, None]          # [1][1][4][2]
    k = _rows(g, "caseA_k").astype(np.float32)[None, None]
    q = _rows(g, "caseA_q").astype(np.float32)[:, None, :]    # [3][1][2]
    out, lse = _single(parent, P, 2, q, k, v)
    np.testing.assert_allclose(out[:, 0, :], _rows(g, "caseA_out"), rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse[:, 0], [float(x) for x in g["caseA_lse"]], atol=1e-12)


def test_hand_worked_scaled_and_masked(golden):
    g = golden("attention_small.txt")
    parent = [int(x) for x in g["parent"]]
    P = int(g["prefix"][0])
    v = _rows(g, "v").astype(np.float32)[None, None]
    k = _rows(g, "caseB_k").astype(np.float32)[None, None]
    q = np.zeros((3, 1, 2), np.float32)
    q[1, 0, :] = [float(x) for x in g["caseB_q_node1"]]
    out, lse = _single(parent, P, 2, q, k, v)
    # q is rounded to fp32, so allow fp32-level error
    np.testing.assert_allclose(out[1, 0], [float(x) for x in g["caseB_out_node1"]], atol=1e-6)
    assert abs(lse[1, 0] - float(g["caseB_lse_node1"][0])) < 1e-6


def _sdpa(q, k, v, mask=None, causal=False, scale=None):
    return F.scaled_dot_product_attention(
        torch.from_numpy(q), torch.from_numpy(k), torch.from_numpy(v),
        attn_mask=None if mask is None else torch.from_numpy(mask), is_causal=causal,
        scale=scale).numpy()


@pytest.mark.parametrize("P", [0, 37])
def test_chain_equals_causal_incremental_decoding(P):
    rng = np.random.default_rng(11)
    n, D, H = 12, 16, 3
    parent, _ = tree_chain(n)
    q = rng.standard_normal((n, H, D)).astype(np.float32)
    k = rng.standard_normal((1, H, P + n, D)).astype(np.float32)
    v = rng.standard_normal((1, H, P + n, D)).astype(np.float32)
    out, _ = oracle.tree_attention(q, k, v, "f32", H, H, np.array([0, n], np.int32), parent,
                                   np.array([P], np.int32))
    qh = q.astype(np.float64).transpose(1, 0, 2)               # [H][n][D]
    kh, vh = k[0].astype(np.float64), v[0].astype(np.float64)
    if P == 0:
        ref = _sdpa(qh, kh, vh, causal=True)
    else:
        m = np.tril(np.ones((n, P + n), dtype=bool), k=P)      # row i sees keys <= P+i
        ref = _sdpa(qh, kh, vh, mask=m)
    np.testing.assert_allclose(out.transpose(1, 0, 2), ref, atol=1e-12)


@pytest.mark.parametrize("seed", range(6))
def test_each_node_equals_attention_over_its_root_path(seed):
    rng = np.random.default_rng(100 + seed)
    n = int(rng.integers(1, 17))
    P = int(rng.integers(0, 20))
    D, H = 8, 2
    parent, _ = tree_random_attach(rng, n, 5)
    q = rng.standard_normal((n, H, D)).astype(np.float32) * 2
    k = rng.standard_normal((1, H, P + n, D)).astype(np.float32)
    v = rng.standard_normal((1, H, P + n, D)).astype(np.float32)
    out, lse = oracle.tree_attention(q, k, v, "f32", H, H, np.array([0, n], np.int32), parent,
                                     np.array([P], np.int32))
    for i in range(n):
        slots = list(range(P)) + [P + j for j in _path(parent, i)]
        for h in range(H):
            qq = q[i, h].astype(np.float64)[None, None]
            kk = k[0, h, slots].astype(np.float64)[None]
            vv = v[0, h, slots].astype(np.float64)[None]
            ref = _sdpa(qq, kk, vv)[0, 0]
            np.testing.assert_allclose(out[i, h], ref, atol=1e-12)
            s = kk[0] @ qq[0, 0] / np.sqrt(D)
            assert abs(lse[i, h] - logsumexp(s)) < 1e-12


def test_relabelling_permutes_outputs():
    rng = np.random.default_rng(7)
    n, P, D, H = 14, 9, 8, 2
    parent, _ = tree_random_attach(rng, n, 6)
    # another topological order: repeatedly pick a random node whose parent is placed
    order, placed = [0], {0}
    while len(order) < n:
        ready = [i for i in range(n) if i not in placed and int(parent[i]) in placed]
        c = ready[int(rng.integers(0, len(ready)))]
        order.append(c)
        placed.add(c)
    new_of = {old: new for new, old in enumerate(order)}
    parent2 = np.array([-1] + [new_of[int(parent[old])] for old in order[1:]], np.int32)
    q = rng.standard_normal((n, H, D)).astype(np.float32)
    k = rng.standard_normal((1, H, P + n, D)).astype(np.float32)
    v = rng.standard_normal((1, H, P + n, D)).astype(np.float32)
    slot_perm = list(range(P)) + [P + old for old in order]
    out1, _ = oracle.tree_attention(q, k, v, "f32", H, H, np.array([0, n], np.int32), parent,
                                    np.array([P], np.int32))
    out2, _ = oracle.tree_attention(q[order], k[:, :, slot_perm], v[:, :, slot_perm], "f32", H, H,
                                    np.array([0, n], np.int32), parent2, np.array([P], np.int32))
    np.testing.assert_allclose(out2, out1[order], atol=1e-12)


def test_single_node_is_one_token_decode():
    rng = np.random.default_rng(3)
    P, D, H = 50, 16, 4
    q = rng.standard_normal((1, H, D)).astype(np.float32)
    k = rng.standard_normal((1, H, P + 1, D)).astype(np.float32)
    v = rng.standard_normal((1, H, P + 1, D)).astype(np.float32)
    out, _ = oracle.tree_attention(q, k, v, "f32", H, H, np.array([0, 1], np.int32),
                                   np.array([-1], np.int32), np.array([P], np.int32))
    ref = _sdpa(q.astype(np.float64).transpose(1, 0, 2), k[0].astype(np.float64),
                v[0].astype(np.float64))
    np.testing.assert_allclose(out.transpose(1, 0, 2), ref, atol=1e-12)


def test_closed_forms_constant_values_and_zero_queries():
    rng = np.random.default_rng(4)
    n, P, D, H = 10, 6, 4, 1
    parent, _ = tree_random_attach(rng, n, 4)
    k = rng.standard_normal((1, H, P + n, D)).astype(np.float32)
    vconst = np.tile(np.array([1.5, -2.0, 0.25, 3.0], np.float32), (1, H, P + n, 1))
    q = rng.standard_normal((n, H, D)).astype(np.float32)
    out, _ = oracle.tree_attention(q, k, vconst, "f32", H, H, np.array([0, n], np.int32), parent,
                                   np.array([P], np.int32))
    np.testing.assert_allclose(out[:, 0], np.tile(vconst[0, 0, 0], (n, 1)), atol=1e-12)
    v = rng.standard_normal((1, H, P + n, D)).astype(np.float32)
    out, lse = oracle.tree_attention(np.zeros_like(q), k, v, "f32", H, H,
                                     np.array([0, n], np.int32), parent, np.array([P], np.int32))
    for i in range(n):
        slots = list(range(P)) + [P + j for j in _path(parent, i)]
        np.testing.assert_allclose(out[i, 0], v[0, 0, slots].astype(np.float64).mean(0),
                                   atol=1e-12)
        assert abs(lse[i, 0] - np.log(len(slots))) < 1e-12


def test_gqa_equals_mha_with_repeated_kv_heads():
    rng = np.random.default_rng(9)
    n, P, D, Hq, Hkv = 9, 13, 8, 8, 2
    parent, _ = tree_random_attach(rng, n, 4)
    q = rng.standard_normal((n, Hq, D)).astype(np.float32)
    k = rng.standard_normal((1, Hkv, P + n, D)).astype(np.float32)
    v = rng.standard_normal((1, Hkv, P + n, D)).astype(np.float32)
    args = (np.array([0, n], np.int32), parent, np.array([P], np.int32))
    out_g, _ = oracle.tree_attention(q, k, v, "f32", Hq, Hkv, *args)
    G = Hq // Hkv
    kr, vr = np.repeat(k, G, axis=1), np.repeat(v, G, axis=1)
    out_m, _ = oracle.tree_attention(q, kr, vr, "f32", Hq, Hq, *args)
    np.testing.assert_allclose(out_g, out_m, atol=1e-12)


def test_multi_request_batches_are_independent():
    rng = np.random.default_rng(21)
    wl = build_workload("t", rng, dtype="f32", Hq=2, Hkv=2, D=8, V=0, prefix_lens=[5, 11],
                        trees=[tree_random_attach(rng, 6, 3), tree_random_attach(rng, 4, 3)],
                        max_depth=3)
    out, _ = oracle.tree_attention(wl.q, wl.k_cache, wl.v_cache, "f32", 2, 2, wl.node_off,
                                   wl.parent, wl.prefix_len)
    for b in range(2):
        lo, hi = int(wl.node_off[b]), int(wl.node_off[b + 1])
        n = hi - lo
        P = int(wl.prefix_len[b])
        sub, _ = oracle.tree_attention(wl.q[lo:hi], wl.k_cache[b:b + 1, :, :P + n],
                                       wl.v_cache[b:b + 1, :, :P + n], "f32", 2, 2,
                                       np.array([0, n], np.int32), wl.parent[lo:hi],
                                       np.array([P], np.int32))
        np.testing.assert_allclose(out[lo:hi], sub, atol=1e-12)


def test_sampled_rows_match_full_computation():
    rng = np.random.default_rng(22)
    n, P, D, H = 12, 20, 8, 4
    parent, _ = tree_random_attach(rng, n, 5)
    q = rng.standard_normal((n, H, D)).astype(np.float32)
    k = rng.standard_normal((1, H, P + n, D)).astype(np.float32)
    v = rng.standard_normal((1, H, P + n, D)).astype(np.float32)
    args = ("f32", H, H, np.array([0, n], np.int32), parent, np.array([P], np.int32))
    full, _ = oracle.tree_attention(q, k, v, *args)
    part, _ = oracle.tree_attention(q, k, v, *args, nodes=[3, 7], heads=[1, 2])
    np.testing.assert_allclose(part[[3, 7]][:, [1, 2]], full[[3, 7]][:, [1, 2]], atol=0)
    assert np.isnan(part[0]).all() and np.isnan(part[3, 0]).all()


def test_bf16_decoding_and_rounding():
    bits = np.array([0x3F80, 0xC000, 0x3E80, 0x0000, 0x8000], np.uint16)
    np.testing.assert_array_equal(oracle.decode_values(bits, "bf16"), [1.0, -2.0, 0.25, 0.0, -0.0])
    # round to nearest, ties to even, on values exactly between two bf16 numbers
    x = np.array([1.0 + 2.0 ** -8, 1.0 + 3 * 2.0 ** -8, 1.0 + 2.0 ** -8 + 2.0 ** -20], np.float32)
    np.testing.assert_array_equal(f32_to_bf16_bits(x), np.array([0x3F80, 0x3F82, 0x3F81], np.uint16))
