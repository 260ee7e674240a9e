"""Pins for the oracle's paged-KV helpers: a hand-worked gather, the closed
form of an identity table, and compaction on a pool agreeing with compaction
on the contiguous caches it describes."""

import numpy as np

import oracle
from synth import build_workload, make_paged, tree_random_attach


def test_hand_worked_gather():
    # 3 blocks of 2 rows, 1 head, D = 1: block j row r holds 10 j + r
    pool = np.array([[[[0], [1]]], [[[10], [11]]], [[[20], [21]]]], np.float32)
    table = np.array([[2, 0], [1, 1]], np.int32)
    g = oracle.gather_paged(pool, table, 2)
    assert g.shape == (2, 1, 4, 1)
    assert g[0, 0, :, 0].tolist() == [20, 21, 0, 1]
    assert g[1, 0, :, 0].tolist() == [10, 11, 10, 11]


def test_identity_table_is_a_reshape():
    rng = np.random.default_rng(0)
    B, Hkv, mb, bs, D = 3, 2, 4, 8, 5
    caches = rng.standard_normal((B, Hkv, mb * bs, D)).astype(np.float32)
    # block b * mb + j holds rows j*bs .. of request b
    pool = caches.reshape(B, Hkv, mb, bs, D).transpose(0, 2, 1, 3, 4).reshape(B * mb, Hkv, bs, D)
    table = np.arange(B * mb, dtype=np.int32).reshape(B, mb)
    assert np.array_equal(oracle.gather_paged(pool, table, bs), caches)


def test_scattered_layout_round_trip_and_spares():
    wl = build_workload("p", np.random.default_rng(1), dtype="bf16", Hq=2, Hkv=2, D=64, V=0,
                        prefix_lens=[40, 7], trees=[tree_random_attach(np.random.default_rng(2),
                                                                       9, 4)] * 2, max_depth=4)
    kp, vp, table = make_paged(3, wl.k_cache, wl.v_cache, 16, spare=2)
    assert kp.shape[0] == table.size + 2 and len(set(table.ravel().tolist())) == table.size
    g = oracle.gather_paged(kp, table, 16)
    assert np.array_equal(g[:, :, :wl.S_max], wl.k_cache)
    spares = sorted(set(range(kp.shape[0])) - set(table.ravel().tolist()))
    assert all((kp[s] == np.uint16(0x4480)).all() for s in spares)


def test_paged_compaction_matches_contiguous():
    rng = np.random.default_rng(4)
    trees = [tree_random_attach(rng, int(rng.integers(2, 40)), 7) for _ in range(3)]
    wl = build_workload("pc", rng, dtype="bf16", Hq=2, Hkv=2, D=64, V=0,
                        prefix_lens=[5, 33, 64], trees=trees, max_depth=7)
    kp, vp, table = make_paged(5, wl.k_cache, wl.v_cache, 32)
    mp = wl.max_depth + 1
    al = np.zeros(wl.B, np.int32)
    an = np.full((wl.B, mp), -1, np.int32)
    for b in range(wl.B):
        lo, hi = int(wl.node_off[b]), int(wl.node_off[b + 1])
        path = oracle.root_path(wl.parent[lo:hi], hi - lo - 1)[::-1]
        an[b, :len(path)] = path
        al[b] = len(path) - 1
    k2, v2, src, nl, st = oracle.kv_compact_paged(kp, vp, table, 32, wl.prefix_len, al, an, mp)
    kc, vc, src_c, nl_c, st_c = oracle.kv_compact(wl.k_cache, wl.v_cache, wl.prefix_len, al, an,
                                                  mp)
    assert st == st_c == 0
    assert np.array_equal(src, src_c) and np.array_equal(nl, nl_c)
    assert np.array_equal(oracle.gather_paged(k2, table, 32)[:, :, :wl.S_max], kc)
    assert np.array_equal(oracle.gather_paged(v2, table, 32)[:, :, :wl.S_max], vc)
    # blocks the table does not name are untouched
    spares = sorted(set(range(kp.shape[0])) - set(table.ravel().tolist()))
    assert all(np.array_equal(k2[s], kp[s]) for s in spares)
