"""Pins of the decode-time append (the oracle's append) and of Quest
metadata kept up to date by it: after any sequence of appends the block
min/max boxes equal those recomputed from the grown cache, the stored rows
are the appended ones, resident pool slots keep their blocks' bytes, and
full sequences do not move."""
import numpy as np

import oracle


def test_append_rows_lengths_and_pool():
    r = np.random.default_rng(1)
    B, Hkv, T, D, cap = 3, 2, 64, 8, 3
    k = r.standard_normal((B, Hkv, T, D)).astype(np.float32)
    v = r.standard_normal((B, Hkv, T, D)).astype(np.float32)
    lens = np.array([15, 63, 64], np.int32)  # a partial block, the last free token, a full sequence
    sb = np.array([[0, 0 + 15 // 16, -1], [3, -1, 1], [2, 3, 0], [0, 1, 2], [3, 2, 1], [-1, -1, 3]], np.int32)
    sb[0] = [0, -1, -1]
    pk = np.zeros((B, Hkv, cap, 16, D), np.float32)
    pv = np.zeros_like(pk)
    for rr in range(B * Hkv):  # every resident slot starts with its block's bytes
        b, j = divmod(rr, Hkv)
        for s, blk in enumerate(sb[rr]):
            if blk >= 0:
                pk[b, j, s] = k[b, j, 16 * blk:16 * blk + 16]
                pv[b, j, s] = v[b, j, 16 * blk:16 * blk + 16]
    nk = r.standard_normal((B, Hkv, D)).astype(np.float32)
    nv = r.standard_normal((B, Hkv, D)).astype(np.float32)
    k0, v0 = k.copy(), v.copy()
    oracle.append(nk, nv, lens, k, v, sb, pk, pv)
    assert lens.tolist() == [16, 64, 64]
    assert np.array_equal(k[0, :, 15], nk[0]) and np.array_equal(v[1, :, 63], nv[1])
    assert np.array_equal(k[2], k0[2]) and np.array_equal(v[2], v0[2])  # full: untouched
    changed = np.argwhere(np.any(k != k0, axis=-1))
    assert sorted(map(tuple, changed.tolist())) == [(0, 0, 15), (0, 1, 15), (1, 0, 63), (1, 1, 63)]
    for rr in range(B * Hkv):
        b, j = divmod(rr, Hkv)
        for s, blk in enumerate(sb[rr]):
            if blk >= 0:
                assert np.array_equal(pk[b, j, s], k[b, j, 16 * blk:16 * blk + 16])
                assert np.array_equal(pv[b, j, s], v[b, j, 16 * blk:16 * blk + 16])


def test_quest_boxes_stay_exact_under_appends():
    # min/max boxes maintained one token at a time (new block: the token
    # itself; else element-wise min/max with it) equal the recomputed ones
    r = np.random.default_rng(2)
    B, Hkv, T, D = 2, 2, 96, 16
    k = r.standard_normal((B, Hkv, T, D)).astype(np.float32)
    v = np.zeros_like(k)
    lens = np.array([5, 32], np.int32)
    meta = oracle.quest_meta(k, lens)
    for _ in range(40):
        nk = r.standard_normal((B, Hkv, D)).astype(np.float32)
        old = lens.copy()
        oracle.append(nk, np.zeros_like(nk), lens, k, v)
        for b in range(B):
            t = int(old[b])
            n = t // 16
            if t % 16 == 0:
                meta[b, :, n, 0] = nk[b]
                meta[b, :, n, 1] = nk[b]
            else:
                meta[b, :, n, 0] = np.minimum(meta[b, :, n, 0], nk[b])
                meta[b, :, n, 1] = np.maximum(meta[b, :, n, 1], nk[b])
        assert np.array_equal(meta, oracle.quest_meta(k, lens))
