"""Pins of the cross-layer prefetch as the oracle models it: the next
layer's working set is first updated with the previous layer's selection
(an ordinary LRU step), then with its own.  HiSparse promo, insight 3: top-k
picks overlap between layers, so fetching the previous layer's picks for the
next layer early hides about half of the remaining miss cost.

Checked here: with room for every block the two steps compose as plain set
arithmetic; a hand-worked case where the hint evicts a block the real pick
needs; and on the host-tier recipe (about half of the blocks shared between
adjacent layers) the real misses after the hint are about half of those
without it, at the price of extra prefetched blocks.
"""
import numpy as np

import oracle
from top_sparse_kv_block_amd import synth


def _step(lru, sel, nb):
    sel = np.asarray(sel, np.int32).reshape(lru.rows, -1)
    cnt = np.full(lru.rows, sel.shape[1], np.int32)
    return lru.step(sel, cnt, nb)


def test_hint_then_pick_is_set_arithmetic_when_nothing_is_evicted():
    rng = np.random.default_rng(7)
    nb, k, cap = 512, 16, 512
    lru = oracle.LRU(1, cap)
    resident = set()
    for _ in range(12):
        hint = sorted(rng.choice(nb, k, replace=False).tolist())
        pick = sorted(set(rng.choice(hint, k // 2, replace=False).tolist())
                      | set(rng.choice(nb, k, replace=False).tolist()))[:k]
        pick = sorted(pick)
        h = _step(lru, hint, nb)
        assert h["miss_count"][0] == len(set(hint) - resident)
        resident |= set(hint)
        out = _step(lru, pick, nb)
        assert out["miss_count"][0] == len(set(pick) - resident)
        np.testing.assert_array_equal(out["sel_hit"][0, :len(pick)], [b in resident for b in pick])
        resident |= set(pick)
        assert set(lru.slot_block()[0][lru.slot_block()[0] >= 0].tolist()) == resident


def test_hint_can_evict_a_block_the_pick_needs():
    # 4 slots filled with 1, 2, 3, 4 (touched in that order: 1 is the least recent)
    lru = oracle.LRU(1, 4)
    for b in (1, 2, 3, 4):
        _step(lru, [b], 16)
    h = _step(lru, [5, 6], 16)  # the hint evicts the two least recent: 1 and 2
    np.testing.assert_array_equal(h["miss_block"][0], [5, 6])
    np.testing.assert_array_equal(h["miss_slot"][0], [0, 1])
    out = _step(lru, [2, 5, 7], 16)  # 5 is a hit; 2 was evicted by the hint; 7 is new
    np.testing.assert_array_equal(out["sel_hit"][0], [0, 1, 0])
    np.testing.assert_array_equal(out["miss_block"][0], [2, 7, -1])
    np.testing.assert_array_equal(out["miss_slot"][0], [2, 3, -1])  # 3 then 4 are the least recent left
    np.testing.assert_array_equal(lru.slot_block()[0], [5, 6, 2, 7])


def test_prefetch_halves_the_misses_on_the_host_tier_recipe():
    w = synth.WORKLOADS["host_tier_32l"].scaled(batch=2, layers=4, steps=5)
    sels = synth.gen_layer_selections(w)  # [steps, layers, B, Hkv, k]
    P, k, C, nb = w.rows, w.k_blocks, w.capacity, w.nb_max
    plain = [oracle.LRU(P, C) for _ in range(w.layers)]
    pref = [oracle.LRU(P, C) for _ in range(w.layers)]
    base = real = extra = 0
    cnt = np.full(P, k, np.int32)
    for s in range(w.steps):
        for l in range(w.layers):
            sel = sels[s, l].reshape(P, k)
            m0 = plain[l].step(sel, cnt, nb)["miss_count"].sum()
            if l > 0:
                extra_l = pref[l].step(sels[s, l - 1].reshape(P, k), cnt, nb)["miss_count"].sum()
            m1 = pref[l].step(sel, cnt, nb)["miss_count"].sum()
            if s > 0 and l > 0:
                base, real, extra = base + m0, real + m1, extra + extra_l
    # about k/5 new blocks per row and layer, half of them shared with the layer before
    assert 0.15 * k * P * 12 < base < 0.25 * k * P * 12
    assert 0.4 < real / base < 0.6, (real, base)
    # the hint itself fetches the shared new blocks and the previous layer's own new ones
    assert extra > base * 0.8
