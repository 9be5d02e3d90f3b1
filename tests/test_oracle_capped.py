"""Pins of the importance-capped working set (the oracle's capped step).

OasisKV summary, key module 3: only the delta moves, and when the capped
cache has no room the least important blocks are evicted.  Checked against a
hand-worked sequence, against an independent priority-queue implementation
(``lru_list.HeapCapped``) on random sequences, and against invariants that
hold whatever the order.
"""
import json
import os

import numpy as np
import pytest

import oracle
from oracle.lru_list import HeapCapped

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "capped_hand.json")


def _one(table, S, k, scores, nb):
    sel = np.full((1, k), -1, dtype=np.int32)
    sel[0, :len(S)] = S
    return oracle.capped_step(table, sel, np.array([len(S)], np.int32), np.asarray(scores, np.float64)[None], nb)


def test_hand_worked_sequence():
    g = json.load(open(GOLDEN))
    table = np.full((1, g["capacity"]), -1, dtype=np.int32)
    for st in g["steps"]:
        out = _one(table, st["sel"], g["k"], st["scores"], g["nb"])
        n = len(st["sel"])
        assert out["sel_slot"][0, :n].tolist() == st["sel_slot"], st["why"]
        assert out["sel_hit"][0, :n].tolist() == st["sel_hit"], st["why"]
        m = int(out["miss_count"][0])
        assert [[int(b), int(s)] for b, s in zip(out["miss_block"][0, :m], out["miss_slot"][0, :m])] == st["misses"]
        assert table[0].tolist() == st["table"], st["why"]


@pytest.mark.parametrize("cap,k,nb,ties", [(8, 8, 64, False), (16, 8, 64, False), (40, 32, 300, True), (5, 3, 12, True)])
def test_c_oracle_matches_priority_queue(cap, k, nb, ties):
    r = np.random.default_rng(cap * 100 + k)
    rows = 3
    table = np.full((rows, cap), -1, dtype=np.int32)
    heaps = [HeapCapped(cap) for _ in range(rows)]
    cur = [sorted(r.choice(nb, size=k, replace=False).tolist()) for _ in range(rows)]
    for step in range(12):
        scores = r.standard_normal((rows, nb))
        if ties:
            scores = np.round(scores * 2) / 2
        sel = np.full((rows, k), -1, dtype=np.int32)
        cnt = np.zeros(rows, np.int32)
        for i in range(rows):
            if step:
                keep = set(r.choice(cur[i], size=int(0.7 * k), replace=False).tolist())
                while len(keep) < k:
                    keep.add(int(r.integers(0, nb)))
                cur[i] = sorted(keep)
            n = int(r.integers(1, k + 1)) if step % 5 == 4 else k  # partial selections now and then
            sel[i, :n] = cur[i][:n]
            cnt[i] = n
        out = oracle.capped_step(table, sel, cnt, scores, nb)
        for i in range(rows):
            n = cnt[i]
            ref = heaps[i].step(sel[i, :n].tolist(), {b: scores[i, b] for b in range(nb)})
            assert out["sel_slot"][i, :n].tolist() == ref[0]
            assert out["sel_hit"][i, :n].tolist() == ref[1]
            m = out["miss_count"][i]
            assert list(zip(out["miss_block"][i, :m].tolist(), out["miss_slot"][i, :m].tolist())) == ref[2]
            assert table[i].tolist() == heaps[i].slot_block


def test_evicted_blocks_are_never_more_important_than_kept_ones():
    r = np.random.default_rng(5)
    cap, k, nb = 24, 16, 200
    table = np.full((1, cap), -1, dtype=np.int32)
    for step in range(20):
        scores = r.standard_normal((1, nb))
        S = sorted(r.choice(nb, size=k, replace=False).tolist())
        before = table.copy()
        out = _one(table, S, k, scores[0], nb)
        evicted = [b for b in before[0] if b >= 0 and b not in set(table[0].tolist())]
        kept_unselected = [b for b in table[0] if b >= 0 and b not in set(S)]
        for e in evicted:
            assert e not in S
            for kb in kept_unselected:
                assert (scores[0, e], e) < (scores[0, kb], kb)
        # hits + misses = |S|, slots unique, every selected block resident
        assert out["sel_hit"][0, :k].sum() + out["miss_count"][0] == k
        res = table[0][table[0] >= 0]
        assert len(set(res.tolist())) == len(res) and set(S) <= set(res.tolist())


def test_invalid_rows_are_left_untouched():
    table = np.array([[3, -1, 7], [1, 1, -1], [0, 2, -1]], dtype=np.int32)
    sel = np.array([[3, 5], [1, 2], [2, 2]], dtype=np.int32)  # row 1: table holds block 1 twice; row 2: not ascending
    before = table.copy()
    out = oracle.capped_step(table, sel, np.array([2, 2, 2], np.int32), np.zeros((3, 10)), 10)
    assert out["miss_count"].tolist()[1:] == [-1, -1]
    assert np.array_equal(table[1:], before[1:])
    assert out["miss_count"][0] == 1 and table[0].tolist() == [3, 5, 7]  # the empty slot 1 takes block 5
