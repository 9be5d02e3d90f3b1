"""Pins of the oracle's working-set step and fetch (CPU only)."""
import json
import os

import numpy as np
from hypothesis import given, settings, strategies as st

import oracle
from oracle.lru_list import ListLRU

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def test_hand_worked_sequences():
    with open(os.path.join(GOLD, "lru_hand.json")) as f:
        g = json.load(f)
    for seq in g["sequences"]:
        C, k, nbl = seq["capacity"], seq["k"], seq["nb_limit"]
        c_lru, py_lru = oracle.LRU(1, C), ListLRU(C)
        for st_ in seq["steps"]:
            S = st_["S"]
            sel = np.full((1, k), -1, dtype=np.int32)
            sel[0, :len(S)] = S
            out = c_lru.step(sel, np.array([len(S)], dtype=np.int32), nbl)
            py = py_lru.step(S, nbl)
            if st_.get("invalid"):
                assert out["miss_count"][0] == -1 and py is None
            else:
                n = len(S)
                assert out["sel_slot"][0, :n].tolist() == st_["sel_slot"]
                assert out["sel_hit"][0, :n].tolist() == st_["sel_hit"]
                m = out["miss_count"][0]
                got = list(zip(out["miss_block"][0, :m].tolist(), out["miss_slot"][0, :m].tolist()))
                assert [list(x) for x in got] == st_["misses"]
                assert py == (st_["sel_slot"], st_["sel_hit"], [tuple(x) for x in st_["misses"]])
            assert c_lru.slot_block()[0].tolist() == st_["slot_block"]
            order = c_lru.order()[0]
            assert order[order >= 0].tolist() == st_["lru_order"]
            assert list(py_lru.lru.keys()) == st_["lru_order"]


def _chain(r, nb, k, steps, retain):
    cur = sorted(r.choice(nb, size=k, replace=False).tolist())
    out = [cur]
    for _ in range(steps - 1):
        keep = r.choice(cur, size=int(retain * k), replace=False).tolist() if retain > 0 else []
        s = set(keep)
        while len(s) < k:
            s.add(int(r.integers(0, nb)))
        cur = sorted(s)
        out.append(cur)
    return out


@settings(max_examples=60, deadline=None)
@given(cap=st.integers(1, 24), k=st.integers(1, 24), nb=st.integers(1, 60), steps=st.integers(1, 12),
       retain=st.sampled_from([0.0, 0.5, 0.8, 1.0]), seed=st.integers(0, 2**31 - 1))
def test_c_list_agrees_with_python_list(cap, k, nb, steps, retain, seed):
    k = min(k, cap, nb)
    r = np.random.default_rng(seed)
    rows = 3
    c_lru = oracle.LRU(rows, cap)
    py = [ListLRU(cap) for _ in range(rows)]
    chains = [_chain(r, nb, k, steps, retain) for _ in range(rows)]
    for t in range(steps):
        sel = np.full((rows, k), -1, dtype=np.int32)
        cnt = np.zeros(rows, dtype=np.int32)
        for i in range(rows):
            S = chains[i][t][: int(r.integers(0, k + 1))] if r.random() < 0.2 else chains[i][t]
            sel[i, :len(S)] = S
            cnt[i] = len(S)
        out = c_lru.step(sel, cnt, nb)
        for i in range(rows):
            S = sel[i, :cnt[i]].tolist()
            p = py[i].step(S, nb)
            n = cnt[i]
            assert out["sel_slot"][i, :n].tolist() == p[0]
            assert out["sel_hit"][i, :n].tolist() == p[1]
            m = out["miss_count"][i]
            assert list(zip(out["miss_block"][i, :m].tolist(), out["miss_slot"][i, :m].tolist())) == p[2]
        assert c_lru.slot_block().tolist() == [p.slot_block for p in py]


def test_timestamp_form_matches_list():
    # The list order equals ascending (last-touch step, block id): within a
    # step blocks are touched in ascending id order.  This is the form a
    # parallel implementation uses; checked here against the list.
    r = np.random.default_rng(21)
    cap, k, nb, steps = 16, 6, 40, 30
    lru = oracle.LRU(1, cap)
    stamp = {}
    for t, S in enumerate(_chain(r, nb, k, steps, 0.5)):
        sel = np.array([S], dtype=np.int32)
        out = lru.step(sel, np.array([k], dtype=np.int32), nb)
        sb = lru.slot_block()[0]
        for s in out["sel_slot"][0]:
            stamp[int(s)] = t
        order = lru.order()[0]
        order = order[order >= 0].tolist()
        assert order == sorted(order, key=lambda s: (stamp[s], sb[s]))


def test_transfer_invariant_when_capacity_equals_budget():
    # With capacity = budget the resident set after a step is the selection,
    # so the blocks moved equal |S_now - S_last| ("KV Cache 塞不进 HBM 了" §2.1)
    r = np.random.default_rng(22)
    k, nb = 8, 64
    lru = oracle.LRU(1, k)
    prev = set()
    for S in _chain(r, nb, k, 20, 0.8):
        out = lru.step(np.array([S], dtype=np.int32), np.array([k], dtype=np.int32), nb)
        assert out["miss_count"][0] == len(set(S) - prev)
        assert set(lru.slot_block()[0].tolist()) == set(S)
        prev = set(S)


def test_transfer_bound_when_capacity_exceeds_budget():
    r = np.random.default_rng(23)
    k, cap, nb = 8, 16, 64
    lru = oracle.LRU(1, cap)
    prev_sel, prev_res = set(), set()
    for S in _chain(r, nb, k, 25, 0.6):
        out = lru.step(np.array([S], dtype=np.int32), np.array([k], dtype=np.int32), nb)
        m = out["miss_count"][0]
        assert m == len(set(S) - prev_res) <= len(set(S) - prev_sel)
        assert int(out["sel_hit"][0].sum()) + m == len(S)
        res = lru.slot_block()[0]
        assert set(S) <= set(res.tolist())
        occ = res[res >= 0]
        assert len(occ) == len(set(occ.tolist()))
        prev_sel, prev_res = set(S), set(occ.tolist())


def test_flush_moves_everything_again():
    lru = oracle.LRU(1, 4)
    S = np.array([[2, 5, 7]], dtype=np.int32)
    c = np.array([3], dtype=np.int32)
    assert lru.step(S, c, 10)["miss_count"][0] == 3
    assert lru.step(S, c, 10)["miss_count"][0] == 0
    lru.flush()
    out = lru.step(S, c, 10)
    assert out["miss_count"][0] == 3 and out["sel_slot"][0].tolist() == [0, 1, 2]


def test_gather_copies_blocks_bit_exact():
    r = np.random.default_rng(24)
    B, Hkv, T, D, cap, k = 2, 2, 64, 8, 3, 2
    src_k = r.standard_normal((B, Hkv, T, D)).astype(np.float32)
    src_v = r.standard_normal((B, Hkv, T, D)).astype(np.float32)
    pk = np.zeros((B, Hkv, cap, 16, D), dtype=np.float32)
    pv = np.zeros_like(pk)
    mb = np.array([[1, 3], [0, -1], [2, -1], [-1, -1]], dtype=np.int32)
    ms = np.array([[2, 0], [1, -1], [0, -1], [-1, -1]], dtype=np.int32)
    mc = np.array([2, 1, 1, 0], dtype=np.int32)
    oracle.gather(mb, ms, mc, src_k, src_v, pk, pv)
    assert np.array_equal(pk[0, 0, 2], src_k[0, 0, 16:32]) and np.array_equal(pv[0, 0, 0], src_v[0, 0, 48:64])
    assert np.array_equal(pk[0, 1, 1], src_k[0, 1, 0:16]) and np.array_equal(pv[1, 0, 0], src_v[1, 0, 32:48])
    assert not pk[1, 1].any() and not pk[0, 0, 1].any()


def _padded(out, i, k):
    return (out["sel_slot"][i].tolist() == [-1] * k and out["sel_hit"][i].tolist() == [0] * k
            and out["miss_block"][i].tolist() == [-1] * k and out["miss_slot"][i].tolist() == [-1] * k)


def test_hand_worked_loaded_tables():
    # rows started from a given slot table and stamps; refused tables
    # (an unselected block held twice, a selected one held twice, ids out of
    # range) leave the row untouched with padded lists
    with open(os.path.join(GOLD, "lru_loaded.json")) as f:
        g = json.load(f)
    for seq in g["sequences"]:
        C, k, nbl = seq["capacity"], seq["k"], seq["nb_limit"]
        c_lru, py_lru = oracle.LRU(1, C), ListLRU(C)
        c_lru.load(np.array([seq["table"]], np.int32), np.array([seq["stamps"]], np.uint32))
        py_lru.load(seq["table"], seq["stamps"])
        order = c_lru.order()[0]
        assert order[order >= 0].tolist() == seq["order"] == list(py_lru.lru.keys()), seq["why"]
        for st_ in seq["steps"]:
            S = st_["S"]
            sel = np.full((1, k), -1, dtype=np.int32)
            sel[0, :len(S)] = S
            out = c_lru.step(sel, np.array([len(S)], dtype=np.int32), nbl)
            py = py_lru.step(S, nbl)
            if st_.get("invalid"):
                assert out["miss_count"][0] == -1 and _padded(out, 0, k) and py is None, seq["why"]
            else:
                n = len(S)
                assert out["sel_slot"][0, :n].tolist() == st_["sel_slot"], seq["why"]
                assert out["sel_hit"][0, :n].tolist() == st_["sel_hit"], seq["why"]
                m = out["miss_count"][0]
                got = list(zip(out["miss_block"][0, :m].tolist(), out["miss_slot"][0, :m].tolist()))
                assert [list(x) for x in got] == st_["misses"], seq["why"]
                assert py == (st_["sel_slot"], st_["sel_hit"], [tuple(x) for x in st_["misses"]])
            assert c_lru.slot_block()[0].tolist() == st_["slot_block"] == py_lru.slot_block, seq["why"]
            order = c_lru.order()[0]
            assert order[order >= 0].tolist() == st_["lru_order"] == list(py_lru.lru.keys()), seq["why"]


def test_unselected_duplicate_is_refused_by_both_policies():
    # the same table, once with the duplicated block selected and once not:
    # both the LRU and the importance-capped step refuse both
    table = np.array([[7, 3, 3, -1], [7, 3, 3, -1], [7, 3, 4, -1]], np.int32)
    sel = np.array([[7, 8], [3, 8], [7, 8]], np.int32)
    cnt = np.array([2, 2, 2], np.int32)
    lru = oracle.LRU(3, 4)
    lru.load(table, np.zeros((3, 4), np.uint32))
    out = lru.step(sel, cnt, 20)
    assert out["miss_count"].tolist() == [-1, -1, 1]
    assert _padded(out, 0, 2) and _padded(out, 1, 2)
    assert lru.slot_block()[:2].tolist() == table[:2].tolist()
    capped = table.copy()
    out = oracle.capped_step(capped, sel, cnt, np.zeros((3, 20)), 20)
    assert out["miss_count"].tolist() == [-1, -1, 1]
    assert _padded(out, 0, 2) and _padded(out, 1, 2)
    assert capped[:2].tolist() == table[:2].tolist() and capped[2].tolist() == [7, 3, 4, 8]


@settings(max_examples=80, deadline=None)
@given(cap=st.integers(1, 20), k=st.integers(1, 20), nb=st.integers(1, 40), steps=st.integers(1, 8),
       corrupt=st.sampled_from([0.0, 0.3]), seed=st.integers(0, 2**31 - 1))
def test_loaded_tables_c_agrees_with_python(cap, k, nb, steps, corrupt, seed):
    # random tables (some with a block held twice or an id out of range) and
    # random stamps, then random selections: the C list and the Python list
    # agree on every step, refused rows included
    k = min(k, cap, nb)
    r = np.random.default_rng(seed)
    rows = 4
    table = np.full((rows, cap), -1, np.int32)
    stamps = r.integers(0, 5, size=(rows, cap)).astype(np.uint32)
    for i in range(rows):
        n = int(r.integers(0, min(cap, nb) + 1))
        table[i, r.choice(cap, size=n, replace=False)] = r.choice(nb, size=n, replace=False)
        if r.random() < corrupt and n >= 1:
            s = int(r.integers(0, cap))
            table[i, s] = r.choice([int(table[i][table[i] >= 0][0]), nb, -2])
    c_lru = oracle.LRU(rows, cap)
    c_lru.load(table, stamps)
    py = [ListLRU(cap) for _ in range(rows)]
    for i in range(rows):
        py[i].load(table[i].tolist(), stamps[i].tolist())
    for t in range(steps):
        sel = np.full((rows, k), -1, np.int32)
        cnt = np.zeros(rows, np.int32)
        for i in range(rows):
            n = int(r.integers(0, k + 1))
            sel[i, :n] = np.sort(r.choice(nb, size=n, replace=False))
            cnt[i] = n
        out = c_lru.step(sel, cnt, nb)
        for i in range(rows):
            p = py[i].step(sel[i, :cnt[i]].tolist(), nb)
            if p is None:
                assert out["miss_count"][i] == -1 and _padded(out, i, k)
                continue
            n = cnt[i]
            assert out["sel_slot"][i, :n].tolist() == p[0]
            assert out["sel_hit"][i, :n].tolist() == p[1]
            m = out["miss_count"][i]
            assert list(zip(out["miss_block"][i, :m].tolist(), out["miss_slot"][i, :m].tolist())) == p[2]
        assert c_lru.slot_block().tolist() == [p.slot_block for p in py]
        order = c_lru.order()
        assert [o[o >= 0].tolist() for o in order] == [list(p.lru.keys()) for p in py]


def test_snapshot_restore_continues_bit_identically():
    # checkpoint / resume of the working set: run T steps; separately run
    # T/2 steps, save the table and each slot's last-touch step, start a
    # fresh list from them and run the other T/2.  The later steps' lists
    # and tables are identical (the block table can be saved and restored:
    # KV-Cache 压缩技术的工程原理 §6.1)
    r = np.random.default_rng(31)
    rows, cap, k, nb, T = 3, 12, 8, 50, 10
    chains = [_chain(r, nb, k, T, 0.6) for _ in range(rows)]

    def sel_at(t):
        sel = np.array([chains[i][t] for i in range(rows)], np.int32)
        return sel, np.full(rows, k, np.int32)

    full = oracle.LRU(rows, cap)
    ref = [full.step(*sel_at(t), nb) for t in range(T)]
    first = oracle.LRU(rows, cap)
    touch = np.zeros((rows, cap), np.uint32)
    for t in range(T // 2):
        out = first.step(*sel_at(t), nb)
        for i in range(rows):
            touch[i, out["sel_slot"][i][out["sel_slot"][i] >= 0]] = t + 1
    resumed = oracle.LRU(rows, cap)
    resumed.load(first.slot_block(), touch)
    assert resumed.order().tolist() == first.order().tolist()
    for t in range(T // 2, T):
        out = resumed.step(*sel_at(t), nb)
        for key in ref[t]:
            assert np.array_equal(out[key], ref[t][key]), (t, key)
    assert resumed.slot_block().tolist() == full.slot_block().tolist()
