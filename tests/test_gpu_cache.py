"""GPU parity of stage 3 (working-set manager + miss fetch) against the oracle.

The GPU's stamp/atomic-clock LRU must reproduce the oracle's linked list bit
for bit given the same selections: slot of every selected block, hit flags,
the compacted (block, slot) miss list, the miss count and the slot table.
The fetched pool blocks must equal the source bytes.
"""
import numpy as np
import pytest
import torch

import oracle
from top_sparse_kv_block_amd import binding as B
from top_sparse_kv_block_amd import synth
from top_sparse_kv_block_amd.step import LayerBuffers, StepConfig
from gpu_util import assert_lists, assert_lru_state, dev, host, log, to_dtype

pytestmark = pytest.mark.gpu


def _chains(r, rows, nb, k, steps, retain, partial=0.0):
    out = []
    for _ in range(rows):
        cur = sorted(r.choice(nb, size=k, replace=False).tolist())
        seq = []
        for t in range(steps):
            if t:
                keep = r.choice(cur, size=int(retain * k), replace=False).tolist() if retain else []
                s = set(keep)
                while len(s) < k:
                    s.add(int(r.integers(0, nb)))
                cur = sorted(s)
            S = cur[: int(r.integers(0, k + 1))] if r.random() < partial else cur
            seq.append(S)
        out.append(seq)
    return out


def _pack(chains, t, k):
    rows = len(chains)
    sel = np.full((rows, k), -1, dtype=np.int32)
    cnt = np.zeros(rows, dtype=np.int32)
    for i in range(rows):
        S = chains[i][t]
        sel[i, :len(S)] = S
        cnt[i] = len(S)
    return sel, cnt


def _compare(buf, out, rows, k):
    np.testing.assert_array_equal(host(buf.miss_count).reshape(rows), out["miss_count"])
    np.testing.assert_array_equal(host(buf.sel_slot).reshape(rows, k), out["sel_slot"])
    np.testing.assert_array_equal(host(buf.sel_hit).reshape(rows, k), out["sel_hit"])
    np.testing.assert_array_equal(host(buf.miss_block).reshape(rows, k), out["miss_block"])
    np.testing.assert_array_equal(host(buf.miss_slot).reshape(rows, k), out["miss_slot"])


@pytest.mark.parametrize("Bsz,Hkv,cap,k,nb,retain,partial,dtype,D", [
    (1, 2, 16, 8, 64, 0.8, 0.0, "f32", 64),       # tiny workload shape
    (2, 4, 8, 8, 64, 0.8, 0.0, "bf16", 128),     # capacity = budget
    (2, 4, 128, 128, 2048, 0.8, 0.0, "bf16", 128),  # throughput workload row shape
    (2, 8, 256, 128, 8192, 0.8, 0.2, "bf16", 128),  # host-tier row shape, partial selections
    (1, 3, 37, 20, 100, 0.5, 0.3, "f32", 128),
    (1, 2, 1024, 1024, 4096, 0.9, 0.0, "bf16", 64),  # largest capacity and budget
])
def test_working_set_steps_match_linked_list(Bsz, Hkv, cap, k, nb, retain, partial, dtype, D):
    r = np.random.default_rng(cap * 7 + k)
    rows, T = Bsz * Hkv, nb * 16
    cfg = StepConfig(Bsz, Hkv, Hkv, D, T, dtype, k, cap)
    buf = LayerBuffers(cfg)
    src_k = to_dtype(r.standard_normal((Bsz, Hkv, T, D)), dtype)
    src_v = to_dtype(r.standard_normal((Bsz, Hkv, T, D)), dtype)
    dk, dv = dev(src_k), dev(src_v)
    pool_k = np.zeros((Bsz, Hkv, cap, 16, D), dtype=src_k.dtype)
    pool_v = np.zeros_like(pool_k)
    lru = oracle.LRU(rows, cap)
    chains = _chains(r, rows, nb, k, 8, retain, partial)
    for t in range(8):
        sel, cnt = _pack(chains, t, k)
        buf.sel_blocks.copy_(dev(sel).view(Bsz, Hkv, k))
        buf.sel_count.copy_(dev(cnt).view(Bsz, Hkv))
        log("cache_update", (Bsz, Hkv, cap, k, nb), "step", t)
        buf.cache_update(dk, dv)
        torch.cuda.synchronize()
        out = lru.step(sel, cnt, nb)
        oracle.gather(out["miss_block"], out["miss_slot"], out["miss_count"], src_k, src_v, pool_k, pool_v)
        _compare(buf, out, rows, k)
        np.testing.assert_array_equal(host(buf.slot_block).reshape(rows, cap), lru.slot_block())
        np.testing.assert_array_equal(host(buf.pool_k), pool_k)
        np.testing.assert_array_equal(host(buf.pool_v), pool_v)
    assert np.all(host(buf.clock) == 8)


def test_transfer_count_equals_selection_delta_when_capacity_equals_budget():
    r = np.random.default_rng(5)
    Bsz, Hkv, k, nb = 2, 4, 32, 512
    cfg = StepConfig(Bsz, Hkv, Hkv, 128, nb * 16, "bf16", k, k)
    buf = LayerBuffers(cfg, pool=False)
    chains = _chains(r, Bsz * Hkv, nb, k, 10, 0.8)
    for t in range(10):
        sel, cnt = _pack(chains, t, k)
        buf.sel_blocks.copy_(dev(sel).view(Bsz, Hkv, k))
        buf.sel_count.copy_(dev(cnt).view(Bsz, Hkv))
        log("cache_update list-only step", t)
        buf.cache_update(None, None)  # list only: the no-IO control
        torch.cuda.synchronize()
        mc = host(buf.miss_count).reshape(-1)
        for i in range(Bsz * Hkv):
            prev = set(chains[i][t - 1]) if t else set()
            assert mc[i] == len(set(chains[i][t]) - prev)


def _lists(buf):
    return {f: host(getattr(buf, f)) for f in ("miss_count", "sel_slot", "sel_hit", "miss_block", "miss_slot")}


def _start(buf, table, stamps, clock):
    buf.slot_block.copy_(dev(np.asarray(table, np.int32)).view(buf.slot_block.shape))
    buf.slot_stamp.copy_(dev(np.asarray(stamps, np.int32)).view(buf.slot_stamp.shape))
    buf.clock.copy_(dev(np.asarray(clock, np.int32)).view(buf.clock.shape))


@pytest.mark.parametrize("importance", [False, True])
def test_invalid_rows_match_the_oracle(importance):
    # bad selections and corrupt tables (a selected block held twice, an
    # unselected one held twice, ids out of range) are refused: miss_count
    # -1, padded lists, table, stamps, clock and pool untouched; the valid
    # rows beside them step normally.  Everything against the oracle started
    # from the same table (LRU list ordered by (stamp, block); capped step).
    Bsz, Hkv, cap, k, nb, D = 1, 10, 8, 4, 64, 64
    rows, T = Bsz * Hkv, nb * 16
    r = np.random.default_rng(3 + importance)
    cfg = StepConfig(Bsz, Hkv, Hkv, D, T, "f32", k, cap)
    buf = LayerBuffers(cfg)
    src_k = r.standard_normal((Bsz, Hkv, T, D)).astype(np.float32)
    src_v = r.standard_normal((Bsz, Hkv, T, D)).astype(np.float32)
    base = [1, 5, 9, 12, 30, -1, 40, -1]
    table = np.array([base] * rows, np.int32)
    table[4, 5] = 9      # unselected block 9 held twice
    table[5, 5] = 5      # selected block 5 held twice
    table[6, 7] = nb     # id past the end
    table[7, 5] = -2     # id below -1
    stamps = np.tile(np.array([3, 3, 2, 5, 1, 0, 4, 0], np.int32), (rows, 1))
    clock = np.full(rows, 5, np.int32)
    sel = np.array([[1, 5, 5, 12],      # duplicate selection
                    [3, 2, 7, 8],       # not ascending
                    [0, 1, 2, nb],      # out of range
                    [2, 3, 4, 6],       # count > k (below)
                    [1, 5, 20, 21],     # table: unselected duplicate
                    [1, 5, 20, 21],     # table: selected duplicate
                    [1, 5, 20, 21],     # table: id past the end
                    [1, 5, 20, 21],     # table: id below -1
                    [1, 5, 20, 21],     # valid: two hits, two misses
                    [0, 9, 40, 63]], np.int32)
    cnt = np.array([4, 4, 4, 9, 4, 4, 4, 4, 4, 4], np.int32)
    scores = r.standard_normal((rows, nb)).astype(np.float32)
    pool0 = r.standard_normal((Bsz, Hkv, cap, 16, D)).astype(np.float32)
    _start(buf, table, stamps, clock)
    buf.pool_k.copy_(dev(pool0))
    buf.pool_v.copy_(dev(-pool0))
    buf.sel_blocks.copy_(dev(sel).view(Bsz, Hkv, k))
    buf.sel_count.copy_(dev(cnt).view(Bsz, Hkv))
    buf.scores.copy_(dev(scores).view(Bsz, Hkv, nb))
    log("cache_update invalid rows, importance", importance)
    buf.cache_update(dev(src_k), dev(src_v), importance=importance)
    torch.cuda.synchronize()
    pool_k, pool_v = pool0.copy(), -pool0
    if importance:
        ref_table = table.copy()
        out = oracle.capped_step(ref_table, sel, cnt, scores.astype(np.float64), nb)
        np.testing.assert_array_equal(host(buf.slot_block).reshape(rows, cap), ref_table)
    else:
        lru = oracle.LRU(rows, cap)
        lru.load(table, stamps)
        out = lru.step(sel, cnt, nb)
        assert_lru_state(host(buf.slot_block), host(buf.slot_stamp), lru)
    assert out["miss_count"].tolist() == [-1] * 8 + [2, 2]
    assert_lists(_lists(buf), out, rows, k)
    oracle.gather(out["miss_block"], out["miss_slot"], out["miss_count"], src_k, src_v, pool_k, pool_v)
    np.testing.assert_array_equal(host(buf.pool_k), pool_k)
    np.testing.assert_array_equal(host(buf.pool_v), pool_v)
    # refused rows keep their stamps and clock; valid rows advance once
    st = host(buf.slot_stamp).reshape(rows, cap)
    np.testing.assert_array_equal(st[:8], stamps[:8])
    assert host(buf.clock).reshape(-1).tolist() == [5] * 8 + [6, 6]


def test_attention_after_a_refused_update_reads_nothing():
    # a refused row's padded lists make the separate attention (fetch on
    # attend) skip the row: out 0, lse -inf, its pool unchanged; the oracle
    # attends over an empty selection for it
    w = synth.WORKLOADS["tiny"].scaled(steps=1)
    data = synth.gen_workload(w)
    cfg = StepConfig(w.batch, w.n_q_heads, w.n_kv_heads, w.head_dim, w.ctx, w.dtype, w.k_blocks, w.capacity)
    buf = LayerBuffers(cfg)
    K, V, lens = data["K"], data["V"], data["seq_lens"]
    rows, cap, k, nb = w.rows, w.capacity, w.k_blocks, w.nb_max
    table = np.full((rows, cap), -1, np.int32)
    table[0, :3] = [4, 7, 4]  # row 0: block 4 held twice (not selected below)
    stamps = np.zeros((rows, cap), np.int32)
    sel = np.array([np.arange(10, 10 + k)] * rows, np.int32)
    cnt = np.full(rows, k, np.int32)
    _start(buf, table, stamps, np.zeros(rows, np.int32))
    buf.sel_blocks.copy_(dev(sel).view(buf.sel_blocks.shape))
    buf.sel_count.copy_(dev(cnt).view(buf.sel_count.shape))
    # stale lists from an earlier step must not leak into the attention
    buf.sel_slot.copy_(dev(np.tile(np.arange(k, dtype=np.int32), (rows, 1))).view(buf.sel_slot.shape))
    buf.sel_hit.zero_()
    log("refused update then attention")
    buf.cache_update(None, None)
    buf.attention(dev(data["q"][0]), dev(lens), dev(K), dev(V))
    torch.cuda.synchronize()
    lru = oracle.LRU(rows, cap)
    lru.load(table, stamps)
    out = lru.step(sel, cnt, nb)
    assert out["miss_count"].tolist() == [-1, k]
    assert_lists(_lists(buf), out, rows, k)
    pool_k = np.zeros((w.batch, w.n_kv_heads, cap, 16, w.head_dim), np.float32)
    pool_v = np.zeros_like(pool_k)
    oracle.gather(out["miss_block"], out["miss_slot"], out["miss_count"], K, V, pool_k, pool_v)
    np.testing.assert_array_equal(host(buf.pool_k), pool_k)
    np.testing.assert_array_equal(host(buf.pool_v), pool_v)
    att_cnt = np.where(out["miss_count"] < 0, 0, cnt).reshape(w.batch, w.n_kv_heads)
    o_ref, lse_ref = oracle.attention(data["q"][0], K, V, sel.reshape(w.batch, w.n_kv_heads, k), att_cnt, lens,
                                      1.0 / np.sqrt(w.head_dim))
    assert np.abs(host(buf.out) - o_ref).max() <= 1e-4
    G = w.group
    assert not host(buf.out)[0, :G].any() and np.all(np.isneginf(host(buf.lse)[0, :G]))
    assert np.abs(host(buf.lse)[0, G:] - lse_ref[0, G:]).max() <= 1e-4


def test_flush_refetches_everything():
    r = np.random.default_rng(6)
    Bsz, Hkv, cap, k, nb = 1, 2, 16, 8, 128
    cfg = StepConfig(Bsz, Hkv, Hkv, 128, nb * 16, "bf16", k, cap)
    buf = LayerBuffers(cfg)
    sk = to_dtype(r.standard_normal((Bsz, Hkv, nb * 16, 128)), "bf16")
    sv = to_dtype(r.standard_normal((Bsz, Hkv, nb * 16, 128)), "bf16")
    sel = np.array([[[2, 4, 8, 16, 32, 64, 100, 127]] * 2], dtype=np.int32)
    buf.sel_blocks.copy_(dev(sel))
    buf.sel_count.fill_(8)
    for expect in (8, 0):
        log("cache_update flush test", expect)
        buf.cache_update(dev(sk), dev(sv))
        torch.cuda.synchronize()
        assert host(buf.miss_count).tolist() == [[expect, expect]]
    buf.slot_block.fill_(-1)  # flush
    buf.cache_update(dev(sk), dev(sv))
    torch.cuda.synchronize()
    assert host(buf.miss_count).tolist() == [[8, 8]]
    assert host(buf.sel_slot)[0, 0].tolist() == list(range(8))


@pytest.mark.parametrize("Bsz,Hkv,cap,k,nb,retain,partial,ties", [
    (1, 2, 16, 8, 64, 0.8, 0.0, False),
    (2, 4, 128, 128, 2048, 0.8, 0.0, False),   # throughput workload row shape
    (2, 8, 256, 128, 8192, 0.8, 0.2, True),    # host-tier row shape, partial selections, tied scores
    (1, 3, 37, 20, 100, 0.5, 0.3, True),
])
def test_importance_capped_eviction_matches_oracle(Bsz, Hkv, cap, k, nb, retain, partial, ties):
    # importance-capped eviction (OasisKV summary, key module 3): the same
    # hits and misses, victims by (this step's score, block id); bit-exact
    # against the oracle's capped step given the same selections and scores
    r = np.random.default_rng(cap * 11 + k)
    rows, T, D = Bsz * Hkv, nb * 16, 64
    cfg = StepConfig(Bsz, Hkv, Hkv, D, T, "f32", k, cap)
    buf = LayerBuffers(cfg)
    src_k = r.standard_normal((Bsz, Hkv, T, D)).astype(np.float32)
    src_v = r.standard_normal((Bsz, Hkv, T, D)).astype(np.float32)
    dk, dv = dev(src_k), dev(src_v)
    pool_k = np.zeros((Bsz, Hkv, cap, 16, D), dtype=np.float32)
    pool_v = np.zeros_like(pool_k)
    table = np.full((rows, cap), -1, dtype=np.int32)
    chains = _chains(r, rows, nb, k, 8, retain, partial)
    for t in range(8):
        sel, cnt = _pack(chains, t, k)
        scores = r.standard_normal((rows, nb)).astype(np.float32)
        if ties:
            scores = np.round(scores * 2) / 2
        scores[:, ::17] = -np.inf  # blocks past a row's end score -inf
        buf.sel_blocks.copy_(dev(sel).view(Bsz, Hkv, k))
        buf.sel_count.copy_(dev(cnt).view(Bsz, Hkv))
        buf.scores.copy_(dev(scores).view(Bsz, Hkv, nb))
        log("cache_update importance", (Bsz, Hkv, cap, k, nb), "step", t)
        buf.cache_update(dk, dv, importance=True)
        torch.cuda.synchronize()
        out = oracle.capped_step(table, sel, cnt, scores.astype(np.float64), nb)
        oracle.gather(out["miss_block"], out["miss_slot"], out["miss_count"], src_k, src_v, pool_k, pool_v)
        _compare(buf, out, rows, k)
        np.testing.assert_array_equal(host(buf.slot_block).reshape(rows, cap), table)
        np.testing.assert_array_equal(host(buf.pool_k), pool_k)
        np.testing.assert_array_equal(host(buf.pool_v), pool_v)
    assert np.all(host(buf.clock) == 8)


def test_switching_between_lru_and_importance_eviction():
    # a row can change policy between steps: the state is the same slot table
    r = np.random.default_rng(21)
    Bsz, Hkv, cap, k, nb = 1, 4, 24, 16, 200
    rows = Bsz * Hkv
    cfg = StepConfig(Bsz, Hkv, Hkv, 64, nb * 16, "f32", k, cap)
    buf = LayerBuffers(cfg, pool=False)
    table = np.full((rows, cap), -1, dtype=np.int32)
    chains = _chains(r, rows, nb, k, 6, 0.6)
    replaced = False
    for t in range(6):
        sel, cnt = _pack(chains, t, k)
        scores = r.standard_normal((rows, nb)).astype(np.float32)
        buf.sel_blocks.copy_(dev(sel).view(Bsz, Hkv, k))
        buf.sel_count.copy_(dev(cnt).view(Bsz, Hkv))
        buf.scores.copy_(dev(scores).view(Bsz, Hkv, nb))
        log("policy switch step", t)
        buf.cache_update(None, None, importance=(t % 2 == 1))
        torch.cuda.synchronize()
        if t % 2 == 1:
            before = table.copy()
            out = oracle.capped_step(table, sel, cnt, scores.astype(np.float64), nb)
            _compare(buf, out, rows, k)
            np.testing.assert_array_equal(host(buf.slot_block).reshape(rows, cap), table)
            replaced |= not np.array_equal(table, before)  # the capped steps did evict
        else:  # an LRU step: carry its table into the next capped step
            table = host(buf.slot_block).reshape(rows, cap).copy()
    assert replaced
