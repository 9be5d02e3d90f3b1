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
from top_sparse_kv_block_amd.step import LayerBuffers, StepConfig
from gpu_util import dev, host, log, to_dtype

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


def test_invalid_rows_are_flagged_and_left_untouched():
    Bsz, Hkv, cap, k, nb = 1, 4, 8, 4, 64
    cfg = StepConfig(Bsz, Hkv, Hkv, 64, nb * 16, "f32", k, cap)
    buf = LayerBuffers(cfg, pool=False)
    good = np.array([[1, 5, 9, 12]] * 4, dtype=np.int32)
    buf.sel_blocks.copy_(dev(good).view(1, 4, k))
    buf.sel_count.fill_(4)
    log("cache_update warm-up")
    buf.cache_update(None, None)
    torch.cuda.synchronize()
    before = host(buf.slot_block).copy()
    stamps = host(buf.slot_stamp).copy()
    bad = np.array([[1, 5, 5, 12],      # duplicate
                    [3, 2, 7, 8],       # not ascending
                    [0, 1, 2, 64],      # out of range (NB = 64)
                    [2, 3, 4, 6]], dtype=np.int32)
    cnt = np.array([4, 4, 4, 9], dtype=np.int32)  # last row: count > k
    buf.sel_blocks.copy_(dev(bad).view(1, 4, k))
    buf.sel_count.copy_(dev(cnt).view(1, 4))
    log("cache_update invalid rows")
    buf.cache_update(None, None)
    torch.cuda.synchronize()
    assert host(buf.miss_count).tolist() == [[-1, -1, -1, -1]]
    np.testing.assert_array_equal(host(buf.slot_block), before)
    np.testing.assert_array_equal(host(buf.slot_stamp), stamps)


def test_corrupt_slot_table_is_flagged():
    Bsz, Hkv, cap, k, nb = 1, 2, 4, 2, 32
    cfg = StepConfig(Bsz, Hkv, Hkv, 64, nb * 16, "f32", k, cap)
    buf = LayerBuffers(cfg, pool=False)
    buf.slot_block.copy_(dev(np.array([[[3, 3, -1, -1], [1, 99, -1, -1]]], dtype=np.int32)))
    buf.sel_blocks.copy_(dev(np.array([[[3, 4], [1, 2]]], dtype=np.int32)))
    buf.sel_count.fill_(2)
    log("cache_update corrupt table")
    buf.cache_update(None, None)
    torch.cuda.synchronize()
    assert host(buf.miss_count).tolist() == [[-1, -1]]


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
