"""GPU parity of the one-launch selection (sparse_kv_select): top-k and the
LRU working-set update in one workgroup per row must give exactly what the
two calls give in sequence (sparse_kv_topk, then sparse_kv_cache_update):
selection, lists, slot table, stamps, clock and, with a source, the pool.

Scores are seeded random rows that drift from step to step (so hits, misses
and evictions all occur), at row lengths covering each launch shape: up to
8192 blocks (512 threads), up to 16384 (1024 threads) and the two-launch
long-row selection beyond (chunk candidates, then selection and update), with
ragged lengths, forced sink / recent blocks and a working
set larger than the budget.
"""
import numpy as np
import pytest
import torch

import oracle
from top_sparse_kv_block_amd import binding as B
from gpu_util import assert_lists, assert_lru_state, dev, host, log

pytestmark = pytest.mark.gpu

FIELDS = ("sel_blocks", "sel_count", "sel_slot", "sel_hit", "miss_block", "miss_slot", "miss_count")


def _state(P, k, C, device="cuda"):
    i32 = dict(dtype=torch.int32, device=device)
    return dict(sel_blocks=torch.empty(P, k, **i32), sel_count=torch.empty(P, **i32),
                slot_block=torch.full((P, C), -1, **i32), slot_stamp=torch.zeros(P, C, **i32),
                clock=torch.zeros(P, **i32), sel_slot=torch.empty(P, k, **i32),
                sel_hit=torch.empty(P, k, dtype=torch.uint8, device=device), miss_block=torch.empty(P, k, **i32),
                miss_slot=torch.empty(P, k, **i32), miss_count=torch.empty(P, **i32))


@pytest.mark.parametrize("B_,Hkv,T,k,C,sink,recent,steps", [
    (2, 4, 16 * 2048, 128, 128, 0, 0, 4),         # 2048 blocks, C = k
    (3, 2, 16 * 8192, 32, 48, 64, 128, 4),        # 8192 blocks with forced blocks, C > k
    (1, 3, 16 * 12000, 64, 64, 16, 16, 3),        # 1024 threads
    (1, 2, 16 * 40000, 128, 160, 0, 256, 3),      # long rows: 1024-block chunks, 5120 candidates
    (1, 2, 16 * 65536, 1024, 1024, 32, 0, 2),     # 4096-block chunks, 16384 candidates, C = k = 1024
])
def test_select_equals_topk_then_update(B_, Hkv, T, k, C, sink, recent, steps):
    rng = np.random.default_rng(T + k)
    P, NB, D = B_ * Hkv, T // 16, 64
    shape = B.make_shape(B_, 4 * Hkv, Hkv, D, T, "f32")
    lens = rng.integers(T // 2, T + 1, size=B_).astype(np.int32)
    lens[0] = T
    dl = dev(lens)
    K = torch.randn(B_, Hkv, T, D, device="cuda")
    V = torch.randn(B_, Hkv, T, D, device="cuda")
    a, b = _state(P, k, C), _state(P, k, C)
    pa = [torch.zeros(P, C, 16, D, device="cuda") for _ in range(2)]
    pb = [torch.zeros(P, C, 16, D, device="cuda") for _ in range(2)]
    wsb = B.sparse_kv_topk_workspace_bytes(shape, k)
    ws = [torch.empty(wsb, dtype=torch.uint8, device="cuda") if wsb else None for _ in range(2)]
    base = rng.standard_normal((P, NB)).astype(np.float32)
    for t in range(steps):
        sc = dev((base + 0.3 * rng.standard_normal((P, NB))).astype(np.float32))
        log("select", (B_, Hkv, T, k, C, sink, recent), "step", t)
        B.sparse_kv_topk(shape, sc, dl, k, sink, recent, a["sel_blocks"], a["sel_count"], ws[0])
        B.sparse_kv_cache_update(shape, k, C, a["sel_blocks"], a["sel_count"], a["slot_block"], a["slot_stamp"],
                                 a["clock"], a["sel_slot"], a["sel_hit"], a["miss_block"], a["miss_slot"],
                                 a["miss_count"], K, V, B.SKV_SRC_DEVICE, pa[0], pa[1])
        B.sparse_kv_select(shape, sc, dl, k, sink, recent, C, b["sel_blocks"], b["sel_count"], b["slot_block"],
                           b["slot_stamp"], b["clock"], b["sel_slot"], b["sel_hit"], b["miss_block"], b["miss_slot"],
                           b["miss_count"], K, V, B.SKV_SRC_DEVICE, pb[0], pb[1], ws[1])
        torch.cuda.synchronize()
        for f in FIELDS + ("slot_block", "slot_stamp", "clock"):
            np.testing.assert_array_equal(host(b[f]), host(a[f]), err_msg=f"{f} at step {t}")
        for x, y in zip(pa, pb):
            assert torch.equal(x, y)
        # the selection itself against the oracle (the kernels' fp32 scores)
        o_sel, o_cnt = oracle.topk(host(sc).reshape(B_, Hkv, NB).astype(np.float64), lens, k, T, sink=sink,
                                   recent=recent)
        np.testing.assert_array_equal(host(b["sel_blocks"]).reshape(o_sel.shape), o_sel)
        np.testing.assert_array_equal(host(b["sel_count"]).reshape(o_cnt.shape), o_cnt)
        if t > 0:
            m = host(b["miss_count"])
            assert 0 < m.sum() < host(b["sel_count"]).sum()


def test_select_lists_only_and_corrupt_tables():
    # rows whose table holds an id past the end, an unselected block twice
    # and a selected block twice are refused (miss_count -1, padded lists,
    # table, stamps and clock untouched); the selection itself is still
    # written.  Against the oracle's top-k of the same scores and its list
    # started from the same table.
    B_, Hkv, NB, k, C = 2, 2, 1024, 16, 16
    P, T = B_ * Hkv, 16 * NB
    shape = B.make_shape(B_, 4 * Hkv, Hkv, 64, T, "f32")
    scores = np.random.default_rng(0).standard_normal((P, NB)).astype(np.float32)
    lens = np.array([T, T], np.int32)
    o_sel, o_cnt = oracle.topk(scores.reshape(B_, Hkv, NB).astype(np.float64), lens, k, T)
    o_sel, o_cnt = o_sel.reshape(P, k), o_cnt.reshape(P)
    unselected = [b for b in range(NB) if b not in set(o_sel[1].tolist())][:1] * 2
    table = np.full((P, C), -1, np.int32)
    table[0, :2] = [5, NB + 3]                # an id past the end
    table[1, 3:5] = unselected                # an unselected block twice
    table[2, [1, 6]] = o_sel[2, 3]            # a selected block twice
    table[3, :3] = [o_sel[3, 0], 7, o_sel[3, 5]]  # valid
    stamps = np.tile(np.arange(C, dtype=np.int32)[::-1].copy(), (P, 1))
    s = _state(P, k, C)
    s["slot_block"].copy_(dev(table))
    s["slot_stamp"].copy_(dev(stamps))
    log("select corrupt tables")
    B.sparse_kv_select(shape, dev(scores), dev(lens), k, 0, 0, C, s["sel_blocks"], s["sel_count"],
                       s["slot_block"], s["slot_stamp"], s["clock"], s["sel_slot"], s["sel_hit"], s["miss_block"],
                       s["miss_slot"], s["miss_count"])
    torch.cuda.synchronize()
    np.testing.assert_array_equal(host(s["sel_blocks"]), o_sel)
    np.testing.assert_array_equal(host(s["sel_count"]), o_cnt)
    lru = oracle.LRU(P, C)
    lru.load(table, stamps)
    out = lru.step(o_sel, o_cnt, NB)
    assert out["miss_count"].tolist()[:3] == [-1, -1, -1] and out["miss_count"][3] == k - 2
    assert_lists({f: host(s[f]) for f in FIELDS}, out, P, k)
    assert_lru_state(host(s["slot_block"]), host(s["slot_stamp"]), lru)
    np.testing.assert_array_equal(host(s["slot_stamp"])[:3], stamps[:3])
    assert host(s["clock"]).tolist() == [0, 0, 0, 1]


@pytest.mark.parametrize("sink,recent", [(0, 0), (16, 48)])
def test_select_rows_shorter_than_the_budget(sink, recent):
    """Rows with at most k valid blocks (take-all, no score reads), a partial
    5-block row, an empty row and a row of exactly k blocks, C > k."""
    B_, Hkv, T, k, C, D = 4, 2, 16 * 1024, 32, 40, 64
    P, NB = B_ * Hkv, T // 16
    rng = np.random.default_rng(7 + sink)
    shape = B.make_shape(B_, 4 * Hkv, Hkv, D, T, "f32")
    dl = dev(np.array([T, 16 * 5 - 3, 0, 16 * k], dtype=np.int32))
    K = torch.randn(B_, Hkv, T, D, device="cuda")
    V = torch.randn(B_, Hkv, T, D, device="cuda")
    a, b = _state(P, k, C), _state(P, k, C)
    pa = [torch.zeros(P, C, 16, D, device="cuda") for _ in range(2)]
    pb = [torch.zeros(P, C, 16, D, device="cuda") for _ in range(2)]
    base = rng.standard_normal((P, NB)).astype(np.float32)
    for t in range(3):
        sc = dev((base + 0.3 * rng.standard_normal((P, NB))).astype(np.float32))
        log("select short rows", (sink, recent), "step", t)
        B.sparse_kv_topk(shape, sc, dl, k, sink, recent, a["sel_blocks"], a["sel_count"])
        B.sparse_kv_cache_update(shape, k, C, a["sel_blocks"], a["sel_count"], a["slot_block"], a["slot_stamp"],
                                 a["clock"], a["sel_slot"], a["sel_hit"], a["miss_block"], a["miss_slot"],
                                 a["miss_count"], K, V, B.SKV_SRC_DEVICE, pa[0], pa[1])
        B.sparse_kv_select(shape, sc, dl, k, sink, recent, C, b["sel_blocks"], b["sel_count"], b["slot_block"],
                           b["slot_stamp"], b["clock"], b["sel_slot"], b["sel_hit"], b["miss_block"], b["miss_slot"],
                           b["miss_count"], K, V, B.SKV_SRC_DEVICE, pb[0], pb[1])
        torch.cuda.synchronize()
        for f in FIELDS + ("slot_block", "slot_stamp", "clock"):
            np.testing.assert_array_equal(host(b[f]), host(a[f]), err_msg=f"{f} at step {t}")
        for x, y in zip(pa, pb):
            assert torch.equal(x, y)
    counts = host(b["sel_count"]).reshape(B_, Hkv)
    assert (counts[1] == 5).all() and (counts[2] == 0).all() and (counts[3] == k).all()
