"""The fused select -> update -> attend call equals the three separate calls
(top-k, list-only working-set update, attention with fetch on attend) bit for
bit, step after step, and equals the oracle through the step tests."""
import numpy as np
import pytest
import torch

import oracle
from top_sparse_kv_block_amd import binding as B
from top_sparse_kv_block_amd import synth
from top_sparse_kv_block_amd.step import LayerBuffers, StepConfig, decode_step
from gpu_util import assert_lists, assert_lru_state, dev, host, log

pytestmark = pytest.mark.gpu

FIELDS = ("out", "lse", "sel_blocks", "sel_count", "slot_block", "slot_stamp", "clock", "sel_slot", "sel_hit",
          "miss_block", "miss_slot", "miss_count", "pool_k", "pool_v")


@pytest.mark.parametrize("name,kw,steps,splits", [
    ("tiny", {}, 4, 0),
    ("tiny", dict(capacity=8), 4, 0),
    ("llama8b_32k", dict(batch=2, ctx=4096, budget=512), 6, 0),
    ("llama8b_32k", dict(batch=2, ctx=4096, budget=512), 4, 5),
    ("llama8b_32k", dict(batch=2, ctx=4096, budget=512), 3, 32),
    # one split per row: the fused kernel writes the output and commits the
    # plan itself (no merge launch)
    ("llama8b_32k", dict(batch=2, ctx=4096, budget=512), 4, 1),
    ("quest_128k", dict(batch=2, ctx=8192), 4, 1),
    ("lookahead_1m", dict(ctx=16 * 20000), 3, 1),
    ("llama8b_32k", dict(batch=3, ctx=2048 + 16 * 7, budget=256, capacity=40, ragged=True), 4, 0),
    ("quest_128k", dict(batch=2, ctx=8192), 4, 0),
    # rows just past 2048 and 4096 blocks: the 8- and 16-keys-per-thread variants
    ("llama8b_32k", dict(batch=1, ctx=32768 + 16 * 5, budget=2048), 3, 0),
    ("quest_128k", dict(batch=1, ctx=65536 + 16 * 3), 3, 0),
    # the largest budget and working set (1024 blocks of 1024 slots), and the largest GQA group (16)
    ("llama8b_32k", dict(batch=1, ctx=65536, budget=16384, capacity=1024), 2, 0),
    ("llama8b_32k", dict(batch=2, n_kv_heads=2, ctx=4096, budget=512), 3, 0),
    # bf16 with D = 64, float32 with D = 128, and one head per group (MHA)
    ("llama8b_32k", dict(batch=2, head_dim=64, ctx=4096, budget=512), 3, 0),
    ("tiny", dict(head_dim=128), 3, 0),
    ("llama8b_32k", dict(batch=2, n_q_heads=8, ctx=4096, budget=512), 3, 0),
    ("lookahead_1m", dict(ctx=16384), 3, 0),
    # rows past 8192 blocks (32 keys per thread) and past 16384 (the top-k's
    # chunk launch, then every workgroup selects from the candidates): Quest
    # grown past 128K with sink / recent, ragged rows of 20000 blocks, the
    # 1M-context rows of 65536 blocks
    ("quest_128k", dict(batch=1, ctx=131072 + 16 * 3), 3, 0),
    ("llama8b_32k", dict(batch=3, ctx=16 * 20000, budget=1024, capacity=100, ragged=True), 3, 0),
    ("quest_128k", dict(batch=2, n_kv_heads=2, n_q_heads=8, ctx=16 * 40000 + 5 * 16), 3, 0),
    ("lookahead_1m", {}, 2, 0),
    # the largest budget over 40000 blocks: 4096-block chunks, 10240
    # candidates per row (32 per thread in the selection)
    ("lookahead_1m", dict(n_kv_heads=2, n_q_heads=16, ctx=16 * 40000, budget=16 * 1024, capacity=1024), 2, 0),
])
def test_fused_equals_separate_calls(name, kw, steps, splits):
    w = synth.WORKLOADS[name].scaled(steps=steps, **kw)
    data = synth.gen_workload(w)
    mode = B.SKV_SCORE_QUEST if w.scoring == "quest" else B.SKV_SCORE_BLOCKMAX
    shape = B.make_shape(w.batch, w.n_q_heads, w.n_kv_heads, w.head_dim, w.ctx, w.dtype)
    # equal split counts on both paths (each call's own default differs)
    splits = splits or B.sparse_kv_select_attend_splits(shape, w.k_blocks)
    cfg = StepConfig(w.batch, w.n_q_heads, w.n_kv_heads, w.head_dim, w.ctx, w.dtype, w.k_blocks, w.capacity,
                     mode=mode, n_queries=w.n_score_queries, sink=w.sink, recent=w.recent, num_splits=splits)
    a, b = LayerBuffers(cfg), LayerBuffers(cfg)
    K, V, lens = dev(data["K"]), dev(data["V"]), dev(data["seq_lens"])
    keys = K
    if mode == B.SKV_SCORE_QUEST:
        keys = torch.empty(w.batch, w.n_kv_heads, w.nb_max, 2, w.head_dim, dtype=cfg.torch_dtype, device="cuda")
        B.sparse_kv_quest_meta(cfg.shape, K, lens, keys)
    for t in range(steps):
        log("fused vs separate", name, kw, "step", t)
        q, sq = dev(data["q"][t]), dev(data["score_q"][t])
        decode_step(a, q, sq, keys, lens, K, V, fused=False)
        decode_step(b, q, sq, keys, lens, K, V, fused=True)
        torch.cuda.synchronize()
        for f in FIELDS:
            np.testing.assert_array_equal(host(getattr(b, f)), host(getattr(a, f)), err_msg=f"{f} at step {t}")


def test_fused_refuses_corrupt_tables():
    # row 0's table holds an id past the end, row 1's an unselected block
    # twice: both are refused (miss_count -1, padded lists, table, stamps and
    # clock untouched, out 0, lse -inf).  Against the oracle: its top-k of
    # the step's scores, its list started from the same table, its attention
    # (an empty selection for a refused row).
    w = synth.WORKLOADS["tiny"].scaled(batch=2, steps=1)
    data = synth.gen_workload(w)
    cfg = StepConfig(w.batch, w.n_q_heads, w.n_kv_heads, w.head_dim, w.ctx, w.dtype, w.k_blocks, w.capacity)
    buf = LayerBuffers(cfg)
    K, V, lens = data["K"], data["V"], data["seq_lens"]
    rows, cap, k, nb = w.rows, w.capacity, w.k_blocks, w.nb_max
    table = np.full((rows, cap), -1, dtype=np.int32)
    table[0, :2] = [5, nb + 3]
    table[1, 2:5] = [nb - 1, 6, nb - 1]
    stamps = np.tile(np.arange(cap, dtype=np.int32), (rows, 1))
    buf.slot_block.copy_(dev(table).view(buf.slot_block.shape))
    buf.slot_stamp.copy_(dev(stamps).view(buf.slot_stamp.shape))
    log("fused corrupt tables")
    decode_step(buf, dev(data["q"][0]), dev(data["score_q"][0]), dev(K), dev(lens), dev(K), dev(V), fused=True)
    torch.cuda.synchronize()
    # the top-k decision in the kernel's precision (its fp32 scores); the
    # selection must then avoid block nb - 1 for row 1's refusal to be about
    # an unselected duplicate
    o_sel, o_cnt = oracle.topk(host(buf.scores).astype(np.float64), lens, k, w.ctx)
    np.testing.assert_array_equal(host(buf.sel_blocks), o_sel)
    np.testing.assert_array_equal(host(buf.sel_count), o_cnt)
    assert nb - 1 not in o_sel.reshape(rows, k)[1].tolist()
    lru = oracle.LRU(rows, cap)
    lru.load(table, stamps)
    out = lru.step(o_sel.reshape(rows, k), o_cnt.reshape(rows), nb)
    assert out["miss_count"].tolist()[:2] == [-1, -1] and (out["miss_count"][2:] == k).all()
    assert_lists({f: host(getattr(buf, f)) for f in FIELDS[7:12]}, out, rows, k)
    assert_lru_state(host(buf.slot_block), host(buf.slot_stamp), lru)
    np.testing.assert_array_equal(host(buf.slot_stamp).reshape(rows, cap)[:2], stamps[:2])
    assert host(buf.clock).reshape(-1).tolist() == [0, 0] + [1] * (rows - 2)
    att_cnt = np.where(out["miss_count"] < 0, 0, o_cnt.reshape(-1)).reshape(o_cnt.shape)
    o_ref, lse_ref = oracle.attention(data["q"][0], K, V, o_sel, att_cnt, lens, 1.0 / np.sqrt(w.head_dim))
    assert np.abs(host(buf.out) - o_ref).max() <= 1e-4
    G = w.group
    out_rows, lse_rows = host(buf.out).reshape(rows, G, -1), host(buf.lse).reshape(rows, G)
    assert not out_rows[:2].any() and np.all(np.isneginf(lse_rows[:2]))
    assert np.abs(lse_rows[2:] - lse_ref.reshape(rows, G)[2:]).max() <= 1e-4
    pool_k = np.zeros((w.batch, w.n_kv_heads, cap, 16, w.head_dim), np.float32)
    pool_v = np.zeros_like(pool_k)
    oracle.gather(out["miss_block"], out["miss_slot"], out["miss_count"], K, V, pool_k, pool_v)
    np.testing.assert_array_equal(host(buf.pool_k), pool_k)
    np.testing.assert_array_equal(host(buf.pool_v), pool_v)


@pytest.mark.parametrize("capacity,ctx", [(32, 4096), (48, 4096), (40, 16 * 20000)])
def test_fused_rows_shorter_than_the_budget(capacity, ctx):
    """Rows with at most k valid blocks take every valid block without
    reading their scores; an empty row selects and attends nothing.  Lengths:
    full, a partial 5-block row, empty, exactly k blocks; also with rows
    allocated past 16384 blocks (the chunk launch skips such rows)."""
    w = synth.WORKLOADS["llama8b_32k"].scaled(batch=4, ctx=ctx, budget=512, capacity=capacity, steps=3)
    data = synth.gen_workload(w)
    lens_np = np.array([w.ctx, 16 * 5 - 3, 0, 16 * w.k_blocks], dtype=np.int32)
    splits = B.sparse_kv_select_attend_splits(B.make_shape(w.batch, w.n_q_heads, w.n_kv_heads, w.head_dim, w.ctx,
                                                           w.dtype), w.k_blocks)
    cfg = StepConfig(w.batch, w.n_q_heads, w.n_kv_heads, w.head_dim, w.ctx, w.dtype, w.k_blocks, w.capacity,
                     num_splits=splits)
    a, b = LayerBuffers(cfg), LayerBuffers(cfg)
    K, V, lens = dev(data["K"]), dev(data["V"]), dev(lens_np)
    for t in range(w.steps):
        log("fused vs separate, short rows", capacity, "step", t)
        q, sq = dev(data["q"][t]), dev(data["score_q"][t])
        decode_step(a, q, sq, K, lens, K, V, fused=False)
        decode_step(b, q, sq, K, lens, K, V, fused=True)
        torch.cuda.synchronize()
        for f in FIELDS:
            np.testing.assert_array_equal(host(getattr(b, f)), host(getattr(a, f)), err_msg=f"{f} at step {t}")
    counts = host(b.sel_count).reshape(w.batch, w.n_kv_heads)
    assert (counts[1] == 5).all() and (counts[2] == 0).all() and (counts[3] == w.k_blocks).all()
    assert not host(b.out)[2].any() and np.all(np.isneginf(host(b.lse)[2]))
