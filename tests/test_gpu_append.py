"""GPU parity of the decode-time append (and of decoding while the cache grows).

The append is byte copies plus an exact min/max update, so everything is
compared bit for bit: the grown keys/values and lengths against the oracle's
append, the incrementally kept Quest boxes against boxes recomputed from the
grown cache (by the oracle and by the library's own metadata kernel), and
resident pool slots against their source blocks.  Then whole decode steps run
on a cache that grows by one token per step (Quest scoring, blocks filling up
and new blocks opening), each stage checked against the oracle.
"""
import math

import numpy as np
import pytest
import torch

import oracle
from top_sparse_kv_block_amd import binding as B
from top_sparse_kv_block_amd import synth
from top_sparse_kv_block_amd.step import LayerBuffers, StepConfig
from gpu_util import dev, host, log, max_rel_row_err, to_dtype

pytestmark = pytest.mark.gpu


def _meta_bits(meta64, dtype):
    return to_dtype(meta64, dtype)


@pytest.mark.parametrize("dtype,D", [("bf16", 128), ("f32", 64), ("bf16", 64)])
def test_append_matches_oracle(dtype, D):
    r = np.random.default_rng(3)
    Bsz, Hkv, Hq, T, cap = 5, 2, 8, 256, 6
    rows = Bsz * Hkv
    k = to_dtype(r.standard_normal((Bsz, Hkv, T, D)), dtype)
    v = to_dtype(r.standard_normal((Bsz, Hkv, T, D)), dtype)
    lens = np.array([0, 15, 16, 250, 256], np.int32)  # empty, partial, aligned, near full, full
    cfg = StepConfig(Bsz, Hq, Hkv, D, T, dtype, 4, cap)
    buf = LayerBuffers(cfg)
    # resident blocks include each row's current partial block
    sb = np.full((rows, cap), -1, np.int32)
    for rr in range(rows):
        b = rr // Hkv
        sb[rr, 0] = min(lens[b] // 16, T // 16 - 1)
        sb[rr, 3] = (sb[rr, 0] + 3) % (T // 16)
    pk = np.zeros((Bsz, Hkv, cap, 16, D), k.dtype)
    pv = np.zeros_like(pk)
    for rr in range(rows):
        b, j = divmod(rr, Hkv)
        for s, blk in enumerate(sb[rr]):
            if blk >= 0:
                pk[b, j, s] = k[b, j, 16 * blk:16 * blk + 16]
                pv[b, j, s] = v[b, j, 16 * blk:16 * blk + 16]
    buf.slot_block.copy_(dev(sb).view(Bsz, Hkv, cap))
    buf.pool_k.copy_(dev(pk))
    buf.pool_v.copy_(dev(pv))
    dk, dv, dl = dev(k), dev(v), dev(lens)
    meta = torch.empty(Bsz, Hkv, T // 16, 2, D, dtype=cfg.torch_dtype, device="cuda")
    B.sparse_kv_quest_meta(cfg.shape, dk, dl, meta)
    for step in range(40):
        nk = to_dtype(r.standard_normal((Bsz, Hkv, D)), dtype)
        nv = to_dtype(r.standard_normal((Bsz, Hkv, D)), dtype)
        log("append", dtype, D, "step", step)
        buf.append(dev(nk), dev(nv), dl, dk, dv, meta)
        oracle.append(nk, nv, lens, k, v, sb, pk, pv)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(host(dl), lens)
    np.testing.assert_array_equal(host(dk), k)
    np.testing.assert_array_equal(host(dv), v)
    np.testing.assert_array_equal(host(buf.pool_k), pk)
    np.testing.assert_array_equal(host(buf.pool_v), pv)
    got_meta = host(meta)
    np.testing.assert_array_equal(got_meta, _meta_bits(oracle.quest_meta(k, lens), dtype))
    fresh = torch.empty_like(meta)
    B.sparse_kv_quest_meta(cfg.shape, dk, dl, fresh)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(got_meta, host(fresh))


def test_decoding_while_the_cache_grows():
    # Quest-scored steps with one new token per step: lengths cross block
    # boundaries, new blocks open with a one-token box, the working set keeps
    # fresh copies of partial blocks, attention sees the new tokens
    w = synth.WORKLOADS["quest_128k"].scaled(batch=2, ctx=2048, budget=256, capacity=24, steps=1)
    T = 2048 + 64
    r = np.random.default_rng(8)
    data = synth.gen_workload(w)
    k = np.zeros((w.batch, w.n_kv_heads, T, w.head_dim), np.uint16)
    v = np.zeros_like(k)
    k[:, :, :2048], v[:, :, :2048] = data["K"], data["V"]
    lens = np.array([2048 - 5, 2048 - 30], np.int32)
    cfg = StepConfig(w.batch, w.n_q_heads, w.n_kv_heads, w.head_dim, T, "bf16", w.k_blocks, w.capacity,
                     mode=B.SKV_SCORE_QUEST, sink=w.sink, recent=w.recent)
    buf = LayerBuffers(cfg)
    dk, dv, dl = dev(k), dev(v), dev(lens)
    meta = torch.empty(w.batch, w.n_kv_heads, T // 16, 2, w.head_dim, dtype=torch.bfloat16, device="cuda")
    B.sparse_kv_quest_meta(cfg.shape, dk, dl, meta)
    lru = oracle.LRU(w.rows, w.capacity)
    scale = 1.0 / math.sqrt(w.head_dim)
    P, nb = w.rows, T // 16
    for step in range(24):
        nk = to_dtype(r.standard_normal((w.batch, w.n_kv_heads, w.head_dim)), "bf16")
        nv = to_dtype(r.standard_normal((w.batch, w.n_kv_heads, w.head_dim)), "bf16")
        q = to_dtype(r.standard_normal((w.batch, w.n_q_heads, w.head_dim)), "bf16")
        log("grow + step", step, "lens", lens.tolist())
        buf.append(dev(nk), dev(nv), dl, dk, dv, meta)
        oracle.append(nk, nv, lens, k, v)
        buf.score(dev(q)[:, None], meta, dl)
        buf.select_attend(dev(q), dl, dk, dv)
        torch.cuda.synchronize()
        np.testing.assert_array_equal(host(dl), lens)
        # scores: Quest bound from the oracle's recomputed boxes (fp32 accumulation bound)
        meta_ref = oracle.quest_meta(k, lens)
        ref = oracle.score_quest(q[:, None], meta_ref, lens, scale, T=T)
        got = host(buf.scores).astype(np.float64)
        fin = np.isfinite(ref)
        assert np.array_equal(fin, np.isfinite(got))
        assert np.abs(got[fin] - ref[fin]).max() <= 1e-3 * max(1.0, np.abs(ref[fin]).max())
        # top-k exact on the GPU's scores, working set exact on the GPU's selection
        g_sel, g_cnt = host(buf.sel_blocks), host(buf.sel_count)
        s_sel, s_cnt = oracle.topk(got, lens, w.k_blocks, T, sink=w.sink, recent=w.recent)
        np.testing.assert_array_equal(g_sel, s_sel)
        np.testing.assert_array_equal(g_cnt, s_cnt)
        out = lru.step(g_sel.reshape(P, -1), g_cnt.reshape(P), nb)
        np.testing.assert_array_equal(host(buf.miss_count).reshape(P), out["miss_count"])
        np.testing.assert_array_equal(host(buf.sel_slot).reshape(P, -1), out["sel_slot"])
        # every resident slot holds its (possibly grown) block
        pk, pv = host(buf.pool_k).reshape(P, w.capacity, 16, w.head_dim), host(buf.pool_v).reshape(
            P, w.capacity, 16, w.head_dim)
        for rr, row in enumerate(lru.slot_block()):
            b, j = divmod(rr, w.n_kv_heads)
            for s_, blk in enumerate(row):
                if blk >= 0:
                    assert np.array_equal(pk[rr, s_], k[b, j, 16 * blk:16 * blk + 16])
                    assert np.array_equal(pv[rr, s_], v[b, j, 16 * blk:16 * blk + 16])
        o_ref, _ = oracle.attention(q, k, v, g_sel, g_cnt, lens, scale)
        err = max_rel_row_err(host(buf.out), o_ref)
        assert err <= 2e-2 and err <= 1e-4, err


@pytest.mark.timeout(400)
def test_growth_full_size_sampled():
    # the benchmark's growth shape: the 32K workload (8 x 8 rows) with every
    # sequence full at 32768 tokens and room for more; each step appends one
    # token per sequence, then scores (exact block max) and runs the fused
    # call, so the rows pass 2048 blocks.  Checked: lengths and appended rows,
    # sampled score rows, every row of top-k and of the working set, sampled
    # attention heads
    w = synth.WORKLOADS["llama8b_32k"].scaled(steps=1)
    room = 48
    T = w.ctx + room
    r = np.random.default_rng(11)
    data = synth.gen_workload(w)
    k = np.zeros((w.batch, w.n_kv_heads, T, w.head_dim), np.uint16)
    v = np.zeros_like(k)
    k[:, :, :w.ctx], v[:, :, :w.ctx] = data["K"], data["V"]
    lens = data["seq_lens"].copy()
    cfg = StepConfig(w.batch, w.n_q_heads, w.n_kv_heads, w.head_dim, T, "bf16", w.k_blocks, w.capacity)
    buf = LayerBuffers(cfg)
    dk, dv, dl = dev(k), dev(v), dev(lens)
    lru = oracle.LRU(w.rows, w.capacity)
    scale = 1.0 / math.sqrt(w.head_dim)
    P, nb = w.rows, T // 16
    rows, heads = [0, 37, 63], [(0, 0), (4, 18), (7, 31)]
    for step in range(4):
        nk = to_dtype(r.standard_normal((w.batch, w.n_kv_heads, w.head_dim)), "bf16")
        nv = to_dtype(r.standard_normal((w.batch, w.n_kv_heads, w.head_dim)), "bf16")
        q = to_dtype(r.standard_normal((w.batch, w.n_q_heads, w.head_dim)), "bf16")
        log("full-size growth step", step, "len", int(lens[0]))
        buf.append(dev(nk), dev(nv), dl, dk, dv)
        oracle.append(nk, nv, lens, k, v)
        buf.score(dev(q)[:, None], dk, dl)
        buf.select_attend(dev(q), dl, dk, dv)
        torch.cuda.synchronize()
        np.testing.assert_array_equal(host(dl), lens)
        got = host(buf.scores).astype(np.float64)
        for rr in rows:
            b, j = divmod(rr, w.n_kv_heads)
            G = w.group
            np.testing.assert_array_equal(host(dk[b, j, lens[b] - 1]), k[b, j, lens[b] - 1])
            ref = oracle.score_blockmax(np.ascontiguousarray(q[b:b + 1, None, j * G:(j + 1) * G]),
                                        np.ascontiguousarray(k[b:b + 1, j:j + 1]), lens[b:b + 1], scale)[0, 0]
            fin = np.isfinite(ref)
            assert np.array_equal(fin, np.isfinite(got[b, j]))
            assert np.abs(got[b, j][fin] - ref[fin]).max() <= 1e-3 * max(1.0, np.abs(ref[fin]).max())
        g_sel, g_cnt = host(buf.sel_blocks), host(buf.sel_count)
        s_sel, s_cnt = oracle.topk(got, lens, w.k_blocks, T)
        np.testing.assert_array_equal(g_sel, s_sel)
        np.testing.assert_array_equal(g_cnt, s_cnt)
        out = lru.step(g_sel.reshape(P, -1), g_cnt.reshape(P), nb)
        for f in ("sel_slot", "sel_hit", "miss_block", "miss_slot"):
            np.testing.assert_array_equal(host(getattr(buf, f)).reshape(P, -1), out[f], f)
        np.testing.assert_array_equal(host(buf.slot_block).reshape(P, -1), lru.slot_block())
        g_out = host(buf.out)
        for b in sorted({b for b, _ in heads}):
            o_ref, _ = oracle.attention(q[b:b + 1], k[b:b + 1], v[b:b + 1], g_sel[b:b + 1], g_cnt[b:b + 1],
                                        lens[b:b + 1], scale)
            hh = [h for bb, h in heads if bb == b]
            assert max_rel_row_err(g_out[b, hh], o_ref[0, hh]) <= 1e-4
    assert lens.min() == w.ctx + 4 and nb_of_len(lens.min()) > 2048


def nb_of_len(n):
    return (int(n) + 15) // 16
