"""GPU parity of the lag-1 pipeline: attention at step t over the selection
of step t-1 (step 0 over its own) on the current stream, while step t's
score, top-k and working-set update run on a side stream.

After every step: the top-k bit-exact against the oracle's top-k of the
GPU's own scores, the working-set lists and slot table bit-exact against the
oracle LRU, every resident slot's bytes equal to its source block (except the
misses this step listed, which the next step's attention fetches), and the
output within tolerance of the oracle's attention over the lagged selection.
"""
import math

import numpy as np
import pytest
import torch

import oracle
from top_sparse_kv_block_amd import binding as B
from top_sparse_kv_block_amd import synth
from top_sparse_kv_block_amd.step import Lag1Pipeline, LayerBuffers, StepConfig
from gpu_util import dev, host, log, max_rel_row_err

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("name,kw,heads", [
    ("tiny", dict(steps=5, heavy=0, sigma=0.5), None),
    ("llama8b_32k", dict(batch=2, ctx=4096, budget=512, capacity=64, steps=5), None),
    ("llama8b_32k", dict(batch=3, ctx=2048 + 16 * 7, budget=256, capacity=40, ragged=True, steps=4), None),
    ("quest_128k", dict(batch=2, ctx=8192, capacity=64, steps=4), None),
    # the benchmark's lag-1 shape: full 32K workload with 256 slots; sampled heads
    ("llama8b_32k", dict(capacity=256, steps=3), [(0, 0), (3, 17), (7, 31)]),
])
def test_lag1_pipeline_against_oracle(name, kw, heads):
    w = synth.WORKLOADS[name].scaled(**kw)
    data = synth.gen_workload(w)
    q, sq, K, V, lens = data["q"], data["score_q"], data["K"], data["V"], data["seq_lens"]
    mode = B.SKV_SCORE_QUEST if w.scoring == "quest" else B.SKV_SCORE_BLOCKMAX
    cfg = StepConfig(w.batch, w.n_q_heads, w.n_kv_heads, w.head_dim, w.ctx, w.dtype, w.k_blocks, w.capacity,
                     mode=mode, n_queries=w.n_score_queries, sink=w.sink, recent=w.recent)
    pipe = Lag1Pipeline(LayerBuffers(cfg))
    buf = pipe.buf
    dK, dV, dlens = dev(K), dev(V), dev(lens)
    keys = dK
    if mode == B.SKV_SCORE_QUEST:
        keys = torch.empty(w.batch, w.n_kv_heads, w.nb_max, 2, w.head_dim, dtype=cfg.torch_dtype, device="cuda")
        B.sparse_kv_quest_meta(cfg.shape, dK, dlens, keys)
    scale = 1.0 / math.sqrt(w.head_dim)
    P, k, C = w.rows, w.k_blocks, w.capacity
    lru = oracle.LRU(P, C)
    sels, cnts = [], []
    for t in range(w.steps):
        log("lag-1", name, kw, "step", t)
        pipe.step(dev(q[t]), dev(sq[t]), keys, dlens, dK, dV)
        pipe.join()
        torch.cuda.synchronize()
        cur = pipe.lists[t % 2]
        g_sel, g_cnt = host(cur.sel_blocks), host(cur.sel_count)
        s_sel, s_cnt = oracle.topk(host(buf.scores).astype(np.float64), lens, k, w.ctx, sink=w.sink,
                                   recent=w.recent)
        np.testing.assert_array_equal(g_cnt, s_cnt)
        np.testing.assert_array_equal(g_sel, s_sel)
        sels.append(g_sel)
        cnts.append(g_cnt)
        out = lru.step(g_sel.reshape(P, k), g_cnt.reshape(P), w.nb_max)
        for f in ("sel_slot", "sel_hit", "miss_block", "miss_slot"):
            np.testing.assert_array_equal(host(getattr(cur, f)).reshape(P, k), out[f], f)
        np.testing.assert_array_equal(host(cur.miss_count).reshape(P), out["miss_count"])
        sb = lru.slot_block()
        np.testing.assert_array_equal(host(buf.slot_block).reshape(P, C), sb)
        pk = host(buf.pool_k).reshape(P, C, 16, w.head_dim)
        pv = host(buf.pool_v).reshape(P, C, 16, w.head_dim)
        for r_ in range(P):
            b, j = divmod(r_, w.n_kv_heads)
            pending = set(out["miss_block"][r_, :out["miss_count"][r_]].tolist())
            for s_, blk in enumerate(sb[r_]):
                if blk >= 0 and blk not in pending:
                    assert np.array_equal(pk[r_, s_], K[b, j, 16 * blk:16 * blk + 16]), (t, r_, blk)
                    assert np.array_equal(pv[r_, s_], V[b, j, 16 * blk:16 * blk + 16]), (t, r_, blk)
        a_sel, a_cnt = oracle.lagged(sels)[t], oracle.lagged(cnts)[t]
        np.testing.assert_array_equal(host(pipe.attended().sel_blocks), a_sel)
        g_out = host(buf.out)
        hs = [(b, h) for b in range(w.batch) for h in range(w.n_q_heads)] if heads is None else heads
        for b in sorted({b for b, _ in hs}):
            o_ref, _ = oracle.attention(q[t][b:b + 1], K[b:b + 1], V[b:b + 1], a_sel[b:b + 1], a_cnt[b:b + 1],
                                        lens[b:b + 1], scale)
            hh = [h for bb, h in hs if bb == b]
            if w.dtype == "f32":
                assert np.abs(g_out[b, hh] - o_ref[0, hh]).max() <= 1e-4
            err = max_rel_row_err(g_out[b, hh], o_ref[0, hh])
            assert err <= 1e-4, (b, err)
    # the lag is real: some step attended over a selection other than its own
    assert any(not np.array_equal(sels[t], sels[t - 1]) for t in range(1, w.steps))


def test_lag1_needs_twice_the_budget_in_slots():
    w = synth.WORKLOADS["tiny"]
    cfg = StepConfig(w.batch, w.n_q_heads, w.n_kv_heads, w.head_dim, w.ctx, w.dtype, w.k_blocks, 2 * w.k_blocks - 1)
    with pytest.raises(ValueError):
        Lag1Pipeline(LayerBuffers(cfg))
