"""Whole decode steps on the GPU against the oracle, step by step.

Each step runs the four library calls; the oracle then checks every stage:
scores within the fp32 accumulation bound, the top-k set bit-exact against
the oracle's top-k of the GPU's own float32 scores and within the 1e-5
swap tolerance against the oracle's fp64 scores, the working set bit-exact
given the GPU's selection, the pool bytes, and the attention output within
tolerance (computed by the oracle straight from the source K/V).
"""
import math

import numpy as np
import pytest
import torch

import oracle
from top_sparse_kv_block_amd import binding as B
from top_sparse_kv_block_amd import synth
from top_sparse_kv_block_amd.step import LayerBuffers, StepConfig, decode_step
from gpu_util import assert_lru_state, dev, host, log, max_rel_row_err, topk_swaps_ok

pytestmark = pytest.mark.gpu

GAMMA = 16 * 2.0 ** -24


def _abs(a):
    return (a & np.uint16(0x7FFF)) if a.dtype == np.uint16 else np.abs(a)


def _forced_sets(w, lens):
    out = []
    for b in range(w.batch):
        L = int(lens[b])
        nv = -(-L // 16)
        f = set()
        if nv > w.k_blocks:
            if w.sink:
                f |= set(range(-(-min(w.sink, L) // 16)))
            if w.recent:
                f |= set(range(max(0, L - w.recent) // 16, nv))
        out += [f] * w.n_kv_heads
    return out


def _exact_bound(sq_t, K, lens, scale, b, j, G):
    """scale * max over the block's valid tokens and the row's query rows of
    sum_d |q_d| |k_d|: the size of the terms an fp32 accumulation adds, for
    the score tolerance (NumPy float32; only a tolerance, not a reference)."""
    qa = np.abs(synth.bf16_bits_to_f32(sq_t[b, :, j * G:(j + 1) * G]) if sq_t.dtype == np.uint16
                else sq_t[b, :, j * G:(j + 1) * G]).astype(np.float32).reshape(-1, sq_t.shape[-1])
    L = int(lens[b])
    nb = K.shape[2] // 16
    out = np.full(nb, -np.inf)
    if L == 0:
        return out
    kr = K[b, j, :L]
    ka = np.abs(synth.bf16_bits_to_f32(kr) if kr.dtype == np.uint16 else kr).astype(np.float32)
    tok = (ka @ qa.T).max(axis=1).astype(np.float64)
    nv = -(-L // 16)
    pad = np.full(nv * 16, -np.inf)
    pad[:L] = tok
    out[:nv] = scale * pad.reshape(nv, 16).max(axis=1)
    return out


def run_workload(w, steps=None, rows=None, heads=None, check_scores=True, fetch_on_attend=True, fused=False,
                 select=False):
    """Run `steps` steps of workload `w`; check rows `rows` (None = all) of
    the scores and the pool, and (b, h) pairs `heads` (None = all) of the
    attention.  Top-k and the working set are checked on every row."""
    steps = steps or w.steps
    data = synth.gen_workload(w.scaled(steps=steps))
    q, sq, K, V, lens = data["q"], data["score_q"], data["K"], data["V"], data["seq_lens"]
    mode = B.SKV_SCORE_QUEST if w.scoring == "quest" else B.SKV_SCORE_BLOCKMAX
    cfg = StepConfig(w.batch, w.n_q_heads, w.n_kv_heads, w.head_dim, w.ctx, w.dtype, w.k_blocks, w.capacity,
                     mode=mode, n_queries=w.n_score_queries, sink=w.sink, recent=w.recent)
    buf = LayerBuffers(cfg)
    dK, dV, dlens = dev(K), dev(V), dev(lens)
    scale = 1.0 / math.sqrt(w.head_dim)
    P, G = w.rows, w.group
    if mode == B.SKV_SCORE_QUEST:
        meta = torch.empty(w.batch, w.n_kv_heads, w.nb_max, 2, w.head_dim, dtype=cfg.torch_dtype, device="cuda")
        B.sparse_kv_quest_meta(cfg.shape, dK, dlens, meta)
        keys_or_meta = meta
        meta_ref = oracle.quest_meta(K, lens)
        box = np.maximum(np.abs(meta_ref[..., 0, :]), np.abs(meta_ref[..., 1, :]))
        box_meta = np.ascontiguousarray(np.stack([box, box], -2))
    else:
        keys_or_meta = dK
    lru = oracle.LRU(P, w.capacity)
    forced = _forced_sets(w, lens)
    rows = list(range(P)) if rows is None else rows
    hs = [(b, h) for b in range(w.batch) for h in range(w.n_q_heads)] if heads is None else heads
    total_miss = 0
    for t in range(steps):
        log(w.name, "step", t, (w.batch, w.n_q_heads, w.n_kv_heads, w.head_dim, w.ctx))
        decode_step(buf, dev(q[t]), dev(sq[t]), keys_or_meta, dlens, dK, dV, fetch_on_attend=fetch_on_attend,
                    fused=fused, select=select)
        torch.cuda.synchronize()
        g_scores = host(buf.scores).astype(np.float64)
        g_sel, g_cnt = host(buf.sel_blocks), host(buf.sel_count)
        # stage 1: rows against the fp64 oracle
        ora_rows = {}
        if check_scores:
            all_rows = len(rows) == P
            if all_rows:  # one oracle call over every row (its rows run in parallel)
                if mode == B.SKV_SCORE_QUEST:
                    ref_all = oracle.score_quest(sq[t], meta_ref, lens, scale, T=w.ctx)
                else:
                    ref_all = oracle.score_blockmax(sq[t], K, lens, scale)
            for r_ in rows:
                b, j = divmod(r_, w.n_kv_heads)
                qr = np.ascontiguousarray(sq[t][b:b + 1, :, j * G:(j + 1) * G])
                if mode == B.SKV_SCORE_QUEST:
                    ref = ref_all[b, j] if all_rows else oracle.score_quest(
                        qr, np.ascontiguousarray(meta_ref[b:b + 1, j:j + 1]), lens[b:b + 1], scale, T=w.ctx)[0, 0]
                    qa = np.abs(synth.bf16_bits_to_f32(qr) if qr.dtype == np.uint16 else qr).astype(np.float32)
                    bound = oracle.score_quest(qa, np.ascontiguousarray(box_meta[b:b + 1, j:j + 1]), lens[b:b + 1],
                                               scale, T=w.ctx)[0, 0]
                else:
                    ref = ref_all[b, j] if all_rows else oracle.score_blockmax(
                        qr, np.ascontiguousarray(K[b:b + 1, j:j + 1]), lens[b:b + 1], scale)[0, 0]
                    bound = _exact_bound(sq[t], K, lens, scale, b, j, G)
                got = g_scores[b, j]
                fin = np.isfinite(ref)
                assert np.array_equal(fin, np.isfinite(got)), f"row {r_}"
                assert np.all(np.abs(got[fin] - ref[fin]) <= GAMMA * bound[fin] + 2.0 ** -23 * np.abs(ref[fin])), \
                    f"scores of row {r_} step {t}"
                ora_rows[r_] = ref
        # stage 2: exact on the GPU's scores, tolerance rule on fp64 scores
        s_sel, s_cnt = oracle.topk(g_scores, lens, w.k_blocks, w.ctx, sink=w.sink, recent=w.recent)
        np.testing.assert_array_equal(g_cnt, s_cnt)
        np.testing.assert_array_equal(g_sel, s_sel)
        for r_ in sorted(ora_rows):
            b = r_ // w.n_kv_heads
            o_sel, o_cnt = oracle.topk(ora_rows[r_][None, None], lens[b:b + 1], w.k_blocks, w.ctx, sink=w.sink,
                                       recent=w.recent)
            bad = topk_swaps_ok(g_sel.reshape(P, -1)[r_:r_ + 1], g_cnt.reshape(P)[r_:r_ + 1], o_sel[0], o_cnt[0],
                                ora_rows[r_][None], forced=[forced[r_]])
            assert not bad, bad[:5]
        # stage 3: bit-exact given the GPU's selection
        out = lru.step(g_sel.reshape(P, -1), g_cnt.reshape(P), w.nb_max)
        np.testing.assert_array_equal(host(buf.miss_count).reshape(P), out["miss_count"])
        np.testing.assert_array_equal(host(buf.sel_slot).reshape(P, -1), out["sel_slot"])
        np.testing.assert_array_equal(host(buf.sel_hit).reshape(P, -1), out["sel_hit"])
        np.testing.assert_array_equal(host(buf.miss_block).reshape(P, -1), out["miss_block"])
        np.testing.assert_array_equal(host(buf.miss_slot).reshape(P, -1), out["miss_slot"])
        assert_lru_state(host(buf.slot_block), host(buf.slot_stamp), lru, f"step {t}")
        total_miss += int(out["miss_count"].sum())
        # pool bytes equal the source blocks the slots hold
        pk = host(buf.pool_k).reshape(P, w.capacity, 16, w.head_dim)
        pv = host(buf.pool_v).reshape(P, w.capacity, 16, w.head_dim)
        sb = lru.slot_block()
        for r_ in rows:
            b, j = divmod(r_, w.n_kv_heads)
            occ = np.nonzero(sb[r_] >= 0)[0]
            blk = sb[r_, occ]
            src_k = K[b, j].reshape(-1, 16, w.head_dim)[blk]
            src_v = V[b, j].reshape(-1, 16, w.head_dim)[blk]
            assert np.array_equal(pk[r_, occ], src_k) and np.array_equal(pv[r_, occ], src_v), f"pool row {r_}"
        # stage 4: attention from the source by block id
        g_out = host(buf.out)
        bs = sorted({b for b, _ in hs})
        o_ref, _ = oracle.attention(np.ascontiguousarray(q[t][bs]), np.ascontiguousarray(K[bs]),
                                    np.ascontiguousarray(V[bs]), g_sel[bs], g_cnt[bs], lens[bs], scale)
        for i, b in enumerate(bs):
            hh = [h for bb, h in hs if bb == b]
            err = max_rel_row_err(g_out[b, hh], o_ref[i, hh])
            if w.dtype == "f32":
                assert np.abs(g_out[b, hh] - o_ref[i, hh]).max() <= 1e-4
            assert err <= 2e-2 and err <= 1e-4, (err, b)
    return total_miss


def test_tiny_workload_all_steps():
    run_workload(synth.WORKLOADS["tiny"])


def test_tiny_workload_capacity_equals_budget_transfer_invariant():
    w = synth.WORKLOADS["tiny"].scaled(capacity=8)
    run_workload(w)


@pytest.mark.parametrize("fetch_on_attend", [True, False])
def test_llama8b_reduced_context(fetch_on_attend):
    w = synth.WORKLOADS["llama8b_32k"].scaled(batch=2, ctx=4096, budget=512)
    run_workload(w, steps=6, fetch_on_attend=fetch_on_attend)


def test_llama8b_ragged_lengths():
    w = synth.WORKLOADS["llama8b_32k"].scaled(batch=3, ctx=2048 + 16 * 7, budget=256, capacity=40, ragged=True)
    run_workload(w, steps=4)


def test_quest_reduced():
    w = synth.WORKLOADS["quest_128k"].scaled(batch=2, ctx=8192)
    run_workload(w, steps=5)


def test_lookahead_drafts_reduced():
    w = synth.WORKLOADS["lookahead_1m"].scaled(ctx=16384)
    run_workload(w, steps=3)


@pytest.mark.timeout(900)
@pytest.mark.parametrize("fused", [False, True])
def test_llama8b_full_size_all_steps(fused):
    # the benchmarked workload at full size (8 x 8 rows of 2048 blocks, 32
    # steps; the benchmark runs the fused call): every score row, top-k row,
    # working-set row, pool slot and attention head of every step
    run_workload(synth.WORKLOADS["llama8b_32k"], fused=fused)


def test_tiny_workload_fused():
    run_workload(synth.WORKLOADS["tiny"], fused=True)


@pytest.mark.timeout(900)
def test_quest_full_size_all_steps():
    # Quest-scored 128K-context workload at full size (4 x 8 rows, 8192
    # blocks per row, 512-token budget with 4 sink and 128 recent tokens
    # forced), fused call, all 16 steps: every row and head
    run_workload(synth.WORKLOADS["quest_128k"], fused=True)


@pytest.mark.timeout(900)
def test_lookahead_1m_full_size_fused():
    # the benchmark's path at full size (8 rows of 65536 blocks, 32 scoring
    # query rows per kv head, matrix-core scoring): score, then the fused
    # call (the top-k's chunk launch, selection + working-set update +
    # attention with fetch on attend, merge + commit); all 8 steps, every
    # row and head
    run_workload(synth.WORKLOADS["lookahead_1m"], fused=True)


@pytest.mark.timeout(900)
def test_lookahead_1m_full_size_one_launch_select():
    # the same workload through the selection call (the top-k's chunk
    # launch, then selection + working-set update) and attention with fetch
    # on attend; 4 steps, every row and head
    run_workload(synth.WORKLOADS["lookahead_1m"], steps=4, select=True)


@pytest.mark.timeout(900)
def test_lookahead_1m_full_size_four_calls():
    # the same workload through the four separate calls (long-row top-k),
    # two steps, every row and head
    run_workload(synth.WORKLOADS["lookahead_1m"], steps=2)


@pytest.mark.parametrize("fetch_on_attend", [True, False])
def test_llama8b_reduced_one_launch_select(fetch_on_attend):
    w = synth.WORKLOADS["llama8b_32k"].scaled(batch=2, ctx=4096, budget=512)
    run_workload(w, steps=4, select=True, fetch_on_attend=fetch_on_attend)
