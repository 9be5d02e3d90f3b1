"""Checkpoint / resume of a layer's working set on the GPU.

All cache state lives in caller buffers (slot table, stamps, clock, pool),
so saving them and restoring them into fresh buffers must continue the run
exactly: T steps straight through against T/2 steps, a snapshot copied to
host memory, a restore into new buffers and the other T/2 steps.  The later
steps' selections, lists, state, pool and outputs are bit-identical, and the
resumed lists equal the oracle list's (run straight through on the same
selections).  The block table is what gets saved and restored, as with the
block-table snapshot and rollback of KV-Cache 压缩技术的工程原理 §6.1.
"""
import numpy as np
import pytest
import torch

import oracle
from top_sparse_kv_block_amd import synth
from top_sparse_kv_block_amd.step import LayerBuffers, StepConfig, decode_step
from gpu_util import assert_lru_state, dev, host, log

pytestmark = pytest.mark.gpu

FIELDS = ("out", "lse", "sel_blocks", "sel_count", "slot_block", "slot_stamp", "clock", "sel_slot", "sel_hit",
          "miss_block", "miss_slot", "miss_count", "pool_k", "pool_v")
STATE = ("slot_block", "slot_stamp", "clock", "pool_k", "pool_v")


@pytest.mark.parametrize("fused", [False, True])
def test_snapshot_restore_continues_bit_identically(fused):
    T = 8
    w = synth.WORKLOADS["llama8b_32k"].scaled(batch=2, ctx=4096, budget=512, capacity=48, steps=T)
    data = synth.gen_workload(w)
    cfg = StepConfig(w.batch, w.n_q_heads, w.n_kv_heads, w.head_dim, w.ctx, w.dtype, w.k_blocks, w.capacity,
                     num_splits=4)
    K, V, lens = dev(data["K"]), dev(data["V"]), dev(data["seq_lens"])

    def step(buf, t):
        log("snapshot/restore", "fused" if fused else "four calls", "step", t)
        decode_step(buf, dev(data["q"][t]), dev(data["score_q"][t]), K, lens, K, V, fused=fused)
        torch.cuda.synchronize()
        return {f: host(getattr(buf, f)).copy() for f in FIELDS}

    straight = LayerBuffers(cfg)
    ref = [step(straight, t) for t in range(T)]
    first = LayerBuffers(cfg)
    for t in range(T // 2):
        step(first, t)
    snap = {f: getattr(first, f).detach().cpu().clone() for f in STATE}
    del first
    resumed = LayerBuffers(cfg)
    for f in STATE:
        getattr(resumed, f).copy_(snap[f])
    lru = oracle.LRU(w.rows, w.capacity)
    for t in range(T):
        out = lru.step(ref[t]["sel_blocks"].reshape(w.rows, -1), ref[t]["sel_count"].reshape(-1), w.nb_max)
        if t < T // 2:
            continue
        got = step(resumed, t)
        for f in FIELDS:
            np.testing.assert_array_equal(got[f], ref[t][f], err_msg=f"{f} at step {t}")
        for f in ("sel_slot", "sel_hit", "miss_block", "miss_slot", "miss_count"):
            np.testing.assert_array_equal(got[f].reshape(out[f].shape), out[f], err_msg=f"{f} vs oracle at {t}")
        assert_lru_state(got["slot_block"], got["slot_stamp"], lru, f"step {t}")
    assert int(ref[T - 1]["miss_count"].sum()) > 0
