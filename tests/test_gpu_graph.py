"""A whole decode step captured into a HIP graph replays to the same results
as eager execution (the library only enqueues kernels: no allocation, no
host synchronisation, no memset inside a step)."""
import numpy as np
import pytest
import torch

from top_sparse_kv_block_amd import synth
from top_sparse_kv_block_amd.step import Lag1Pipeline, LayerBuffers, StepConfig, decode_step
from gpu_util import dev, host, log

pytestmark = pytest.mark.gpu


def _state(buf):
    return [host(t).copy() for t in (buf.out, buf.lse, buf.sel_blocks, buf.sel_count, buf.slot_block, buf.slot_stamp,
                                     buf.clock, buf.sel_slot, buf.sel_hit, buf.miss_count, buf.pool_k, buf.pool_v)]


@pytest.mark.parametrize("fetch_on_attend", [True, False])
def test_graph_replays_match_eager(fetch_on_attend):
    w = synth.WORKLOADS["llama8b_32k"].scaled(batch=2, ctx=4096, budget=512, steps=3)
    data = synth.gen_workload(w)
    cfg = StepConfig(w.batch, w.n_q_heads, w.n_kv_heads, w.head_dim, w.ctx, w.dtype, w.k_blocks, w.capacity)
    buf = LayerBuffers(cfg)
    q, sq = dev(data["q"]), dev(data["score_q"])
    K, V, lens = dev(data["K"]), dev(data["V"]), dev(data["seq_lens"])

    def steps():
        for t in range(w.steps):
            decode_step(buf, q[t], sq[t], K, lens, K, V, fetch_on_attend=fetch_on_attend)

    log("graph eager reference", fetch_on_attend)
    buf.reset()
    buf.pool_k.zero_()
    buf.pool_v.zero_()
    steps()
    torch.cuda.synchronize()
    ref = _state(buf)

    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        steps()
    torch.cuda.synchronize()
    for rep in range(3):
        log("graph replay", rep)
        buf.reset()  # eager work between replays
        buf.pool_k.zero_()
        buf.pool_v.zero_()
        buf.out.fill_(7.0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for a, b in zip(_state(buf), ref):
            np.testing.assert_array_equal(a, b)


@pytest.mark.parametrize("path", ["fused", "select", "lag1"])
def test_graph_replays_match_eager_other_paths(path):
    # the fused call, the one-launch select + attention, and the lag-1
    # pipeline (two streams joined inside the capture)
    cap = 64 if path == "lag1" else None
    w = synth.WORKLOADS["llama8b_32k"].scaled(batch=2, ctx=4096, budget=512, steps=4)
    if cap:
        w = w.scaled(capacity=cap)
    data = synth.gen_workload(w)
    cfg = StepConfig(w.batch, w.n_q_heads, w.n_kv_heads, w.head_dim, w.ctx, w.dtype, w.k_blocks, w.capacity)
    buf = LayerBuffers(cfg)
    pipe = Lag1Pipeline(buf) if path == "lag1" else None
    q, sq = dev(data["q"]), dev(data["score_q"])
    K, V, lens = dev(data["K"]), dev(data["V"]), dev(data["seq_lens"])

    def steps():
        if pipe is not None:
            pipe.rewind()
            for t in range(w.steps):
                pipe.step(q[t], sq[t], K, lens, K, V)
            pipe.join()
            return
        for t in range(w.steps):
            decode_step(buf, q[t], sq[t], K, lens, K, V, fused=path == "fused", select=path == "select")

    def clear():
        buf.reset()
        buf.pool_k.zero_()
        buf.pool_v.zero_()

    log("graph eager reference", path)
    clear()
    steps()
    torch.cuda.synchronize()
    ref = _state(buf)

    g = torch.cuda.CUDAGraph()
    clear()
    with torch.cuda.graph(g):
        steps()
    torch.cuda.synchronize()
    for rep in range(3):
        log("graph replay", path, rep)
        clear()  # eager work between replays
        buf.out.fill_(7.0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for a, b in zip(_state(buf), ref):
            np.testing.assert_array_equal(a, b)
