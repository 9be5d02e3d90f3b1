"""The fused call without allocation (sparse_kv_select_attend_noalloc, the
split partials in the library's static device scratch) equals the fused
call with a caller workspace (sparse_kv_select_attend) bit for bit: the
selection, the lists, the working-set state, the pool, the output and the
lse, step after step.  Calls in a row, each with a smaller input than the
one before (the scratch keeps the previous call's contents; the first also
holds the long-row top-k's chunk candidates after the partials), then a call
whose partials would not fit, refused on the host with SKV_ERR_SCRATCH.
Through the C ABI.
"""
import numpy as np
import pytest
import torch

from top_sparse_kv_block_amd import binding as B
from top_sparse_kv_block_amd import synth
from top_sparse_kv_block_amd.step import LayerBuffers, StepConfig
from gpu_util import dev, host, log

pytestmark = pytest.mark.gpu

FIELDS = ("out", "lse", "sel_blocks", "sel_count", "slot_block", "slot_stamp", "clock", "sel_slot", "sel_hit",
          "miss_block", "miss_slot", "miss_count", "pool_k", "pool_v")


def _noalloc(buf, q, lens, K, V):
    c = buf.cfg
    B.sparse_kv_select_attend_noalloc(buf.shape, buf.scores, lens, c.k_blocks, c.sink, c.recent, c.capacity,
                                      buf.sel_blocks, buf.sel_count, buf.slot_block, buf.slot_stamp, buf.clock,
                                      buf.sel_slot, buf.sel_hit, buf.miss_block, buf.miss_slot, buf.miss_count, q,
                                      buf.pool_k, buf.pool_v, K, V, B.SKV_SRC_DEVICE, c.softmax_scale,
                                      buf.fused_splits, buf.out, buf.lse)


def test_noalloc_equals_the_workspace_call_on_two_calls_in_a_row():
    cases = [("llama8b_32k", dict(batch=1, ctx=16 * 20000, budget=1024, capacity=80), 2),  # chunk candidates too
             ("llama8b_32k", dict(batch=4, ctx=8192, budget=1024, capacity=80), 3),
             ("quest_128k", dict(batch=1, n_kv_heads=4, n_q_heads=16, ctx=4096), 2)]  # smaller second input
    for name, kw, steps in cases:
        w = synth.WORKLOADS[name].scaled(steps=steps, **kw)
        data = synth.gen_workload(w)
        mode = B.SKV_SCORE_QUEST if w.scoring == "quest" else B.SKV_SCORE_BLOCKMAX
        cfg = StepConfig(w.batch, w.n_q_heads, w.n_kv_heads, w.head_dim, w.ctx, w.dtype, w.k_blocks, w.capacity,
                         mode=mode, n_queries=w.n_score_queries, sink=w.sink, recent=w.recent)
        a, b = LayerBuffers(cfg), LayerBuffers(cfg)
        K, V, lens = dev(data["K"]), dev(data["V"]), dev(data["seq_lens"])
        keys = K
        if mode == B.SKV_SCORE_QUEST:
            keys = torch.empty(w.batch, w.n_kv_heads, w.nb_max, 2, w.head_dim, dtype=cfg.torch_dtype, device="cuda")
            B.sparse_kv_quest_meta(cfg.shape, K, lens, keys)
        for t in range(steps):
            log("noalloc vs workspace", name, kw, "step", t)
            q, sq = dev(data["q"][t]), dev(data["score_q"][t])
            for buf in (a, b):
                buf.score(sq, keys, lens)
            a.select_attend(q, lens, K, V)
            _noalloc(b, q, lens, K, V)
            torch.cuda.synchronize()
            for f in FIELDS:
                np.testing.assert_array_equal(host(getattr(b, f)), host(getattr(a, f)), err_msg=f"{f} {name} {t}")
        assert int(host(b.miss_count).sum()) >= 0 and np.isfinite(host(b.lse)).any()


def test_noalloc_refuses_partials_beyond_its_scratch():
    # 64 rows x 128 splits x 16 heads x 130 floats = 68 MB of partials > 8 MiB:
    # refused on the host before any launch
    Bsz, Hkv, Hq, D, T, k = 8, 8, 128, 128, 4096, 128
    cfg = StepConfig(Bsz, Hq, Hkv, D, T, "bf16", k, k, num_splits=128)
    need = Bsz * Hkv * 128 * (Hq // Hkv) * (D + 2) * 4
    assert need > B.NOALLOC_SCRATCH_BYTES
    buf = LayerBuffers(cfg)
    K = torch.zeros(Bsz, Hkv, T, D, dtype=torch.bfloat16, device="cuda")
    lens = torch.full((Bsz,), T, dtype=torch.int32, device="cuda")
    q = torch.zeros(Bsz, Hq, D, dtype=torch.bfloat16, device="cuda")
    log("noalloc oversized partials")
    with pytest.raises(B.SparseKVError) as err:
        _noalloc(buf, q, lens, K, K)
    assert err.value.status == 8
    torch.cuda.synchronize()
