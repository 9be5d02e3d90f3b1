"""GPU parity of the host tier: full K/V in pinned, device-mapped host memory.

The host-tier workload (16 x 8 rows, 131072-token context, 32 layers) keeps
each layer's full K/V in host memory and a 256-slot working set per row on
the GPU; the selections are given (the indexer is not run) with ~50% overlap
between adjacent layers and ~80% between adjacent steps.  Here the same
recipe runs reduced (2 sequences, 16K context, 3 layers, 3 steps): every
layer keeps its own working set, misses come over PCIe by block id, and the
lists, the pool bytes and the attention output are checked against the
oracle exactly as for a device source.  Three ways to fetch: the separate
gather of ``sparse_kv_cache_update``, fetch on attend, and the fused call
(fed scores that rank exactly the given selection first).
"""
import math

import numpy as np
import pytest
import torch

import oracle
from top_sparse_kv_block_amd import binding as B
from top_sparse_kv_block_amd import synth
from top_sparse_kv_block_amd.step import LayerBuffers, StepConfig
from gpu_util import dev, host, log, max_rel_row_err

pytestmark = pytest.mark.gpu


def _host_copy(a: np.ndarray) -> B.HostBuffer:
    hb = B.HostBuffer(a.nbytes)
    hb.numpy(a.dtype, a.shape)[...] = a
    return hb


@pytest.mark.parametrize("mode", ["gather", "fetch_on_attend", "fused"])
def test_host_tier_layers_reduced(mode):
    w = synth.WORKLOADS["host_tier_32l"].scaled(batch=2, ctx=16384, layers=3, steps=3)
    sels = synth.gen_layer_selections(w)  # [steps, layers, B, Hkv, k]
    P, k, C, nb = w.rows, w.k_blocks, w.capacity, w.nb_max
    lens = synth.gen_seq_lens(w)
    dlens = dev(lens)
    scale = 1.0 / math.sqrt(w.head_dim)
    layers = []
    try:
        for l in range(w.layers):
            K, V = synth.gen_kv(w, l)
            q, _ = synth.gen_queries(w, l)
            cfg = StepConfig(w.batch, w.n_q_heads, w.n_kv_heads, w.head_dim, w.ctx, w.dtype, k, C)
            layers.append(dict(K=K, V=V, q=q, hk=_host_copy(K), hv=_host_copy(V), buf=LayerBuffers(cfg),
                               lru=oracle.LRU(P, C)))
        for s in range(w.steps):
            for l, L in enumerate(layers):
                log("host tier", mode, "step", s, "layer", l, (w.batch, w.n_kv_heads, w.ctx, k, C))
                buf, sel = L["buf"], sels[s, l]
                cnt = np.full((w.batch, w.n_kv_heads), k, dtype=np.int32)
                hk, hv = L["hk"].device_ptr, L["hv"].device_ptr
                qd = dev(L["q"][s])
                if mode == "fused":
                    sc = np.zeros((w.batch, w.n_kv_heads, nb), dtype=np.float32)
                    np.put_along_axis(sc, sel.astype(np.int64), 1.0, axis=-1)
                    buf.scores.copy_(dev(sc))
                    buf.select_attend(qd, dlens, hk, hv, B.SKV_SRC_HOST_MAPPED)
                else:
                    buf.sel_blocks.copy_(dev(sel))
                    buf.sel_count.copy_(dev(cnt))
                    if mode == "gather":
                        buf.cache_update(hk, hv, B.SKV_SRC_HOST_MAPPED)
                        buf.attention(qd, dlens)
                    else:
                        buf.cache_update(None, None)
                        buf.attention(qd, dlens, hk, hv, B.SKV_SRC_HOST_MAPPED)
                torch.cuda.synchronize()
                np.testing.assert_array_equal(host(buf.sel_blocks), sel)
                out = L["lru"].step(sel.reshape(P, k), cnt.reshape(P), nb)
                for name in ("sel_slot", "sel_hit", "miss_block", "miss_slot"):
                    np.testing.assert_array_equal(host(getattr(buf, name)).reshape(P, k), out[name])
                np.testing.assert_array_equal(host(buf.miss_count).reshape(P), out["miss_count"])
                np.testing.assert_array_equal(host(buf.slot_block).reshape(P, C), L["lru"].slot_block())
                if s == 0:
                    assert out["miss_count"].sum() == P * k  # cold start
                else:
                    assert 0 < out["miss_count"].sum() < P * k
                # every resident slot holds its block's bytes, fetched over PCIe
                pk = host(buf.pool_k).reshape(P, C, 16, w.head_dim)
                pv = host(buf.pool_v).reshape(P, C, 16, w.head_dim)
                sb = L["lru"].slot_block()
                for r_ in range(P):
                    b, j = divmod(r_, w.n_kv_heads)
                    for slot, blk in enumerate(sb[r_]):
                        if blk >= 0:
                            assert np.array_equal(pk[r_, slot], L["K"][b, j, 16 * blk:16 * blk + 16])
                            assert np.array_equal(pv[r_, slot], L["V"][b, j, 16 * blk:16 * blk + 16])
                o_ref, _ = oracle.attention(L["q"][s], L["K"], L["V"], sel, cnt, lens, scale)
                err = max_rel_row_err(host(buf.out), o_ref)
                assert err <= 2e-2 and err <= 1e-4, err
    finally:
        torch.cuda.synchronize()
        for L in layers:
            L["hk"].free()
            L["hv"].free()


@pytest.mark.parametrize("prefetch", [False, True])
def test_layer_sweep_cross_layer_prefetch(prefetch):
    # one decode step over consecutive layers (each with its own host K/V and
    # working set); with prefetch, layer l+1's set is first updated with layer
    # l's selection on a second stream.  The oracle: the same two LRU steps.
    from top_sparse_kv_block_amd.step import layer_sweep
    w = synth.WORKLOADS["host_tier_32l"].scaled(batch=2, ctx=16384, layers=3, steps=3)
    sels = synth.gen_layer_selections(w)
    P, k, C, nb = w.rows, w.k_blocks, w.capacity, w.nb_max
    lens = synth.gen_seq_lens(w)
    dlens = dev(lens)
    scale = 1.0 / math.sqrt(w.head_dim)
    cnt = np.full((w.batch, w.n_kv_heads), k, dtype=np.int32)
    side = torch.cuda.Stream()
    Ks, Vs, qs, hbs, bufs, lrus = [], [], [], [], [], []
    try:
        for l in range(w.layers):
            K, V = synth.gen_kv(w, l)
            q, _ = synth.gen_queries(w, l)
            Ks.append(K), Vs.append(V), qs.append(q)
            hbs.append((_host_copy(K), _host_copy(V)))
            cfg = StepConfig(w.batch, w.n_q_heads, w.n_kv_heads, w.head_dim, w.ctx, w.dtype, k, C)
            bufs.append(LayerBuffers(cfg))
            lrus.append(oracle.LRU(P, C))
        srcs = [(hk.device_ptr, hv.device_ptr) for hk, hv in hbs]
        for s in range(w.steps):
            log("layer sweep, prefetch", prefetch, "step", s)
            for l, buf in enumerate(bufs):
                buf.sel_blocks.copy_(dev(sels[s, l]))
                buf.sel_count.copy_(dev(cnt))
            layer_sweep(bufs, [dev(q[s]) for q in qs], dlens, srcs, B.SKV_SRC_HOST_MAPPED, prefetch=prefetch,
                        side_stream=side)
            torch.cuda.synchronize()
            for l, buf in enumerate(bufs):
                if prefetch and l > 0:
                    pf = lrus[l].step(sels[s, l - 1].reshape(P, k), cnt.reshape(P), nb)
                    np.testing.assert_array_equal(host(buf.pf_miss_count).reshape(P), pf["miss_count"])
                    np.testing.assert_array_equal(host(buf.pf_miss_block).reshape(P, k), pf["miss_block"])
                out = lrus[l].step(sels[s, l].reshape(P, k), cnt.reshape(P), nb)
                for name in ("sel_slot", "sel_hit", "miss_block", "miss_slot"):
                    np.testing.assert_array_equal(host(getattr(buf, name)).reshape(P, k), out[name], name)
                np.testing.assert_array_equal(host(buf.miss_count).reshape(P), out["miss_count"])
                np.testing.assert_array_equal(host(buf.slot_block).reshape(P, C), lrus[l].slot_block())
                if s > 0 and l > 0:
                    # the shared blocks were fetched ahead: about half of the misses remain
                    now, prev = sels[s, l].reshape(P, k), sels[s - 1, l].reshape(P, k)
                    new = sum(len(set(a) - set(b)) for a, b in zip(now, prev))
                    frac = out["miss_count"].sum() / new
                    assert (frac < 0.75) if prefetch else (frac > 0.75), frac
                pk = host(buf.pool_k).reshape(P, C, 16, w.head_dim)
                pv = host(buf.pool_v).reshape(P, C, 16, w.head_dim)
                sb = lrus[l].slot_block()
                for r_ in range(P):
                    b, j = divmod(r_, w.n_kv_heads)
                    for slot, blk in enumerate(sb[r_]):
                        if blk >= 0:
                            assert np.array_equal(pk[r_, slot], Ks[l][b, j, 16 * blk:16 * blk + 16])
                            assert np.array_equal(pv[r_, slot], Vs[l][b, j, 16 * blk:16 * blk + 16])
                o_ref, _ = oracle.attention(qs[l][s], Ks[l], Vs[l], sels[s, l], cnt, lens, scale)
                assert max_rel_row_err(host(buf.out), o_ref) <= 1e-4
    finally:
        torch.cuda.synchronize()
        for hk, hv in hbs:
            hk.free()
            hv.free()


def test_host_source_equals_device_source_bit_exact():
    # the tier does not change any result: the same step from a host-mapped
    # and from a device source gives identical lists, pools and outputs
    w = synth.WORKLOADS["llama8b_32k"].scaled(batch=2, ctx=4096, budget=512, steps=2)
    data = synth.gen_workload(w)
    cfg = StepConfig(w.batch, w.n_q_heads, w.n_kv_heads, w.head_dim, w.ctx, w.dtype, w.k_blocks, w.capacity)
    dK, dV, dlens = dev(data["K"]), dev(data["V"]), dev(data["seq_lens"])
    hk, hv = _host_copy(data["K"]), _host_copy(data["V"])
    try:
        bufs = [LayerBuffers(cfg), LayerBuffers(cfg)]
        for t in range(w.steps):
            log("host vs device source, step", t)
            q, sq = dev(data["q"][t]), dev(data["score_q"][t])
            for i, (sk, sv, kind) in enumerate([(dK, dV, B.SKV_SRC_DEVICE),
                                                (hk.device_ptr, hv.device_ptr, B.SKV_SRC_HOST_MAPPED)]):
                bufs[i].score(sq, dK, dlens)
                bufs[i].select_attend(q, dlens, sk, sv, kind)
            torch.cuda.synchronize()
            for name in ("sel_blocks", "sel_slot", "sel_hit", "miss_block", "miss_slot", "miss_count",
                         "slot_block", "slot_stamp", "pool_k", "pool_v", "out", "lse"):
                np.testing.assert_array_equal(host(getattr(bufs[0], name)), host(getattr(bufs[1], name)), name)
    finally:
        torch.cuda.synchronize()
        hk.free()
        hv.free()


@pytest.mark.timeout(400)
def test_host_tier_full_size_sampled_with_prefetch():
    # the benchmark's host-tier shape: 16 x 8 rows, 131072-token context,
    # 128 of 256 slots, two layers each with its own K/V (8 GiB per layer) in
    # pinned mapped host memory, the cross-layer prefetch on a second stream.
    # Every row's lists and slot table against the oracle's two LRU steps;
    # sampled rows' pool bytes and sampled heads' attention
    from top_sparse_kv_block_amd.step import layer_sweep
    w = synth.WORKLOADS["host_tier_32l"].scaled(layers=2, steps=2)
    sels = synth.gen_layer_selections(w)
    P, k, C, nb = w.rows, w.k_blocks, w.capacity, w.nb_max
    lens = np.full(w.batch, w.ctx, np.int32)
    dlens = dev(lens)
    scale = 1.0 / math.sqrt(w.head_dim)
    cnt = np.full((w.batch, w.n_kv_heads), k, dtype=np.int32)
    n_elem = w.rows * w.ctx * w.head_dim
    side = torch.cuda.Stream()
    g = torch.Generator(device="cuda").manual_seed(41)
    hbs, views, bufs, lrus = [], [], [], []
    try:
        for l in range(w.layers):
            pair = []
            for _ in range(2):
                hb = B.HostBuffer(n_elem * 2)
                hbs.append(hb)
                ht = torch.from_numpy(hb.numpy(np.int16, (n_elem,))).view(torch.bfloat16)
                for off in range(0, n_elem, 1 << 26):
                    n = min(1 << 26, n_elem - off)
                    ht[off:off + n].copy_(torch.randn(n, generator=g, device="cuda").to(torch.bfloat16))
                pair.append(hb)
            views.append([hb.numpy(np.uint16, (w.batch, w.n_kv_heads, w.ctx, w.head_dim)) for hb in pair])
            cfg = StepConfig(w.batch, w.n_q_heads, w.n_kv_heads, w.head_dim, w.ctx, w.dtype, k, C)
            bufs.append(LayerBuffers(cfg))
            lrus.append(oracle.LRU(P, C))
        srcs = [(hbs[2 * l].device_ptr, hbs[2 * l + 1].device_ptr) for l in range(w.layers)]
        rows, heads = [0, 77, 127], [(0, 0), (9, 14), (15, 31)]
        r = np.random.default_rng(5)
        for s in range(w.steps):
            qs = [synth.f32_to_bf16_bits(r.standard_normal((w.batch, w.n_q_heads, w.head_dim)).astype(np.float32))
                  for _ in range(w.layers)]
            for l, buf in enumerate(bufs):
                buf.sel_blocks.copy_(dev(sels[s, l]))
                buf.sel_count.copy_(dev(cnt))
            log("host tier full size, step", s)
            layer_sweep(bufs, [dev(q) for q in qs], dlens, srcs, B.SKV_SRC_HOST_MAPPED, prefetch=True,
                        side_stream=side)
            torch.cuda.synchronize()
            for l, buf in enumerate(bufs):
                if l > 0:
                    pf = lrus[l].step(sels[s, l - 1].reshape(P, k), cnt.reshape(P), nb)
                    np.testing.assert_array_equal(host(buf.pf_miss_count).reshape(P), pf["miss_count"])
                out = lrus[l].step(sels[s, l].reshape(P, k), cnt.reshape(P), nb)
                for name in ("sel_slot", "sel_hit", "miss_block", "miss_slot"):
                    np.testing.assert_array_equal(host(getattr(buf, name)).reshape(P, k), out[name], name)
                np.testing.assert_array_equal(host(buf.miss_count).reshape(P), out["miss_count"])
                sb = lrus[l].slot_block()
                np.testing.assert_array_equal(host(buf.slot_block).reshape(P, C), sb)
                Kh, Vh = views[l]
                pk = host(buf.pool_k).reshape(P, C, 16, w.head_dim)
                pv = host(buf.pool_v).reshape(P, C, 16, w.head_dim)
                for r_ in rows:
                    b, j = divmod(r_, w.n_kv_heads)
                    for slot, blk in enumerate(sb[r_]):
                        if blk >= 0:
                            assert np.array_equal(pk[r_, slot], Kh[b, j, 16 * blk:16 * blk + 16])
                            assert np.array_equal(pv[r_, slot], Vh[b, j, 16 * blk:16 * blk + 16])
                g_out = host(buf.out)
                for b in sorted({b for b, _ in heads}):
                    o_ref, _ = oracle.attention(qs[l][b:b + 1], Kh[b:b + 1], Vh[b:b + 1], sels[s, l][b:b + 1],
                                                cnt[b:b + 1], lens[b:b + 1], scale)
                    hh = [h for bb, h in heads if bb == b]
                    assert max_rel_row_err(g_out[b, hh], o_ref[0, hh]) <= 1e-4
    finally:
        torch.cuda.synchronize()
        for hb in hbs:
            hb.free()
