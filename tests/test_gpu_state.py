"""GPU parity of the working-set consistency check (sparse_kv_check_state)
against the oracle's check: states left by real update steps (consistent),
the same states with one rule broken per row, and seeded random tables with
random corruptions at several capacities."""
import numpy as np
import pytest
import torch

import oracle
from top_sparse_kv_block_amd import binding as B
from top_sparse_kv_block_amd import synth
from top_sparse_kv_block_amd.step import LayerBuffers, StepConfig, decode_step
from gpu_util import dev, host, log

pytestmark = pytest.mark.gpu


def _flags(shape, cap, sb, st, ck):
    rows = shape.batch * shape.n_kv_heads
    flags = torch.full((rows,), -7, dtype=torch.int32, device="cuda")
    B.sparse_kv_check_state(shape, cap, dev(sb), dev(st.view(np.int32)), dev(ck.view(np.int32)), flags)
    torch.cuda.synchronize()
    return host(flags)


def test_states_left_by_updates_and_their_corruptions():
    w = synth.WORKLOADS["llama8b_32k"].scaled(batch=2, ctx=4096, budget=512, capacity=80, steps=4)
    data = synth.gen_workload(w)
    cfg = StepConfig(w.batch, w.n_q_heads, w.n_kv_heads, w.head_dim, w.ctx, w.dtype, w.k_blocks, w.capacity)
    buf = LayerBuffers(cfg)
    K, V, lens = dev(data["K"]), dev(data["V"]), dev(data["seq_lens"])
    for t in range(w.steps):
        log("check_state: update step", t)
        decode_step(buf, dev(data["q"][t]), dev(data["score_q"][t]), K, lens, K, V, fused=True)
    torch.cuda.synchronize()
    rows, cap, nb = w.rows, w.capacity, w.nb_max
    sb = host(buf.slot_block).reshape(rows, cap).copy()
    st = host(buf.slot_stamp).reshape(rows, cap).view(np.uint32).copy()
    ck = host(buf.clock).reshape(rows).view(np.uint32).copy()
    log("check_state: consistent state")
    got = _flags(cfg.shape, cap, sb, st, ck)
    assert got.tolist() == [0] * rows
    assert oracle.check_state(sb, st, ck, nb)[1] == 0
    # one broken rule per row (rows 0-3), all three on row 4, the rest kept
    occ = [np.nonzero(sb[r] >= 0)[0] for r in range(rows)]
    sb[0, occ[0][0]] = nb                       # id past the end
    sb[1, occ[1][1]] = sb[1, occ[1][0]]         # a block in two slots
    st[2, occ[2][2]] = ck[2] + 1                # stamped after the clock
    sb[3, occ[3][0]] = -5                       # id below -1
    sb[4, occ[4][0]], sb[4, occ[4][1]] = nb + 9, sb[4, occ[4][2]]
    st[4, occ[4][3]] = 0xFFFFFFFF
    log("check_state: corrupted rows")
    got = _flags(cfg.shape, cap, sb, st, ck)
    ref, n = oracle.check_state(sb, st, ck, nb)
    np.testing.assert_array_equal(got, ref)
    assert ref.tolist()[:5] == [1, 2, 4, 1, 7] and n == 5


@pytest.mark.parametrize("cap", [1, 33, 128, 1024])
def test_random_tables(cap):
    rng = np.random.default_rng(cap)
    Bsz, Hkv, T = 4, 8, 16 * 4096
    rows, nb = Bsz * Hkv, T // 16
    shape = B.make_shape(Bsz, 4 * Hkv, Hkv, 64, T, "f32")
    sb = np.full((rows, cap), -1, np.int32)
    st = rng.integers(0, 50, size=(rows, cap)).astype(np.uint32)
    ck = rng.integers(40, 60, size=rows).astype(np.uint32)
    for r in range(rows):
        n_occ = rng.integers(0, cap + 1)
        sb[r, rng.permutation(cap)[:n_occ]] = rng.permutation(nb)[:n_occ]
        kind = rng.integers(0, 5)
        occ = np.nonzero(sb[r] >= 0)[0]
        if kind == 1:
            sb[r, rng.integers(0, cap)] = rng.choice([-2, nb, nb + 100, -(1 << 30)])
        elif kind == 2 and len(occ) >= 2:
            sb[r, occ[1]] = sb[r, occ[0]]
        elif kind == 3 and len(occ) >= 1:
            st[r, occ[0]] = ck[r] + rng.integers(1, 5)
    log("check_state random tables, capacity", cap)
    got = _flags(shape, cap, sb, st, ck)
    ref, _ = oracle.check_state(sb, st, ck, nb)
    np.testing.assert_array_equal(got, ref)
    assert ref.any() and (ref == 0).any() if cap >= 33 else True
