"""Whole decode steps over seeded random shapes, against the oracle.

Each case draws a shape inside the library's limits: batch, kv heads, GQA
group (1-16), head dim (64 or 128), dtype, scoring (block max with the
current query or 1-4 drafts, or the Quest bound), context and ragged
lengths, budget, working-set capacity (at least the budget) and forced
sink / recent blocks; some cases have rows of 16385 to 65536 blocks (the
two-launch top-k).  Three steps run through the fused call, the four
separate calls, or the one-launch selection, and every stage is checked
against the oracle by the same checks as the fixed workloads (scores
within the fp32 bound, top-k and working set bit-exact given the GPU's
scores, pool bytes, attention within tolerance).
"""
import numpy as np
import pytest

from top_sparse_kv_block_amd import synth
from test_gpu_step import run_workload

pytestmark = pytest.mark.gpu


def _cases(n=32, seed=20261203):
    rng = np.random.default_rng(seed)
    out = []
    while len(out) < n:
        scoring = ("blockmax", "quest")[int(rng.integers(2))]
        dtype = ("bf16", "f32")[int(rng.integers(2))]
        D = (64, 128)[int(rng.integers(2))]
        hkv = int(rng.choice([1, 2, 3, 4, 8]))
        G = int(rng.choice([1, 2, 4, 8, 16]))
        drafts = int(rng.integers(0, 5)) if scoring == "blockmax" else 0
        if G * max(drafts, 1) > 32:  # query rows per kv head the scoring takes
            continue
        if rng.random() < 0.15:  # rows past 16384 blocks: the top-k's chunk launch first
            dtype, batch, hkv = "bf16", 1, min(hkv, 2)
            ctx = 16 * int(rng.integers(16385, 65537))
        else:
            batch = int(rng.integers(1, 5))
            ctx = 16 * int(rng.integers(2, 1201))
        k = int(rng.integers(1, min(ctx // 16, 1024) + 1))
        cap = int(min(1024, k + int(rng.integers(0, k + 1))))
        sink = recent = 0
        if k >= 8:  # forced blocks (at most 2 + recent/16 + 1) stay within the budget
            sink = 16 * int(rng.integers(0, 3))
            recent = 16 * int(rng.integers(0, k // 4 + 1))
        ragged = bool(rng.integers(2))
        w = synth.WORKLOADS["tiny"].scaled(
            name=f"random{len(out)}", batch=batch, n_q_heads=G * hkv, n_kv_heads=hkv, head_dim=D, dtype=dtype,
            ctx=ctx, budget=16 * k, capacity=cap, steps=3, scoring=scoring, n_drafts=drafts, sink=sink,
            recent=recent, ragged=ragged, seed=int(rng.integers(1 << 30)))
        out.append(w)
    return out


CASES = _cases()


def _id(w):
    return (f"{w.name}-{w.scoring}{w.n_drafts or ''}-{w.dtype}-D{w.head_dim}-B{w.batch}-kv{w.n_kv_heads}"
            f"-G{w.group}-ctx{w.ctx}{'r' if w.ragged else ''}-k{w.k_blocks}-C{w.capacity}-s{w.sink}-r{w.recent}")


@pytest.mark.parametrize("path", ["fused", "four_calls", "select"])
@pytest.mark.parametrize("w", CASES, ids=[_id(w) for w in CASES])
def test_random_shapes(w, path):
    run_workload(w, steps=3, fused=path == "fused", select=path == "select")
