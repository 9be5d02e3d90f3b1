"""GPU parity of stage 1 (block scoring) against the oracle."""
import math

import numpy as np
import pytest
import torch

import oracle
from top_sparse_kv_block_amd import binding as B
from top_sparse_kv_block_amd import synth
from gpu_util import dev, host, log, to_dtype

pytestmark = pytest.mark.gpu

# fp32 accumulation bound: every path from a product to the score passes
# at most 12 roundings (a 4-deep dot2/FMA chain, whose dot2 may round twice,
# and 4 DPP additions) plus the final scale multiply, so
# |gpu - exact| <= 16 * 2^-24 * scale * max sum_d |q_d k_d| + 2^-23 * |s|.
GAMMA = 16 * 2.0 ** -24


def _abs(a):
    return (a & np.uint16(0x7FFF)) if a.dtype == np.uint16 else np.abs(a)


def _score_case(B_, Hq, Hkv, D, T, NQ, dtype, lens, seed, mode="blockmax"):
    r = np.random.default_rng(seed)
    q = to_dtype(r.standard_normal((B_, NQ, Hq, D)), dtype)
    k = to_dtype(r.standard_normal((B_, Hkv, T, D)) * 1.5, dtype)
    lens = np.asarray(lens, dtype=np.int32)
    scale = 1.0 / math.sqrt(D)
    shape = B.make_shape(B_, Hq, Hkv, D, T, dtype)
    nb = T // 16
    scores = torch.empty(B_, Hkv, nb, dtype=torch.float32, device="cuda")
    log("score", mode, dtype, (B_, Hq, Hkv, D, T, NQ), "seed", seed)
    if mode == "blockmax":
        B.sparse_kv_score(shape, B.SKV_SCORE_BLOCKMAX, dev(q), NQ, dev(k), dev(lens), scale, scores)
        ref = oracle.score_blockmax(q, k, lens, scale)
        bound = oracle.score_blockmax(_abs(q), _abs(k), lens, scale)
    else:
        meta = torch.empty(B_, Hkv, nb, 2, D, dtype=torch.float32 if dtype == "f32" else torch.bfloat16, device="cuda")
        B.sparse_kv_quest_meta(shape, dev(k), dev(lens), meta)
        torch.cuda.synchronize()
        meta_ref = oracle.quest_meta(k, lens)
        got_meta = host(meta)
        got_meta64 = synth.bf16_bits_to_f32(got_meta).astype(np.float64) if dtype == "bf16" else got_meta.astype(np.float64)
        np.testing.assert_array_equal(got_meta64, meta_ref)  # min / max are exact
        B.sparse_kv_score(shape, B.SKV_SCORE_QUEST, dev(q), NQ, meta, dev(lens), scale, scores)
        ref = oracle.score_quest(q, meta_ref, lens, scale, T=T)
        box = np.maximum(np.abs(meta_ref[..., 0, :]), np.abs(meta_ref[..., 1, :]))
        abs_meta = np.stack([box, box], axis=-2)
        qa = np.abs(synth.bf16_bits_to_f32(q) if dtype == "bf16" else q).astype(np.float32)
        bound = oracle.score_quest(qa, abs_meta, lens, scale, T=T)
    torch.cuda.synchronize()
    got = host(scores).astype(np.float64)
    fin = np.isfinite(ref)
    assert np.array_equal(fin, np.isfinite(got)), "-inf pattern differs"
    assert np.all(np.isneginf(got[~fin]))
    tol = GAMMA * bound[fin] + 2.0 ** -23 * np.abs(ref[fin])
    err = np.abs(got[fin] - ref[fin])
    assert np.all(err <= tol), f"max err {err.max():.3e}, worst ratio {np.max(err / tol):.3f}"
    return float(err.max())


@pytest.mark.parametrize("dtype,D", [("f32", 64), ("f32", 128), ("bf16", 64), ("bf16", 128)])
def test_blockmax_dtypes_and_dims(dtype, D):
    _score_case(2, 8, 2, D, 256, 1, dtype, [256, 173], seed=1)


@pytest.mark.parametrize("Hq,Hkv,NQ", [(4, 4, 1), (8, 1, 1), (32, 8, 1), (32, 8, 2), (64, 8, 4), (16, 2, 3)])
def test_blockmax_group_and_draft_shapes(Hq, Hkv, NQ):
    _score_case(2, Hq, Hkv, 128, 512, NQ, "bf16", [512, 300], seed=2)


def test_blockmax_ragged_and_degenerate_lengths():
    # several workgroup chunks per row plus a ragged tail; lengths 0, 1, 15,
    # 16, 17 and full
    _score_case(6, 8, 2, 128, 1600, 1, "bf16", [0, 1, 15, 16, 17, 1600], seed=3)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_quest_bound_and_meta(dtype):
    _score_case(3, 32, 8, 128, 1024, 1, dtype, [1024, 999, 5], seed=4, mode="quest")


def test_quest_with_drafts():
    _score_case(2, 16, 2, 64, 512, 2, "bf16", [512, 260], seed=5, mode="quest")


def test_blockmax_full_size_llama8b_sampled_rows():
    # the throughput workload at full size (B=8, 32/8 heads, D=128, 32K
    # context, bf16), same launch as the benchmark; rows checked one by one
    w = synth.WORKLOADS["llama8b_32k"]
    K, _ = synth.gen_kv(w)
    q, sq = synth.gen_queries(w.scaled(steps=2))
    lens = np.full(w.batch, w.ctx, dtype=np.int32)
    shape = B.make_shape(w.batch, w.n_q_heads, w.n_kv_heads, w.head_dim, w.ctx, "bf16")
    scores = torch.empty(w.batch, w.n_kv_heads, w.nb_max, dtype=torch.float32, device="cuda")
    scale = 1.0 / math.sqrt(w.head_dim)
    log("score full-size llama8b rows", shape.batch)
    B.sparse_kv_score(shape, B.SKV_SCORE_BLOCKMAX, dev(sq[1]), 1, dev(K), dev(lens), scale, scores)
    torch.cuda.synchronize()
    got = host(scores).astype(np.float64)
    for b, j in [(0, 0), (3, 5), (7, 7)]:
        qrow = np.ascontiguousarray(sq[1][b:b + 1, :, j * w.group:(j + 1) * w.group])
        krow = np.ascontiguousarray(K[b:b + 1, j:j + 1])
        ref = oracle.score_blockmax(qrow, krow, lens[:1], scale)[0, 0]
        bound = oracle.score_blockmax(_abs(qrow), _abs(krow), lens[:1], scale)[0, 0]
        err = np.abs(got[b, j] - ref)
        assert np.all(err <= GAMMA * bound + 2.0 ** -23 * np.abs(ref)), err.max()
