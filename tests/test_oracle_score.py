"""Pins of the oracle's block scoring (CPU only).

Each test ties the oracle to something other than its own formula: a worked
example, a library routine in a special case, or an invariant the method
fixes.
"""
import json
import math
import os

import numpy as np
import pytest

import oracle
from top_sparse_kv_block_amd import synth

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _load(name):
    with open(os.path.join(GOLD, name)) as f:
        return json.load(f)


def _f(x):
    return -math.inf if x == "-inf" else float(x)


def test_score_hand_worked():
    g = _load("score_hand.json")
    q = np.array(g["q"], dtype=np.float32)
    q2 = np.array(g["q_two_drafts"], dtype=np.float32)
    k = np.array(g["k"], dtype=np.float32)
    for c in g["cases"]:
        lens = np.array([c["seq_len"]], dtype=np.int32)
        s = oracle.score_blockmax(q, k, lens, c["scale"], block=g["block"])[0, 0]
        assert s.tolist() == [_f(x) for x in c["exact"]]
        if "quest" in c:
            meta = oracle.quest_meta(k, lens, block=g["block"])
            sq = oracle.score_quest(q, meta, lens, c["scale"], T=k.shape[2], block=g["block"])[0, 0]
            assert sq.tolist() == [_f(x) for x in c["quest"]]
        if "exact_two_drafts" in c:
            s2 = oracle.score_blockmax(q2, k, lens, c["scale"], block=g["block"])[0, 0]
            assert s2.tolist() == [_f(x) for x in c["exact_two_drafts"]]


def _rand(B=2, NQ=1, Hq=4, Hkv=2, D=8, T=40, seed=0, dtype=np.float32):
    r = np.random.default_rng(seed)
    q = r.standard_normal((B, NQ, Hq, D)).astype(np.float32)
    k = r.standard_normal((B, Hkv, T, D)).astype(np.float32)
    return q, k


def test_single_token_blocks_reduce_to_matmul():
    # block size 1, one query, one head per kv head: the score table is the
    # plain matrix product scale * q K^T (NumPy matmul, not the oracle's loop)
    q, k = _rand(B=2, NQ=1, Hq=3, Hkv=3, D=16, T=24, seed=1)
    lens = np.array([24, 24], dtype=np.int32)
    s = oracle.score_blockmax(q, k, lens, 0.25, block=1)
    ref = 0.25 * np.matmul(q[:, 0, :, None, :].astype(np.float64), np.swapaxes(k, -1, -2).astype(np.float64))[:, :, 0]
    np.testing.assert_allclose(s, ref, rtol=1e-13, atol=1e-13)


def test_block_score_is_max_pool_of_token_scores():
    q, k = _rand(B=1, NQ=1, Hq=2, Hkv=2, D=16, T=64, seed=2)
    lens = np.array([64], dtype=np.int32)
    tok = 0.5 * np.matmul(q[:, 0, :, None, :].astype(np.float64), np.swapaxes(k, -1, -2).astype(np.float64))[:, :, 0]
    s = oracle.score_blockmax(q, k, lens, 0.5, block=16)
    np.testing.assert_allclose(s, tok.reshape(1, 2, 4, 16).max(-1), rtol=1e-13, atol=1e-13)


def test_group_score_is_elementwise_max_over_heads():
    # GQA: the group's score is the element-wise max of the per-head scores
    # ("KV Cache 塞不进 HBM 了" §3 step 3).  Per-head scores come from an MHA
    # call on K repeated per head.
    q, k = _rand(B=2, NQ=1, Hq=8, Hkv=2, D=8, T=48, seed=3)
    lens = np.array([48, 37], dtype=np.int32)
    G = 4
    s = oracle.score_blockmax(q, k, lens, 0.3)
    k_rep = np.repeat(k, G, axis=1)
    per_head = oracle.score_blockmax(q, k_rep, lens, 0.3)
    np.testing.assert_array_equal(s, per_head.reshape(2, 2, G, -1).max(axis=2))


def test_mqa_and_mha_special_cases():
    q, k = _rand(B=1, NQ=1, Hq=4, Hkv=1, D=8, T=32, seed=4)
    lens = np.array([32], dtype=np.int32)
    mqa = oracle.score_blockmax(q, k, lens, 1.0)
    heads = [oracle.score_blockmax(q[:, :, h:h + 1], k, lens, 1.0) for h in range(4)]
    np.testing.assert_array_equal(mqa, np.max(np.stack(heads), axis=0))


def test_zero_noise_drafts_equal_single_query():
    q, k = _rand(B=2, NQ=1, Hq=4, Hkv=2, D=8, T=64, seed=5)
    lens = np.array([64, 50], dtype=np.int32)
    q4 = np.repeat(q, 4, axis=1)
    np.testing.assert_array_equal(oracle.score_blockmax(q4, k, lens, 0.7), oracle.score_blockmax(q, k, lens, 0.7))


def test_drafts_take_the_max_over_queries():
    q, k = _rand(B=1, NQ=3, Hq=2, Hkv=1, D=8, T=32, seed=6)
    lens = np.array([32], dtype=np.int32)
    s = oracle.score_blockmax(q, k, lens, 1.0)
    per = [oracle.score_blockmax(q[:, r:r + 1], k, lens, 1.0) for r in range(3)]
    np.testing.assert_array_equal(s, np.max(np.stack(per), axis=0))


def test_invalid_and_partial_blocks():
    q, k = _rand(B=3, NQ=1, Hq=2, Hkv=1, D=4, T=64, seed=7)
    lens = np.array([64, 17, 0], dtype=np.int32)
    s = oracle.score_blockmax(q, k, lens, 1.0)
    assert np.all(np.isfinite(s[0, 0]))
    assert np.all(np.isfinite(s[1, 0, :2])) and np.all(np.isneginf(s[1, 0, 2:]))
    assert np.all(np.isneginf(s[2, 0]))
    # block 1 of sequence 1 has one valid token: its score ignores tokens 17..31
    one = max(float(np.dot(q[1, 0, h].astype(np.float64), k[1, 0, 16].astype(np.float64))) for h in range(2))
    assert s[1, 0, 1] == one


def test_quest_bound_dominates_and_is_tight_for_single_token_blocks():
    q, k = _rand(B=2, NQ=2, Hq=4, Hkv=2, D=16, T=80, seed=8)
    lens = np.array([80, 53], dtype=np.int32)
    exact = oracle.score_blockmax(q, k, lens, 0.25)
    bound = oracle.score_quest(q, oracle.quest_meta(k, lens), lens, 0.25, T=80)
    fin = np.isfinite(exact)
    assert np.array_equal(fin, np.isfinite(bound))
    assert np.all(bound[fin] >= exact[fin] - 1e-12)
    e1 = oracle.score_blockmax(q, k, lens, 0.25, block=1)
    b1 = oracle.score_quest(q, oracle.quest_meta(k, lens, block=1), lens, 0.25, T=80, block=1)
    np.testing.assert_allclose(b1, e1, rtol=1e-12, atol=1e-12)


def test_quest_meta_is_blockwise_min_max():
    _, k = _rand(B=1, Hkv=2, D=8, T=48, seed=9)
    lens = np.array([40], dtype=np.int32)
    m = oracle.quest_meta(k, lens)
    kk = k.astype(np.float64)
    np.testing.assert_array_equal(m[0, :, 0, 0], kk[0, :, 0:16].min(axis=1))
    np.testing.assert_array_equal(m[0, :, 2, 1], kk[0, :, 32:40].max(axis=1))


def test_bf16_inputs_widen_exactly():
    q, k = _rand(B=1, NQ=1, Hq=2, Hkv=1, D=8, T=32, seed=10)
    qb, kb = synth.f32_to_bf16_bits(q), synth.f32_to_bf16_bits(k)
    lens = np.array([32], dtype=np.int32)
    s_b = oracle.score_blockmax(qb, kb, lens, 1.0)
    s_f = oracle.score_blockmax(synth.bf16_bits_to_f32(qb), synth.bf16_bits_to_f32(kb), lens, 1.0)
    np.testing.assert_array_equal(s_b, s_f)


def test_bf16_rounding_is_nearest_even():
    x = np.array([1.0, 1.00390625, 1.01171875, -2.5, 3.0e38], dtype=np.float32)
    # 1 + 2^-8 is a tie between 1 and 1+2^-7 -> even (1.0); 1 + 3*2^-8 ties up to 1 + 2^-6
    got = synth.bf16_bits_to_f32(synth.f32_to_bf16_bits(x))
    assert got[0] == 1.0 and got[1] == 1.0 and got[2] == 1.015625 and got[3] == -2.5
