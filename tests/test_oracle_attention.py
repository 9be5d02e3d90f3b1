"""Pins of the oracle's sparse attention (CPU only)."""
import json
import math
import os

import numpy as np
import torch

import oracle

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _load(name):
    with open(os.path.join(GOLD, name)) as f:
        return json.load(f)


def test_attention_hand_worked():
    g = _load("attention_hand.json")
    q = np.array(g["q"], dtype=np.float32)
    k = np.array(g["k"], dtype=np.float64).astype(np.float32)
    v = np.array(g["v"], dtype=np.float32)
    sel = np.array([[[0]]], dtype=np.int32)
    cnt = np.array([[1]], dtype=np.int32)
    for c in g["cases"]:
        lens = np.array([c["seq_len"]], dtype=np.int32)
        o, lse = oracle.attention(q, k, v, sel, cnt, lens, 1.0, block=g["block"])
        # k1 = ln 3 rounded to float32; the hand values hold to that rounding
        np.testing.assert_allclose(o[0, 0], c["out"], rtol=0, atol=1e-6)
        assert abs(lse[0, 0] - c["lse"]) < 1e-6


def _rand(B, Hq, Hkv, D, T, seed):
    r = np.random.default_rng(seed)
    q = r.standard_normal((B, Hq, D)).astype(np.float32)
    k = r.standard_normal((B, Hkv, T, D)).astype(np.float32)
    v = r.standard_normal((B, Hkv, T, D)).astype(np.float32)
    return q, k, v


def test_full_budget_is_dense_softmax_attention():
    # budget = whole context: the sparse step must be dense attention.
    # Reference: torch's scaled_dot_product_attention in float64 on the CPU
    # (default scale 1/sqrt(D)), keys of each GQA group repeated per head,
    # ragged lengths masked.
    B, Hq, Hkv, D, T = 3, 8, 2, 16, 80
    q, k, v = _rand(B, Hq, Hkv, D, T, seed=31)
    lens = np.array([80, 41, 1], dtype=np.int32)
    nb = T // 16
    sel = np.tile(np.arange(nb, dtype=np.int32), (B, Hkv, 1))
    cnt = np.full((B, Hkv), nb, dtype=np.int32)
    o, lse = oracle.attention(q, k, v, sel, cnt, lens, 1.0 / math.sqrt(D))
    G = Hq // Hkv
    tq = torch.from_numpy(q.astype(np.float64))[:, :, None, :]
    tk = torch.from_numpy(np.repeat(k, G, axis=1).astype(np.float64))
    tv = torch.from_numpy(np.repeat(v, G, axis=1).astype(np.float64))
    mask = torch.arange(T)[None, None, None, :] < torch.from_numpy(lens)[:, None, None, None]
    ref = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, attn_mask=mask)[:, :, 0]
    np.testing.assert_allclose(o, ref.numpy(), rtol=1e-12, atol=1e-12)
    logits = torch.einsum("bhd,bhtd->bht", tq[:, :, 0], tk) / math.sqrt(D)
    logits = logits.masked_fill(~mask[:, :, 0], -math.inf)
    np.testing.assert_allclose(lse, torch.logsumexp(logits, dim=-1).numpy(), rtol=1e-12, atol=1e-12)


def test_sparse_selection_equals_dense_attention_on_the_kept_tokens():
    B, Hq, Hkv, D, T = 1, 4, 1, 8, 128
    q, k, v = _rand(B, Hq, Hkv, D, T, seed=32)
    lens = np.array([128], dtype=np.int32)
    S = [1, 4, 6]
    sel = np.array([[S]], dtype=np.int32)
    cnt = np.array([[3]], dtype=np.int32)
    o, _ = oracle.attention(q, k, v, sel, cnt, lens, 0.35)
    idx = np.concatenate([np.arange(16 * b, 16 * b + 16) for b in S])
    tq = torch.from_numpy(q.astype(np.float64))[:, :, None, :]
    tk = torch.from_numpy(np.repeat(k[:, :, idx], Hq, axis=1).astype(np.float64))
    tv = torch.from_numpy(np.repeat(v[:, :, idx], Hq, axis=1).astype(np.float64))
    ref = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, scale=0.35)[:, :, 0]
    np.testing.assert_allclose(o, ref.numpy(), rtol=1e-12, atol=1e-12)


def test_equal_logits_give_mean_of_values():
    B, Hq, Hkv, D, T = 1, 2, 1, 8, 64
    _, k, v = _rand(B, Hq, Hkv, D, T, seed=33)
    q = np.zeros((B, Hq, D), dtype=np.float32)
    sel = np.array([[[0, 2]]], dtype=np.int32)
    cnt = np.array([[2]], dtype=np.int32)
    lens = np.array([64], dtype=np.int32)
    o, lse = oracle.attention(q, k, v, sel, cnt, lens, 1.0)
    mean = np.concatenate([v[0, 0, 0:16], v[0, 0, 32:48]]).astype(np.float64).mean(axis=0)
    np.testing.assert_allclose(o[0, 0], mean, rtol=1e-13, atol=1e-13)
    assert abs(lse[0, 0] - math.log(32)) < 1e-13


def test_no_valid_token_gives_zero_output():
    q, k, v = _rand(1, 2, 1, 4, 32, seed=34)
    o, lse = oracle.attention(q, k, v, np.array([[[1]]], dtype=np.int32), np.array([[1]], dtype=np.int32),
                              np.array([10], dtype=np.int32), 1.0)
    assert not o.any() and np.all(np.isneginf(lse))


def test_block_table_indirection_example():
    # the block-table figure's mapping: logical blocks 0..3 live in physical
    # slots 7, 3, 11, 5; attention read through the table equals attention
    # read from the logically contiguous cache
    g = _load("block_table.json")
    phys = g["logical_to_physical"]
    B, Hq, Hkv, D, T = 1, 4, 1, 8, g["tokens"]
    q, k, v = _rand(B, Hq, Hkv, D, T, seed=35)
    cap = 12
    pk = np.zeros((B, Hkv, cap, 16, D), dtype=np.float32)
    pv = np.zeros_like(pk)
    for lb, pb in enumerate(phys):
        pk[0, 0, pb] = k[0, 0, 16 * lb:16 * lb + 16]
        pv[0, 0, pb] = v[0, 0, 16 * lb:16 * lb + 16]
    sel = np.array([[[0, 1, 2, 3]]], dtype=np.int32)
    slot = np.array([[phys]], dtype=np.int32)
    cnt = np.array([[4]], dtype=np.int32)
    lens = np.array([61], dtype=np.int32)
    o_src, l_src = oracle.attention(q, k, v, sel, cnt, lens, 0.5)
    o_pool, l_pool = oracle.attention_pool(q, pk, pv, sel, slot, cnt, lens, 0.5)
    np.testing.assert_allclose(o_pool, o_src, rtol=1e-13, atol=1e-13)
    np.testing.assert_allclose(l_pool, l_src, rtol=1e-13, atol=1e-13)
    wrong = np.array([[[7, 3, 5, 11]]], dtype=np.int32)
    o_bad, _ = oracle.attention_pool(q, pk, pv, sel, wrong, cnt, lens, 0.5)
    assert np.abs(o_bad - o_src).max() > 1e-3


def test_working_set_path_is_exact():
    # Blocks fetched into the working set and read back through the slot
    # table give the same output as reading them from the source (the tier
    # does not change the result: HiSparse promo, insight 1)
    r = np.random.default_rng(36)
    B, Hq, Hkv, D, T, cap, k = 2, 8, 2, 16, 256, 6, 4
    q, kk, vv = _rand(B, Hq, Hkv, D, T, seed=37)
    lens = np.array([256, 200], dtype=np.int32)
    lru = oracle.LRU(B * Hkv, cap)
    pk = np.zeros((B, Hkv, cap, 16, D), dtype=np.float32)
    pv = np.zeros_like(pk)
    for step in range(6):
        sel = np.stack([np.sort(r.choice(-(-int(lens[b]) // 16), size=k, replace=False))
                        for b in range(B) for _ in range(Hkv)]).astype(np.int32).reshape(B, Hkv, k)
        cnt = np.full((B, Hkv), k, dtype=np.int32)
        out = lru.step(sel.reshape(B * Hkv, k), cnt.reshape(-1), 16)
        oracle.gather(out["miss_block"], out["miss_slot"], out["miss_count"], kk, vv, pk, pv)
        o1, l1 = oracle.attention(q, kk, vv, sel, cnt, lens, 0.25)
        o2, l2 = oracle.attention_pool(q, pk, pv, sel, out["sel_slot"].reshape(B, Hkv, k), cnt, lens, 0.25)
        np.testing.assert_allclose(o2, o1, rtol=1e-13, atol=1e-13)
        np.testing.assert_allclose(l2, l1, rtol=1e-13, atol=1e-13)
