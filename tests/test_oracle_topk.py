"""Pins of the oracle's per-row top-k selection (CPU only)."""
import numpy as np
from hypothesis import given, settings, strategies as st

import oracle
from oracle.lru_list import brute_topk


def _forced(len_, sink, recent, block=16):
    nvalid = -(-len_ // block)
    f = set()
    if sink > 0:
        f |= set(range(-(-min(sink, len_) // block)))
    if recent > 0:
        f |= set(range(max(0, len_ - recent) // block, nvalid))
    return f


@settings(max_examples=150, deadline=None)
@given(
    B=st.integers(1, 3), Hkv=st.integers(1, 3), nb=st.integers(1, 24), k=st.integers(1, 12),
    sink=st.sampled_from([0, 4, 20]), recent=st.sampled_from([0, 16, 40]),
    ties=st.booleans(), seed=st.integers(0, 2**31 - 1), data=st.data())
def test_topk_matches_python_sort(B, Hkv, nb, k, sink, recent, ties, seed, data):
    T = nb * 16
    r = np.random.default_rng(seed)
    s = r.standard_normal((B, Hkv, nb))
    if ties:
        s = np.round(s * 2) / 2  # many exact ties: tie-break by block id decides
    lens = np.array([data.draw(st.integers(0, T)) for _ in range(B)], dtype=np.int32)
    nmax_forced = (-(-sink // 16)) + (-(-recent // 16)) + (1 if recent else 0)
    if nmax_forced > k:
        sink = recent = 0
    for b in range(B):
        nvalid = -(-int(lens[b]) // 16)
        s[b, :, nvalid:] = -np.inf
    sel, cnt = oracle.topk(s, lens, k, T, sink=sink, recent=recent)
    for b in range(B):
        nvalid = -(-int(lens[b]) // 16)
        forced = _forced(int(lens[b]), sink, recent) if nvalid > k else set()
        for j in range(Hkv):
            want = brute_topk(list(s[b, j]), nvalid, k, forced)
            assert cnt[b, j] == len(want)
            assert sel[b, j, :cnt[b, j]].tolist() == want
            assert np.all(sel[b, j, cnt[b, j]:] == -1)


def test_topk_invariants_on_random_scores():
    r = np.random.default_rng(11)
    B, Hkv, nb, k = 2, 4, 300, 37
    s = r.standard_normal((B, Hkv, nb))
    lens = np.array([nb * 16, 3000], dtype=np.int32)
    s[1, :, -(-3000 // 16):] = -np.inf
    sel, cnt = oracle.topk(s, lens, k, nb * 16)
    for b in range(B):
        for j in range(Hkv):
            chosen = sel[b, j, :cnt[b, j]]
            assert cnt[b, j] == k
            assert np.all(np.diff(chosen) > 0)
            rest = np.setdiff1d(np.arange(-(-int(lens[b]) // 16)), chosen)
            assert s[b, j, chosen].min() >= s[b, j, rest].max()


def test_budget_at_least_valid_selects_everything():
    s = np.random.default_rng(12).standard_normal((1, 2, 10))
    lens = np.array([150], dtype=np.int32)  # 10 valid blocks (last one partial)
    sel, cnt = oracle.topk(s, lens, 10, 160)
    assert cnt.tolist() == [[10, 10]]
    assert sel[0, 0].tolist() == list(range(10))


def test_sink_and_recent_blocks_are_forced_and_counted_in_budget():
    # tight-budget workload shape: 4 sink tokens and 128 recent tokens kept,
    # budget 32 blocks; at a full 131072-token row that is block 0 plus the
    # last 8 blocks, leaving 23 scored picks
    nb = 8192
    s = np.linspace(1.0, 0.0, nb)[None, None, :].copy()  # block 0 would win anyway: make it lose
    s[0, 0, 0] = -100.0
    s[0, 0, -8:] = -100.0
    lens = np.array([nb * 16], dtype=np.int32)
    sel, cnt = oracle.topk(s, lens, 32, nb * 16, sink=4, recent=128)
    got = sel[0, 0, :cnt[0, 0]].tolist()
    assert cnt[0, 0] == 32
    assert got == [0] + list(range(1, 24)) + list(range(nb - 8, nb))


def test_recent_window_on_a_partial_last_block():
    # len 100: last 20 tokens are 80..99 -> blocks 5 and 6 (block 6 partial)
    s = np.zeros((1, 1, 7))
    lens = np.array([100], dtype=np.int32)
    sel, cnt = oracle.topk(s, lens, 3, 112, sink=0, recent=20)
    assert sel[0, 0, :cnt[0, 0]].tolist() == [0, 5, 6]
