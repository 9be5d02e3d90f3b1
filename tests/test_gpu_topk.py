"""GPU parity of stage 2 (per-row top-k) against the oracle.

Given the same float32 scores the selection is an integer result decided in
the kernel's precision, so the oracle runs on the GPU's own scores (widened
exactly to fp64) and the sets must match bit for bit.
"""
import numpy as np
import pytest
import torch

import oracle
from top_sparse_kv_block_amd import binding as B
from gpu_util import dev, host, log

pytestmark = pytest.mark.gpu


def _run(scores, lens, k, sink=0, recent=0, Hkv=None):
    B_, hkv, nb = scores.shape
    shape = B.make_shape(B_, hkv, hkv, 64, nb * 16, "f32")
    sel = torch.empty(B_, hkv, k, dtype=torch.int32, device="cuda")
    cnt = torch.empty(B_, hkv, dtype=torch.int32, device="cuda")
    wsb = B.sparse_kv_topk_workspace_bytes(shape, k)
    assert (wsb > 0) == (nb > 16384)
    ws = torch.empty(wsb, dtype=torch.uint8, device="cuda") if wsb else None
    log("topk", (B_, hkv, nb), "k", k, "sink", sink, "recent", recent)
    B.sparse_kv_topk(shape, dev(scores.astype(np.float32)), dev(np.asarray(lens, np.int32)), k, sink, recent, sel, cnt,
                     ws)
    torch.cuda.synchronize()
    ref_sel, ref_cnt = oracle.topk(scores.astype(np.float32).astype(np.float64), np.asarray(lens, np.int32), k,
                                   nb * 16, sink=sink, recent=recent)
    np.testing.assert_array_equal(host(cnt), ref_cnt)
    np.testing.assert_array_equal(host(sel), ref_sel)


@pytest.mark.parametrize("nb,k", [(64, 8), (2048, 128), (3000, 100), (8192, 32), (20000, 300), (65536, 128)])
def test_topk_random_scores(nb, k):
    r = np.random.default_rng(nb + k)
    s = r.standard_normal((2, 3, nb)).astype(np.float32)
    _run(s, [nb * 16, nb * 16 - 100], k)


def test_topk_heavy_ties_break_to_lower_ids():
    r = np.random.default_rng(7)
    s = (np.round(r.standard_normal((2, 4, 2048)) * 2) / 2).astype(np.float32)  # few distinct values
    s[1, 0, :] = 1.0  # a whole row of equal scores: the lowest ids win
    s[1, 1, :] = 0.0
    s[1, 1, ::2] = -0.0  # signed zeros compare equal
    _run(s, [32768, 32768], 128)


def test_topk_ragged_lengths_and_small_rows():
    r = np.random.default_rng(8)
    s = r.standard_normal((6, 2, 1024)).astype(np.float32)
    _run(s, [0, 1, 100, 16 * 130, 16 * 129 + 1, 16 * 1024], 130)


@pytest.mark.parametrize("sink,recent", [(4, 128), (20, 0), (0, 40), (16, 17)])
def test_topk_sink_and_recent(sink, recent):
    r = np.random.default_rng(9)
    s = r.standard_normal((3, 2, 8192)).astype(np.float32)
    s[:, :, 0] = -50  # forced blocks must be kept whatever their score
    _run(s, [131072, 131072 - 5, 1000], 32, sink=sink, recent=recent)


# Budgets of at most four keys per wave first bound the threshold from below
# with each wave's m-th largest lane maximum; the cases put ties at the
# threshold, the best blocks in one lane (contiguous ids), waves without any
# candidate (short valid parts, forced ranges) and -inf scores against it.
@pytest.mark.parametrize("nb", [2048, 8192, 16384])
@pytest.mark.parametrize("k", [1, 5, 17, 32, 33, 64])
def test_topk_small_budgets(nb, k):
    r = np.random.default_rng(nb * 7 + k)
    s = r.standard_normal((2, 4, nb)).astype(np.float32)
    s[0, 1] = np.round(s[0, 1] * 2) / 2  # few distinct values: ties at the threshold
    s[0, 2, 100:140] = 9.0 + r.random(40).astype(np.float32)  # the best blocks in one or two lanes
    s[0, 3, :] = 1.0
    s[0, 3, 5 * nb // 8:] = 2.0  # the best keys all in the last waves, equal
    s[1, 0, ::3] = -np.inf
    s[1, 1, :] = -np.inf
    s[1, 1, 7::97] = r.standard_normal(len(range(7, nb, 97))).astype(np.float32)
    _run(s, [nb * 16, 16 * min(nb, 600) + 3], k)
    _run(s, [nb * 16 - 5, nb * 16], k, sink=16 * (k // 8), recent=16 * (k // 3))


def test_topk_rejects_too_many_forced_blocks():
    shape = B.make_shape(1, 1, 1, 64, 1024, "f32")
    t = lambda *a, **kw: torch.zeros(*a, device="cuda", **kw)
    with pytest.raises(B.SparseKVError) as e:
        B.sparse_kv_topk(shape, t(1, 1, 64), t(1, dtype=torch.int32), 4, 16, 64, t(1, 1, 4, dtype=torch.int32),
                         t(1, 1, dtype=torch.int32))
    assert e.value.status == 4


# Rows longer than 16384 blocks are selected in two launches: each chunk of
# 1024, 2048 or 4096 blocks keeps its best blocks in the workspace, then one
# workgroup per row selects from those.  The cases cover every chunk size,
# 4, 8 and 32 candidates per thread in the second launch, a row length not a
# multiple of 4 (scalar loads), a budget not a multiple of 4 (padded chunk
# stride) and k = 1.
@pytest.mark.parametrize("nb,k", [(16385, 64), (32768, 1024), (65536, 128), (65536, 1), (65536, 1024),
                                  (65536, 256), (65536, 257), (65536, 400), (50001, 301)])
def test_topk_long_rows(nb, k):
    r = np.random.default_rng(nb * 7 + k)
    s = r.standard_normal((1, 3, nb)).astype(np.float32)
    s[0, 2, 100:5000] += 6.0  # a dense cluster of high scores in one row
    _run(s, [nb * 16], k)


def test_topk_long_rows_ties_and_fallback():
    r = np.random.default_rng(11)
    nb = 65536
    s = (np.round(r.standard_normal((1, 4, nb)) * 64) / 64).astype(np.float32)  # ties near the threshold
    s[0, 1, :] = 2.0  # all equal: every key reaches the bound -> fallback, lowest ids win
    s[0, 2, :] = (np.arange(nb) % 3).astype(np.float32)  # a third of the row ties at the top
    _run(s, [nb * 16], 128)


def test_topk_long_rows_ragged_sink_recent():
    r = np.random.default_rng(12)
    nb = 40000
    s = r.standard_normal((4, 2, nb)).astype(np.float32)
    s[:, :, 0] = -50
    _run(s, [nb * 16, nb * 16 - 7, 16 * 129 + 3, 16 * 40], 128, sink=4, recent=128)


def test_topk_long_rows_infinite_scores():
    # -inf scores of valid blocks are real candidates: they tie with each
    # other (lowest ids first) and never lose to a chunk's padding
    r = np.random.default_rng(14)
    nb = 40000
    s = r.standard_normal((1, 3, nb)).astype(np.float32)
    s[0, 0, :] = -np.inf
    s[0, 0, 30000:30050] = 1.0     # 50 finite scores, the rest of the budget from -inf ties
    s[0, 1, ::2] = -np.inf         # every other block
    s[0, 2, :] = -np.inf
    s[0, 2, 5] = np.inf
    _run(s, [nb * 16], 128)
    _run(s, [nb * 16], 128, sink=16, recent=64)


def test_topk_long_rows_workspace_checked():
    nb, k = 20000, 64
    shape = B.make_shape(1, 1, 1, 64, nb * 16, "f32")
    need = B.sparse_kv_topk_workspace_bytes(shape, k)
    assert need == 1 * 20 * k * 8  # ceil(20000 / 1024) chunks of k (score, id) pairs
    sc = torch.zeros(1, 1, nb, device="cuda")
    lens = torch.full((1,), nb * 16, dtype=torch.int32, device="cuda")
    sel = torch.empty(1, 1, k, dtype=torch.int32, device="cuda")
    cnt = torch.empty(1, 1, dtype=torch.int32, device="cuda")
    for ws in (None, torch.empty(need - 8, dtype=torch.uint8, device="cuda")):
        with pytest.raises(B.SparseKVError) as e:
            B.sparse_kv_topk(shape, sc, lens, k, 0, 0, sel, cnt, ws)
        assert e.value.status == 5


def test_topk_long_rows_short_valid_lengths():
    # long allocated rows whose valid part is short: chunks past the valid
    # length write nothing and the second launch reads only the chunks that
    # hold valid blocks
    r = np.random.default_rng(13)
    nb = 65536
    s = r.standard_normal((6, 1, nb)).astype(np.float32)
    _run(s, [16 * 130, 16 * 129 + 5, 16 * 300, 16 * 1000 + 1, 16 * 4100, 16 * 128 + 16], 128, sink=4, recent=128)
    _run(s, [16 * 130, 16 * 129 + 5, 16 * 300, 16 * 1000 + 1, 16 * 4100, 16 * 128 + 16], 120)
    # rows of at most k valid blocks take them all (no candidates read), an
    # empty row takes none, and a row whose valid part ends inside a chunk
    _run(s, [0, 16 * 50, 16 * 128, 16 * 128 - 3, 16 * 1024 + 1, 16 * 2048 - 1], 128, sink=4, recent=128)
