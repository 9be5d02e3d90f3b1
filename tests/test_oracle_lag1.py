"""Pins of the lag-1 schedule and of the working-set bound that makes it
safe to overlap.  In the lag-1 pipeline attention at step t reads the slots
of S_{t-1} while the update of step t runs; that is race-free only if the
update never evicts a block of S_{t-1}.  With LRU victims (least recent
first, S_{t-1} the most recent) and capacity C >= 2k it never does: the
update needs |S_t - S_{t-1}| <= k victims and C - |S_{t-1}| >= k slots hold
older blocks or nothing.  Checked by brute force over random and worst-case
(disjoint) selection sequences, and shown tight at C = 2k - 1."""
import numpy as np
import pytest

import oracle


def test_lagged_schedule():
    assert oracle.lagged(["a", "b", "c", "d"]) == ["a", "a", "b", "c"]
    assert oracle.lagged(["a", "b", "c"], lag=0) == ["a", "b", "c"]
    assert oracle.lagged([7]) == [7]


def _victims_of_previous(cap, k, sels, nb):
    """Steps at which the update evicts a slot holding a block of the
    previous step's selection."""
    lru = oracle.LRU(1, cap)
    bad, prev = [], set()
    for t, sel in enumerate(sels):
        before = lru.slot_block()[0].copy()
        s = np.full((1, k), -1, np.int32)
        s[0, :len(sel)] = sel
        out = lru.step(s, np.array([len(sel)], np.int32), nb)
        slots = out["miss_slot"][0, :out["miss_count"][0]]
        if any(before[x] in prev for x in slots):
            bad.append(t)
        prev = set(sel)
    return bad


@pytest.mark.parametrize("churn", [0.1, 0.5, 1.0])
def test_capacity_2k_never_evicts_the_previous_selection(churn):
    rng = np.random.default_rng(int(churn * 10))
    nb, k = 400, 24
    sels, cur = [], sorted(rng.choice(nb, k, replace=False).tolist())
    for _ in range(60):
        keep = [b for b in cur if rng.random() > churn]
        fresh = [b for b in rng.permutation(nb).tolist() if b not in cur][:k - len(keep)]
        n = int(rng.integers(k // 2, k + 1))  # short selections too
        cur = sorted(keep + fresh)[:n] if n < k else sorted(keep + fresh)
        sels.append(cur)
    assert _victims_of_previous(2 * k, k, sels, nb) == []


def test_bound_is_tight():
    # disjoint consecutive selections of k blocks: 2k slots suffice, 2k - 1 do not
    k, nb = 8, 64
    sels = [list(range(i * k, i * k + k)) for i in range(6)]
    assert _victims_of_previous(2 * k, k, sels, nb) == []
    assert _victims_of_previous(2 * k - 1, k, sels, nb) != []
