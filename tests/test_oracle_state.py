"""Pins of the oracle's working-set consistency check (oracle_check_state):
hand-worked states, each breaking one rule of a block table (one resident
block per slot, ids in [-1, NB), no stamp ahead of the row's clock), with the
flags those rules give."""
import numpy as np

import oracle

NB = 10


def _check(rows):
    sb = np.array([r[0] for r in rows], np.int32)
    st = np.array([r[1] for r in rows], np.uint32)
    ck = np.array([r[2] for r in rows], np.uint32)
    return oracle.check_state(sb, st, ck, NB)


def test_each_rule_flags_its_own_bit():
    rows = [
        ([3, -1, 7, 1], [2, 0, 5, 5], 5),      # consistent: 0
        ([3, NB, 7, 1], [2, 0, 5, 5], 5),      # an id past the end: 1
        ([3, -2, 7, 1], [2, 0, 5, 5], 5),      # an id below -1: 1
        ([7, -1, 7, 1], [2, 0, 5, 5], 5),      # block 7 in two slots: 2
        ([3, -1, 7, 1], [2, 0, 6, 5], 5),      # slot 2 stamped after the clock: 4
        ([3, -1, 7, 1], [2, 9, 5, 5], 5),      # an empty slot's stamp is not checked: 0
        ([NB - 1, -1, -1, 0], [0, 0, 0, 0], 0),  # the last block id is valid, clock 0: 0
        ([4, 4, -3, -1], [1, 8, 0, 0], 7),     # all three: 1 | 2 | 4
        ([-1, -1, -1, -1], [4, 4, 4, 4], 0),   # empty row: 0
    ]
    flags, n = _check(rows)
    assert flags.tolist() == [0, 1, 1, 2, 4, 0, 0, 7, 0]
    assert n == 5


def test_stamp_equal_to_the_clock_is_consistent():
    # the slots touched by the last update carry exactly the clock's value
    flags, n = _check([([0, 1, 2, 3], [7, 7, 6, 1], 7), ([0, 1, 2, 3], [8, 7, 6, 1], 7)])
    assert flags.tolist() == [0, 4] and n == 1


def test_duplicates_anywhere_in_the_row():
    # first and last slot, and three copies
    flags, _ = _check([([5, 1, 2, 5], [0] * 4, 0), ([6, 6, 6, -1], [0] * 4, 0), ([0, 1, 2, 3], [0] * 4, 0)])
    assert flags.tolist() == [2, 2, 0]
