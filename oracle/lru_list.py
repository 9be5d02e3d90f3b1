"""Pure-Python working-set simulation (test infrastructure).

A second, independent implementation of the working-set step of the C oracle
(``oracle_lru_step``), written with ``collections.OrderedDict`` as the LRU
list, and a brute-force top-k with Python's ``sorted``.  The tests run both
against the C oracle so that a slip in either shows up as a disagreement.

Policy (HiSparse promo, insights 1-2: a fixed-size GPU working set managed
LRU, hit detection + replacement + fetch in one pass; "KV Cache 塞不进 HBM 了"
§2.1 / §3 step 1: only the difference selected - resident moves):

* hits keep their slot; misses (ascending block id) take victims;
* victims are the empty slots in ascending slot order, then resident slots
  from the least recently used end whose block is not selected;
* afterwards every selected block is touched in ascending block order.

A step refuses (returns None and changes nothing) a selection that is not
strictly ascending, too long or out of range, and a slot table that holds
an id out of range or one block in two slots (the table maps each resident
block to one slot: KV-Cache 压缩技术的工程原理 §5.2).
"""

from __future__ import annotations

import heapq
from collections import OrderedDict


class ListLRU:
    def __init__(self, cap: int):
        self.cap = cap
        self.slot_block = [-1] * cap
        self.lru: "OrderedDict[int, None]" = OrderedDict()  # slot -> None, LRU first

    def flush(self):
        self.slot_block = [-1] * self.cap
        self.lru.clear()

    def load(self, slot_block, last_touch):
        """Start from a given table; ``last_touch[s]`` is the step at which
        slot s was last touched (blocks touched in one step count in
        ascending id order)."""
        self.slot_block = [int(b) for b in slot_block]
        occupied = [s for s in range(self.cap) if self.slot_block[s] >= 0]
        occupied.sort(key=lambda s: (int(last_touch[s]), self.slot_block[s], s))
        self.lru = OrderedDict((s, None) for s in occupied)

    def step(self, S, nb_limit=None):
        """Apply one selection; returns (sel_slot, sel_hit, misses[(block, slot)]) or None if invalid."""
        S = list(S)
        if len(S) > self.cap:
            return None
        if any(b < 0 or (nb_limit is not None and b >= nb_limit) for b in S):
            return None
        if any(S[i] <= S[i - 1] for i in range(1, len(S))):
            return None
        resident = [b for b in self.slot_block if b != -1]
        if any(b < -1 or (nb_limit is not None and b >= nb_limit) for b in self.slot_block):
            return None
        if len(set(resident)) != len(resident):
            return None
        where = {b: s for s, b in enumerate(self.slot_block) if b >= 0}
        chosen = set(S)
        sel_slot = [where.get(b, -1) for b in S]
        sel_hit = [int(s >= 0) for s in sel_slot]
        misses = [b for b, s in zip(S, sel_slot) if s < 0]
        victims = [s for s in range(self.cap) if self.slot_block[s] < 0]
        victims += [s for s in self.lru if self.slot_block[s] not in chosen]
        victims = victims[: len(misses)]
        assert len(victims) == len(misses)
        out_misses = []
        vi = 0
        for i, b in enumerate(S):
            if sel_slot[i] < 0:
                v = victims[vi]
                vi += 1
                self.lru.pop(v, None)
                self.slot_block[v] = b
                sel_slot[i] = v
                out_misses.append((b, v))
        for s in sel_slot:  # ascending block order
            self.lru.pop(s, None)
            self.lru[s] = None
        return sel_slot, sel_hit, out_misses


class HeapCapped:
    """Importance-capped working set with a priority queue (OasisKV summary,
    key module 3: when the capped cache has no room, the least important
    blocks go).  Victims: empty slots by index (a heap of slot numbers), then
    resident unselected blocks by (current score, block id) from a heap."""

    def __init__(self, cap: int):
        self.cap = cap
        self.slot_block = [-1] * cap

    def step(self, S, scores):
        """scores: mapping block -> current score.  Returns (sel_slot, sel_hit, misses[(block, slot)])."""
        S = list(S)
        where = {b: s for s, b in enumerate(self.slot_block) if b >= 0}
        chosen = set(S)
        sel_slot = [where.get(b, -1) for b in S]
        sel_hit = [int(s >= 0) for s in sel_slot]
        empty = [s for s in range(self.cap) if self.slot_block[s] < 0]
        heapq.heapify(empty)
        resident = [(scores[b], b, s) for s, b in enumerate(self.slot_block) if b >= 0 and b not in chosen]
        heapq.heapify(resident)
        out_misses = []
        for i, b in enumerate(S):
            if sel_slot[i] >= 0:
                continue
            v = heapq.heappop(empty) if empty else heapq.heappop(resident)[2]
            self.slot_block[v] = b
            sel_slot[i] = v
            out_misses.append((b, v))
        return sel_slot, sel_hit, out_misses


def brute_topk(scores, n_valid, k, forced=()):
    """Top-k by Python sort on (score desc, id asc) plus forced ids, ascending."""
    if n_valid <= k:
        return list(range(n_valid))
    forced = sorted(set(forced))
    rest = [(-scores[i], i) for i in range(n_valid) if i not in set(forced)]
    rest = sorted(rest)[: max(0, k - len(forced))]
    return sorted(forced + [i for _, i in rest])
