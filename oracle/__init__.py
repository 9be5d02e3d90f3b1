"""CPU oracle of the sparse KV-cache decode step (test infrastructure).

Only ``tests/``, the smoke check and the benchmark's CPU-baseline leg may
import this package.  The product path (``top_sparse_kv_block_amd``) never
does, and this package never imports the product path: the two share no
code.  The arithmetic lives in ``oracle.c`` (plain C, fp64); this module only
marshals NumPy arrays into it.  ``lru_list.py`` is a second, independent
working-set simulation in pure Python used to cross-check the C one.

Each function's docstring names the passage of the pages it follows (by page
title and section); the C source carries the same citations.
"""

from __future__ import annotations

import ctypes as C
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None


def build(verbose: bool = False) -> str:
    """Compile ``oracle.c`` into ``liboracle.so`` with gcc (-O2, OpenMP, no fast math)."""
    src = os.path.join(_HERE, "oracle.c")
    tmp = _LIB_PATH + ".tmp"
    cmd = ["gcc", "-std=c99", "-O2", "-fopenmp", "-fPIC", "-shared", "-Wall", "-Wextra",
           "-Wno-unused-parameter", src, "-o", tmp, "-lm"]
    if verbose:
        print(" ".join(cmd))
    subprocess.run(cmd, check=True)
    os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            build()
        _lib = C.CDLL(_LIB_PATH)
        _declare(_lib)
    return _lib


_i, _d, _p = C.c_int, C.c_double, C.c_void_p


def _declare(L):
    L.oracle_score_blockmax.argtypes = [_i, _i, _i, _i, _i, _i, _i, _i, _p, _p, _p, _d, _i, _p]
    L.oracle_quest_meta.argtypes = [_i, _i, _i, _i, _i, _i, _p, _p, _i, _p]
    L.oracle_score_quest.argtypes = [_i, _i, _i, _i, _i, _i, _i, _p, _p, _i, _p, _i, _d, _i, _p]
    L.oracle_topk.argtypes = [_i, _i, _i, _p, _p, _i, _i, _i, _i, _i, _p, _p]
    L.oracle_lru_create.restype = _p
    L.oracle_lru_create.argtypes = [_i, _i]
    L.oracle_lru_destroy.argtypes = [_p]
    L.oracle_lru_flush.argtypes = [_p]
    L.oracle_lru_get.argtypes = [_p, _p]
    L.oracle_lru_order.argtypes = [_p, _p]
    L.oracle_lru_load.argtypes = [_p, _p, _p]
    L.oracle_lru_step.argtypes = [_p, _i, _i, _p, _p, _p, _p, _p, _p, _p]
    L.oracle_gather.argtypes = [_i, _i, _i, _i, _i, _i, _i, _p, _p, _p, _p, _p, _p, _p]
    L.oracle_capped_step.argtypes = [_i, _i, _i, _i, _i, _p, _p, _p, _p, _p, _p, _p, _p, _p]
    L.oracle_append.argtypes = [_i, _i, _i, _i, _i, _i, _p, _p, _p, _p, _p, _p, _i, _p, _p]
    L.oracle_check_state.argtypes = [_i, _i, _i, _p, _p, _p, _p]
    L.oracle_attention.argtypes = [_i, _i, _i, _i, _i, _i, _i, _p, _p, _p, _p, _p, _i, _p, _d, _p, _p]
    L.oracle_attention_pool.argtypes = [_i, _i, _i, _i, _i, _i, _i, _p, _p, _p, _p, _p, _p, _i, _p, _d, _p, _p]


def _dt(a: np.ndarray) -> int:
    if a.dtype == np.float32:
        return 0
    if a.dtype == np.uint16:
        return 1
    raise TypeError(f"oracle takes float32 or uint16 (bf16 bits), got {a.dtype}")


def _c(a, dtype=None):
    a = np.ascontiguousarray(a, dtype=dtype) if dtype is not None else np.ascontiguousarray(a)
    return a


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(C.c_void_p)


def score_blockmax(q, k, seq_lens, scale, block=16):
    """Exact block scores, fp64.  q [B,NQ,Hq,D], k [B,Hkv,T,D] -> [B,Hkv,NB].

    Block importance = scale * max over queries, group heads and the block's
    valid tokens of q.k ("KV Cache 塞不进 HBM 了" §3 step 3 for the group max;
    OasisKV summary, key module 2 for draft-query block importance).
    """
    q, k = _c(q), _c(k)
    lens = _c(seq_lens, np.int32)
    B, NQ, Hq, D = q.shape
    _, Hkv, T, D2 = k.shape
    assert D == D2 and _dt(q) == _dt(k)
    nb = (T + block - 1) // block
    out = np.empty((B, Hkv, nb), dtype=np.float64)
    rc = lib().oracle_score_blockmax(B, NQ, Hq, Hkv, D, T, block, _dt(k), _ptr(q), _ptr(k), _ptr(lens),
                                     float(scale), nb, _ptr(out))
    assert rc == 0
    return out


def quest_meta(k, seq_lens, block=16):
    """Per-block element-wise key min/max, fp64: [B,Hkv,NB,2,D]."""
    k = _c(k)
    lens = _c(seq_lens, np.int32)
    B, Hkv, T, D = k.shape
    nb = (T + block - 1) // block
    out = np.empty((B, Hkv, nb, 2, D), dtype=np.float64)
    lib().oracle_quest_meta(B, Hkv, D, T, block, _dt(k), _ptr(k), _ptr(lens), nb, _ptr(out))
    return out


def score_quest(q, meta, seq_lens, scale, T, block=16):
    """Quest-style bound scale * max_{r,h} sum_d max(q_d min_d, q_d max_d).

    ``meta`` [B,Hkv,NB,2,D] is float32, uint16 (bf16 bits) or float64.
    """
    q = _c(q)
    lens = _c(seq_lens, np.int32)
    B, NQ, Hq, D = q.shape
    _, Hkv, nb, two, D2 = meta.shape
    assert two == 2 and D2 == D
    meta_c = _c(meta)
    mdt = 2 if meta_c.dtype == np.float64 else _dt(meta_c)
    out = np.empty((B, Hkv, nb), dtype=np.float64)
    rc = lib().oracle_score_quest(B, NQ, Hq, Hkv, D, block, _dt(q), _ptr(q), _ptr(meta_c), mdt, _ptr(lens),
                                  int(T), float(scale), nb, _ptr(out))
    assert rc == 0
    return out


def topk(scores, seq_lens, k_blocks, T, block=16, sink=0, recent=0):
    """Per-row selection under the budget (ascending ids, -1 padded) and counts.

    Budget per head per step ("KV Cache 塞不进 HBM 了" §3 step 2); sink + recent
    + top-scored (same page §2.3); order (score desc, id asc).
    """
    s = _c(scores, np.float64)
    lens = _c(seq_lens, np.int32)
    B, Hkv, nb = s.shape
    sel = np.empty((B, Hkv, k_blocks), dtype=np.int32)
    cnt = np.empty((B, Hkv), dtype=np.int32)
    rc = lib().oracle_topk(B, Hkv, nb, _ptr(s), _ptr(lens), int(T), block, k_blocks, sink, recent,
                           _ptr(sel), _ptr(cnt))
    if rc != 0:
        raise ValueError("forced blocks exceed the budget")
    return sel, cnt


class LRU:
    """Linked-list working set (C), one list per row.  See ``oracle_lru_step``."""

    def __init__(self, rows: int, cap: int):
        self.rows, self.cap = rows, cap
        self._h = lib().oracle_lru_create(rows, cap)

    def __del__(self):
        if getattr(self, "_h", None):
            lib().oracle_lru_destroy(self._h)
            self._h = None

    def flush(self):
        lib().oracle_lru_flush(self._h)

    def load(self, slot_block, slot_stamp):
        """Start every row from a given table: ``slot_block`` [rows, cap]
        int32 as given, the occupied slots ordered least recent first by
        (stamp, block id, slot) from ``slot_stamp`` [rows, cap] (uint32 or
        int32 bits): the stamp is the step of a slot's last touch, and blocks
        touched in one step count in ascending id order.  The table is not
        checked here; a step flags a row whose table is invalid."""
        sb = _c(slot_block, np.int32).reshape(self.rows, self.cap)
        st = _c(np.asarray(slot_stamp).view(np.uint32) if np.asarray(slot_stamp).dtype == np.int32
                else slot_stamp, np.uint32).reshape(self.rows, self.cap)
        lib().oracle_lru_load(self._h, _ptr(sb), _ptr(st))

    def slot_block(self):
        out = np.empty((self.rows, self.cap), dtype=np.int32)
        lib().oracle_lru_get(self._h, _ptr(out))
        return out

    def order(self):
        out = np.empty((self.rows, self.cap), dtype=np.int32)
        lib().oracle_lru_order(self._h, _ptr(out))
        return out

    def step(self, sel, sel_count, nb_limit):
        sel = _c(sel, np.int32).reshape(self.rows, -1)
        cnt = _c(sel_count, np.int32).reshape(self.rows)
        k = sel.shape[1]
        ss = np.full((self.rows, k), -1, dtype=np.int32)
        sh = np.zeros((self.rows, k), dtype=np.uint8)
        mb = np.full((self.rows, k), -1, dtype=np.int32)
        ms = np.full((self.rows, k), -1, dtype=np.int32)
        mc = np.zeros(self.rows, dtype=np.int32)
        lib().oracle_lru_step(self._h, k, int(nb_limit), _ptr(sel), _ptr(cnt), _ptr(ss), _ptr(sh), _ptr(mb),
                              _ptr(ms), _ptr(mc))
        return dict(sel_slot=ss, sel_hit=sh, miss_block=mb, miss_slot=ms, miss_count=mc)


def check_state(slot_block, slot_stamp, clock, nb_limit):
    """Per-row consistency flags of a working-set state (see
    ``oracle_check_state``): 1 = an id outside [-1, nb_limit), 2 = one block
    in two slots, 4 = an occupied slot stamped ahead of the row's clock.
    Returns (flags [rows] int32, number of flagged rows)."""
    sb = _c(slot_block, np.int32)
    rows, cap = sb.shape[0], sb.shape[-1]
    sb = sb.reshape(rows, cap)
    st = _c(np.asarray(slot_stamp).astype(np.uint32).reshape(rows, cap), np.uint32)
    ck = _c(np.asarray(clock).astype(np.uint32).reshape(rows), np.uint32)
    flags = np.empty(rows, dtype=np.int32)
    n = lib().oracle_check_state(rows, cap, int(nb_limit), _ptr(sb), _ptr(st), _ptr(ck), _ptr(flags))
    return flags, int(n)


def capped_step(slot_block, sel, sel_count, scores, nb_limit):
    """Importance-capped eviction step (OasisKV summary, key module 3): hits
    keep their slot; misses (ascending) take the empty slots by index, then
    the unselected resident slots with the lowest current score (ties: lower
    block id).  ``slot_block`` [rows, cap] int32 is updated in place; scores
    [rows, nb_max] are the step's block scores (float64).  Returns the lists
    like ``LRU.step``; a row with invalid input (a bad selection, a table id
    outside [-1, nb_limit) or a block held by two slots) gets miss_count = -1
    and padded lists and is left untouched."""
    assert slot_block.dtype == np.int32 and slot_block.flags.c_contiguous
    rows, cap = slot_block.shape
    sel = _c(sel, np.int32).reshape(rows, -1)
    cnt = _c(sel_count, np.int32).reshape(rows)
    sc = _c(scores, np.float64).reshape(rows, -1)
    k = sel.shape[1]
    ss = np.full((rows, k), -1, dtype=np.int32)
    sh = np.zeros((rows, k), dtype=np.uint8)
    mb = np.full((rows, k), -1, dtype=np.int32)
    ms = np.full((rows, k), -1, dtype=np.int32)
    mc = np.zeros(rows, dtype=np.int32)
    lib().oracle_capped_step(rows, cap, k, int(nb_limit), sc.shape[1], _ptr(sel), _ptr(cnt), _ptr(sc),
                             _ptr(slot_block), _ptr(ss), _ptr(sh), _ptr(mb), _ptr(ms), _ptr(mc))
    return dict(sel_slot=ss, sel_hit=sh, miss_block=mb, miss_slot=ms, miss_count=mc)


def append(new_k, new_v, seq_lens, k, v, slot_block=None, pool_k=None, pool_v=None, block=16):
    """Store one new token per sequence at seq_lens[b] (in place on k, v, the
    pools of resident blocks and seq_lens, which grows by one; full sequences
    are left alone).  new_k/new_v [B,Hkv,D]; k, v [B,Hkv,T,D]; slot_block
    [B*Hkv, cap] or None; pools [B,Hkv,cap,16,D]."""
    B, Hkv, T, D = k.shape
    assert k.flags.c_contiguous and v.flags.c_contiguous and seq_lens.dtype == np.int32
    nk, nv = _c(new_k, k.dtype), _c(new_v, v.dtype)
    if slot_block is None:
        sb, cap, pk, pv = None, 0, None, None
    else:
        sb = _c(slot_block, np.int32)
        cap = sb.shape[-1]
        assert pool_k.flags.c_contiguous and pool_v.flags.c_contiguous
        pk, pv = _ptr(pool_k), _ptr(pool_v)
    lib().oracle_append(B, Hkv, D, T, block, k.itemsize, _ptr(nk), _ptr(nv), _ptr(seq_lens), _ptr(k), _ptr(v),
                        None if sb is None else _ptr(sb), cap, pk, pv)


def gather(miss_block, miss_slot, miss_count, src_k, src_v, pool_k, pool_v, block=16):
    """Copy each missed block's K/V rows into its slot (in place on pool_k/pool_v)."""
    B, Hkv, T, D = src_k.shape
    rows = B * Hkv
    cap = pool_k.shape[2]
    mb = _c(miss_block, np.int32).reshape(rows, -1)
    ms = _c(miss_slot, np.int32).reshape(rows, -1)
    mc = _c(miss_count, np.int32).reshape(rows)
    assert pool_k.flags.c_contiguous and pool_v.flags.c_contiguous
    sk, sv = _c(src_k), _c(src_v)
    lib().oracle_gather(rows, cap, T, D, sk.itemsize, block, mb.shape[1], _ptr(mb), _ptr(ms), _ptr(mc),
                        _ptr(sk), _ptr(sv), _ptr(pool_k), _ptr(pool_v))


def attention(q, k, v, sel, sel_count, seq_lens, scale, block=16):
    """Softmax attention over the selected blocks read from the source, fp64.

    q [B,Hq,D]; k, v [B,Hkv,T,D]; sel [B,Hkv,kmax]; returns (out [B,Hq,D], lse [B,Hq]).
    Exact attention over the kept KV (OasisKV summary, key module 1).
    """
    q, k, v = _c(q), _c(k), _c(v)
    sel = _c(sel, np.int32)
    cnt = _c(sel_count, np.int32)
    lens = _c(seq_lens, np.int32)
    B, Hq, D = q.shape
    _, Hkv, T, _ = k.shape
    out = np.empty((B, Hq, D), dtype=np.float64)
    lse = np.empty((B, Hq), dtype=np.float64)
    rc = lib().oracle_attention(B, Hq, Hkv, D, T, block, _dt(k), _ptr(q), _ptr(k), _ptr(v), _ptr(sel), _ptr(cnt),
                                sel.shape[-1], _ptr(lens), float(scale), _ptr(out), _ptr(lse))
    assert rc == 0
    return out, lse


def attention_pool(q, pool_k, pool_v, sel, sel_slot, sel_count, seq_lens, scale, block=16):
    """Same attention read through the slot table from the pool [B,Hkv,C,block,D]."""
    q, pk, pv = _c(q), _c(pool_k), _c(pool_v)
    sel, sl = _c(sel, np.int32), _c(sel_slot, np.int32)
    cnt, lens = _c(sel_count, np.int32), _c(seq_lens, np.int32)
    B, Hq, D = q.shape
    _, Hkv, cap, blk, _ = pk.shape
    assert blk == block
    out = np.empty((B, Hq, D), dtype=np.float64)
    lse = np.empty((B, Hq), dtype=np.float64)
    rc = lib().oracle_attention_pool(B, Hq, Hkv, D, cap, block, _dt(pk), _ptr(q), _ptr(pk), _ptr(pv), _ptr(sel),
                                     _ptr(sl), _ptr(cnt), sel.shape[-1], _ptr(lens), float(scale), _ptr(out),
                                     _ptr(lse))
    assert rc == 0
    return out, lse


def lagged(per_step, lag=1):
    """The lag-1 schedule ("KV Cache 塞不进 HBM 了", §2.1 and the §3 loop: the
    forward attends over the KV readied at the previous step while the next
    retrieval runs): step t attends over the selection made at step t - lag,
    and the first steps, which have none, over step 0's.  ``per_step`` is a
    sequence indexed by step (selections, counts, ...)."""
    return [per_step[max(t - lag, 0)] for t in range(len(per_step))]
