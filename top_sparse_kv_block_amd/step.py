"""One sparse decode step for one attention layer, on top of the C ABI.

:class:`LayerBuffers` owns the device buffers of one layer (torch allocates
them; torch is only the allocator and the stream provider here) and
:func:`decode_step` enqueues the four library calls on the current stream:
score -> top-k -> cache update (+ miss fetch) -> sparse attention.  Nothing
here computes; there is no host synchronisation inside a step.
"""

from __future__ import annotations

import math
from dataclasses import dataclass

import torch

from . import binding as B


@dataclass
class StepConfig:
    batch: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    max_ctx: int
    dtype: str  # "f32" | "bf16"
    k_blocks: int
    capacity: int
    mode: int = B.SKV_SCORE_BLOCKMAX
    n_queries: int = 1
    sink: int = 0
    recent: int = 0
    num_splits: int = 0
    scale: float | None = None

    @property
    def shape(self) -> B.skv_shape:
        return B.make_shape(self.batch, self.n_q_heads, self.n_kv_heads, self.head_dim, self.max_ctx, self.dtype)

    @property
    def torch_dtype(self):
        return torch.float32 if self.dtype == "f32" else torch.bfloat16

    @property
    def nb(self) -> int:
        return self.max_ctx // 16

    @property
    def softmax_scale(self) -> float:
        return self.scale if self.scale is not None else 1.0 / math.sqrt(self.head_dim)


class LayerBuffers:
    """Selection, working-set state, pool, outputs and workspace of one layer."""

    def __init__(self, cfg: StepConfig, device="cuda", pool=True):
        self.cfg = cfg
        self.shape = cfg.shape
        b, hkv, hq, d, k, c = cfg.batch, cfg.n_kv_heads, cfg.n_q_heads, cfg.head_dim, cfg.k_blocks, cfg.capacity
        i32 = dict(dtype=torch.int32, device=device)
        self.scores = torch.empty(b, hkv, cfg.nb, dtype=torch.float32, device=device)
        self.sel_blocks = torch.empty(b, hkv, k, **i32)
        self.sel_count = torch.empty(b, hkv, **i32)
        self.slot_block = torch.full((b, hkv, c), -1, **i32)
        self.slot_stamp = torch.zeros(b, hkv, c, **i32)
        self.clock = torch.zeros(b, hkv, **i32)
        self.sel_slot = torch.empty(b, hkv, k, **i32)
        self.sel_hit = torch.empty(b, hkv, k, dtype=torch.uint8, device=device)
        self.miss_block = torch.empty(b, hkv, k, **i32)
        self.miss_slot = torch.empty(b, hkv, k, **i32)
        self.miss_count = torch.empty(b, hkv, **i32)
        if pool:
            self.pool_k = torch.zeros(b, hkv, c, 16, d, dtype=cfg.torch_dtype, device=device)
            self.pool_v = torch.zeros(b, hkv, c, 16, d, dtype=cfg.torch_dtype, device=device)
        else:
            self.pool_k = self.pool_v = None
        self.out = torch.empty(b, hq, d, dtype=torch.float32, device=device)
        self.lse = torch.empty(b, hq, dtype=torch.float32, device=device)
        self.splits = cfg.num_splits or B.sparse_decode_attention_splits(self.shape, k)
        self.fused_splits = cfg.num_splits or B.sparse_kv_select_attend_splits(self.shape, k)
        # one workspace for the attention and the fused call (partials and,
        # past 16384 blocks, the top-k's chunk candidates)
        ws = B.sparse_kv_workspace_bytes(self.shape, k, cfg.num_splits)
        self.workspace = torch.empty(max(ws, 256), dtype=torch.uint8, device=device)
        # the top-k's own workspace (rows over 16384 blocks), apart from the
        # attention's so that a selection may run on another stream
        tk = B.sparse_kv_topk_workspace_bytes(self.shape, k)
        self.topk_workspace = torch.empty(tk, dtype=torch.uint8, device=device) if tk else None

    def reset(self):
        """Empty working set (slot table -1, stamps and clock 0)."""
        self.slot_block.fill_(-1)
        self.slot_stamp.zero_()
        self.clock.zero_()

    # stage wrappers -------------------------------------------------------
    def score(self, score_q, keys_or_meta, seq_lens, stream=None):
        c = self.cfg
        B.sparse_kv_score(self.shape, c.mode, score_q, c.n_queries, keys_or_meta, seq_lens, c.softmax_scale,
                          self.scores, stream)

    def topk(self, seq_lens, stream=None):
        c = self.cfg
        B.sparse_kv_topk(self.shape, self.scores, seq_lens, c.k_blocks, c.sink, c.recent, self.sel_blocks,
                         self.sel_count, self.topk_workspace, stream)

    def cache_update(self, src_k, src_v, src_kind=B.SKV_SRC_DEVICE, stream=None, importance=False):
        """importance=True evicts by this step's scores (in self.scores) instead of LRU."""
        c = self.cfg
        if importance:
            B.sparse_kv_cache_update_importance(self.shape, c.k_blocks, c.capacity, self.sel_blocks, self.sel_count,
                                                self.scores, self.slot_block, self.slot_stamp, self.clock,
                                                self.sel_slot, self.sel_hit, self.miss_block, self.miss_slot,
                                                self.miss_count, src_k, src_v, src_kind, self.pool_k, self.pool_v,
                                                stream)
            return
        B.sparse_kv_cache_update(self.shape, c.k_blocks, c.capacity, self.sel_blocks, self.sel_count, self.slot_block,
                                 self.slot_stamp, self.clock, self.sel_slot, self.sel_hit, self.miss_block,
                                 self.miss_slot, self.miss_count, src_k, src_v, src_kind, self.pool_k, self.pool_v,
                                 stream)

    def select(self, seq_lens, src_k=None, src_v=None, src_kind=B.SKV_SRC_DEVICE, stream=None, lists=None):
        """Top-k and working-set update (LRU) in one launch; ``lists`` (an
        object with the list attributes, default self) receives the
        selection and the lists."""
        c, o = self.cfg, lists if lists is not None else self
        B.sparse_kv_select(self.shape, self.scores, seq_lens, c.k_blocks, c.sink, c.recent, c.capacity, o.sel_blocks,
                           o.sel_count, self.slot_block, self.slot_stamp, self.clock, o.sel_slot, o.sel_hit,
                           o.miss_block, o.miss_slot, o.miss_count, src_k, src_v, src_kind, self.pool_k, self.pool_v,
                           self.topk_workspace, stream)

    def prefetch(self, hint: "LayerBuffers", src_k, src_v, src_kind=B.SKV_SRC_DEVICE, stream=None):
        """Cross-layer prefetch: an ordinary working-set update of this layer
        with another layer's selection (hint.sel_blocks / hint.sel_count) as
        the pick, fetching its misses from this layer's source.  Blocks the
        layers share are then hits for this layer's own update.  Its lists go
        to separate buffers (pf_*), so the layer's own lists are untouched."""
        c = self.cfg
        if not hasattr(self, "pf_miss_count"):
            bh, k = self.sel_blocks.shape[:2], c.k_blocks
            self.pf_sel_slot = torch.empty(*bh, k, dtype=torch.int32, device=self.sel_blocks.device)
            self.pf_sel_hit = torch.empty(*bh, k, dtype=torch.uint8, device=self.sel_blocks.device)
            self.pf_miss_block = torch.empty_like(self.pf_sel_slot)
            self.pf_miss_slot = torch.empty_like(self.pf_sel_slot)
            self.pf_miss_count = torch.empty(*bh, dtype=torch.int32, device=self.sel_blocks.device)
        B.sparse_kv_cache_update(self.shape, c.k_blocks, c.capacity, hint.sel_blocks, hint.sel_count,
                                 self.slot_block, self.slot_stamp, self.clock, self.pf_sel_slot, self.pf_sel_hit,
                                 self.pf_miss_block, self.pf_miss_slot, self.pf_miss_count, src_k, src_v, src_kind,
                                 self.pool_k, self.pool_v, stream)

    def append(self, new_k, new_v, seq_lens, keys, values, meta=None, stream=None):
        """Append one token per sequence (seq_lens grows on the device); the
        pool copies of resident blocks stay current."""
        c = self.cfg
        with_pool = self.pool_k is not None
        B.sparse_kv_append(self.shape, new_k, new_v, seq_lens, keys, values, meta,
                           self.slot_block if with_pool else None, c.capacity if with_pool else 0, self.pool_k,
                           self.pool_v, stream)

    def attention(self, q, seq_lens, src_k=None, src_v=None, src_kind=B.SKV_SRC_DEVICE, stream=None):
        """With src_k/src_v the misses are fetched here (fetch on attend)."""
        c = self.cfg
        B.sparse_decode_attention(self.shape, q, self.pool_k, self.pool_v, c.capacity, self.sel_blocks, self.sel_slot,
                                  self.sel_hit, self.sel_count, seq_lens, c.k_blocks, c.softmax_scale, self.splits,
                                  src_k, src_v, src_kind, self.out, self.lse, self.workspace, stream)


    def select_attend(self, q, seq_lens, src_k, src_v, src_kind=B.SKV_SRC_DEVICE, stream=None):
        """Top-k, working-set update and attention (fetching misses) in one call."""
        c = self.cfg
        B.sparse_kv_select_attend(self.shape, self.scores, seq_lens, c.k_blocks, c.sink, c.recent, c.capacity,
                                  self.sel_blocks, self.sel_count, self.slot_block, self.slot_stamp, self.clock,
                                  self.sel_slot, self.sel_hit, self.miss_block, self.miss_slot, self.miss_count, q,
                                  self.pool_k, self.pool_v, src_k, src_v, src_kind, c.softmax_scale,
                                  self.fused_splits, self.out, self.lse, self.workspace, stream)


class _Lists:
    """One set of per-step lists: the selection and the working-set plan."""

    def __init__(self, buf: LayerBuffers, own: bool):
        names = ("sel_blocks", "sel_count", "sel_slot", "sel_hit", "miss_block", "miss_slot", "miss_count")
        for n in names:
            t = getattr(buf, n)
            setattr(self, n, t if own else torch.empty_like(t))


class Lag1Pipeline:
    """Lag-1 decode of one layer: attention at step t runs over the selection
    made at step t-1 (the first step over its own) on the current stream,
    while step t's score and selection (top-k + working-set update in one
    launch) run on a side stream.
    The retrieval for the next step thus overlaps the attention, which uses
    the KV readied at the step before ("KV Cache 塞不进 HBM 了", §2.1 and the
    §3 loop).

    The working set needs capacity >= 2k and LRU eviction: the update of step
    t then never evicts a block of S_{t-1}, which attention at step t may be
    reading or filling (the victims are the least recently used blocks
    outside S_t; S_{t-1}'s blocks carry the newest stamps, and at most
    |S_t - S_{t-1}| + |S_{t-1}| <= 2k slots are needed).  The update only
    builds lists; attention fetches the misses of the selection it attends
    over from the source (fetch on attend).  Two list sets alternate between
    steps.  Results of a step are complete on the current stream after
    :meth:`join`.
    """

    def __init__(self, buf: LayerBuffers, side_stream=None):
        c = buf.cfg
        if c.capacity < 2 * c.k_blocks:
            raise ValueError(f"lag-1 needs capacity >= 2*k_blocks ({c.capacity} < {2 * c.k_blocks})")
        self.buf = buf
        self.side = side_stream if side_stream is not None else torch.cuda.Stream()
        self.lists = [_Lists(buf, True), _Lists(buf, False)]
        self.t = 0
        self._upd_prev = None

    def reset(self):
        self.buf.reset()
        self.rewind()

    def rewind(self):
        """Restart the schedule at step 0 without touching device state
        (e.g. before capturing the same steps into a graph)."""
        self.t = 0
        self._upd_prev = None

    def attended(self) -> _Lists:
        """The list set the last step's attention used."""
        return self.lists[max(self.t - 2, 0) % 2]

    def step(self, q, score_q, keys_or_meta, seq_lens, src_k, src_v, src_kind=B.SKV_SRC_DEVICE, miss_count=None):
        """Enqueue step t.  ``miss_count`` (optional [B, Hkv] int32) receives
        this step's update's miss counts instead of the list set's own."""
        buf, c = self.buf, self.buf.cfg
        main, side = torch.cuda.current_stream(), self.side
        cur = self.lists[self.t % 2]
        # the side stream sees the caller's inputs and the previous step's
        # attention (which read the list set written below)
        side.wait_stream(main)
        if not torch.cuda.is_current_stream_capturing():
            for t in (score_q, keys_or_meta, seq_lens, miss_count):
                if isinstance(t, torch.Tensor):
                    t.record_stream(side)  # the allocator must not reuse them while the side stream reads
        with torch.cuda.stream(side):
            B.sparse_kv_score(buf.shape, c.mode, score_q, c.n_queries, keys_or_meta, seq_lens, c.softmax_scale,
                              buf.scores, side)
            B.sparse_kv_select(buf.shape, buf.scores, seq_lens, c.k_blocks, c.sink, c.recent, c.capacity,
                               cur.sel_blocks, cur.sel_count, buf.slot_block, buf.slot_stamp, buf.clock, cur.sel_slot,
                               cur.sel_hit, cur.miss_block, cur.miss_slot,
                               cur.miss_count if miss_count is None else miss_count, None, None, src_kind,
                               buf.pool_k, buf.pool_v, buf.topk_workspace, side)
        upd = torch.cuda.Event()
        upd.record(side)
        use = self.lists[(self.t - 1) % 2] if self.t > 0 else cur
        if self.t == 0:
            main.wait_event(upd)
        elif self._upd_prev is not None:  # None: already ordered by join()
            main.wait_event(self._upd_prev)
        B.sparse_decode_attention(buf.shape, q, buf.pool_k, buf.pool_v, c.capacity, use.sel_blocks, use.sel_slot,
                                  use.sel_hit, use.sel_count, seq_lens, c.k_blocks, c.softmax_scale, buf.splits,
                                  src_k, src_v, src_kind, buf.out, buf.lse, buf.workspace, main)
        self._upd_prev = upd
        self.t += 1

    def join(self):
        """Make the current stream wait for the side stream's work (call it
        before reading a step's lists, and before a graph capture ends)."""
        torch.cuda.current_stream().wait_stream(self.side)
        self._upd_prev = None


def decode_step(buf: LayerBuffers, q, score_q, keys_or_meta, seq_lens, src_k, src_v, src_kind=B.SKV_SRC_DEVICE,
                stream=None, fetch_on_attend=True, fused=False, select=False):
    """Enqueue one full step: score, top-k, cache update, attention.

    The misses are copied into the pool either by the attention kernel while
    it reads them (fetch_on_attend, the default: one read and one write per
    missed block) or by the cache update's own copy pass.  fused=True runs
    stages 2-4 as the single select-attend call, select=True stages 2-3 as
    one launch (same results either way).
    """
    buf.score(score_q, keys_or_meta, seq_lens, stream)
    if fused:
        buf.select_attend(q, seq_lens, src_k, src_v, src_kind, stream)
        return
    if select:
        if fetch_on_attend:
            buf.select(seq_lens, None, None, src_kind, stream)
            buf.attention(q, seq_lens, src_k, src_v, src_kind, stream)
        else:
            buf.select(seq_lens, src_k, src_v, src_kind, stream)
            buf.attention(q, seq_lens, stream=stream)
        return
    buf.topk(seq_lens, stream)
    if fetch_on_attend:
        buf.cache_update(None, None, src_kind, stream)
        buf.attention(q, seq_lens, src_k, src_v, src_kind, stream)
    else:
        buf.cache_update(src_k, src_v, src_kind, stream)
        buf.attention(q, seq_lens, stream=stream)


def layer_sweep(bufs, q, seq_lens, srcs, src_kind=B.SKV_SRC_DEVICE, prefetch=False, side_stream=None, events=None):
    """Enqueue one decode step over consecutive layers whose selections are
    already in ``bufs[l].sel_blocks`` / ``sel_count`` (a selector outside
    the library picked them).  Per layer: working-set update with the miss
    fetch from ``srcs[l] = (src_k, src_v)``, then attention over the pool.

    prefetch=True adds the cross-layer prefetch: once layer l's own fetch is
    done, layer l+1's working set is updated with layer l's selection on
    ``side_stream`` (fetching layer l+1's bytes of those blocks) while layer
    l attends; layer l+1's own update waits for it and then finds the shared
    blocks resident.  ``events``, if a list, receives per layer a dict of
    (start, end) timing events: "update" (the layer's own update, current
    stream) and, with prefetch, "prefetch" (the next layer's, side stream).
    """
    main = torch.cuda.current_stream()
    if prefetch and side_stream is None:
        raise ValueError("prefetch needs a side stream")
    timed = events is not None

    def ev():
        return torch.cuda.Event(enable_timing=timed)

    pf_done = [None] * len(bufs)
    for l, buf in enumerate(bufs):
        if pf_done[l] is not None:
            main.wait_event(pf_done[l])
        rec = {"update": (ev(), ev())}
        rec["update"][0].record(main)
        buf.cache_update(*srcs[l], src_kind)
        rec["update"][1].record(main)
        if prefetch and l + 1 < len(bufs):
            side_stream.wait_event(rec["update"][1])
            rec["prefetch"] = (ev(), ev())
            rec["prefetch"][0].record(side_stream)
            with torch.cuda.stream(side_stream):
                bufs[l + 1].prefetch(buf, *srcs[l + 1], src_kind, side_stream)
            rec["prefetch"][1].record(side_stream)
            pf_done[l + 1] = rec["prefetch"][1]
        buf.attention(q[l] if isinstance(q, (list, tuple)) else q, seq_lens)
        if timed:
            events.append(rec)
    if prefetch:
        main.wait_stream(side_stream)
