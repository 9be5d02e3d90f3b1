/*
 * sparse_kv.h — C ABI of the sparse KV-cache decode step on MI355X (gfx950).
 *
 * One decode step for one attention layer is four calls, in this order, on
 * one stream:
 *
 *   sparse_kv_score          score every cached 16-token block of every
 *                            (sequence, kv-head) row against the current
 *                            query or the lookahead draft queries
 *   sparse_kv_topk           pick each row's blocks under the KV budget
 *   sparse_kv_cache_update   diff the pick against the row's resident
 *                            working set, detect hits, replace LRU slots,
 *                            list the misses and fetch them into the pool
 *   sparse_decode_attention  GQA decode attention over only the picked
 *                            blocks, split-K with an online-softmax merge
 *
 * Combined forms with the same results: sparse_kv_select (top-k + update in
 * one launch) and sparse_kv_select_attend (top-k + update + attention).
 * Around the step: sparse_kv_cache_update_importance (eviction by this
 * step's scores instead of LRU), sparse_kv_append (decode-time growth),
 * sparse_kv_quest_meta (the Quest boxes), sparse_kv_host_alloc / _free (a
 * host-memory source) and the split / workspace size helpers.
 *
 * The method (pages cited by title and section):
 *  - each head reads only its top-K past positions under a per-head,
 *    per-step KV budget ("KV Cache 塞不进 HBM 了", §1 and §3 steps 1-2);
 *  - within a GQA group the heads' scores are merged by element-wise max
 *    and the group picks one set (same page, §3 step 3);
 *  - block importance may come from lookahead draft queries (OasisKV
 *    summary, method, key module 2);
 *  - only selected - resident moves (same overview page, §2.1; OasisKV
 *    summary, key module 3);
 *  - a fixed-size working set per row is kept LRU with hit detection,
 *    replacement and fetch in one pass with no host synchronisation, and
 *    the full KV may sit in host memory (HiSparse promo, insights 1-2);
 *  - attention over the kept KV is exact (OasisKV summary, key module 1;
 *    HiSparse promo, insight 1).
 *
 * Conventions shared by every call:
 *  - Ownership: the caller allocates every buffer; the library allocates
 *    nothing, keeps no state between calls and never synchronises the host.
 *    All cache state (slot table, stamps, clock, pool) lives in caller
 *    buffers, so layers and snapshots are independent.
 *  - Pointers are device pointers (HBM) unless a parameter says otherwise;
 *    every array is dense row-major.  `stream` is a hipStream_t (NULL = the
 *    default stream); every call only enqueues work on it, so a whole step
 *    can be captured into a HIP graph.
 *  - Notation: B batch, Hq query heads, Hkv kv heads (Hq % Hkv == 0,
 *    G = Hq / Hkv, query head h belongs to kv head h / G), D head_dim,
 *    T = max_ctx tokens allocated per row, block = 16 tokens,
 *    NB = T / 16 blocks per row, row = (b, j) with j the kv head, P = B*Hkv.
 *  - Element type: shape->dtype applies to q, K, V, the Quest metadata and
 *    the pool.  bf16 is passed as raw 16-bit storage.  Scores, outputs and
 *    workspace are float32.
 *  - Errors: each call validates its arguments on the host and returns a
 *    status before launching anything.  A launch failure returns
 *    SKV_ERR_HIP.  Faults inside kernels surface at the caller's next
 *    synchronisation.  No call throws.
 *  - Calls are thread-safe: they touch no global state (except
 *    sparse_kv_select_attend_noalloc, see there).
 */
#ifndef SPARSE_KV_H
#define SPARSE_KV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum skv_status {
    SKV_OK = 0,
    SKV_ERR_NULL = 1,        /* a required pointer is NULL */
    SKV_ERR_SHAPE = 2,       /* sizes inconsistent or outside the supported range */
    SKV_ERR_DTYPE = 3,       /* dtype not supported */
    SKV_ERR_CAPACITY = 4,    /* capacity < k_blocks, or forced blocks exceed k_blocks */
    SKV_ERR_WORKSPACE = 5,   /* workspace missing or smaller than required */
    SKV_ERR_UNSUPPORTED = 6, /* a valid request this library does not implement */
    SKV_ERR_HIP = 7,         /* the HIP runtime reported an error at launch */
    SKV_ERR_SCRATCH = 8      /* sparse_kv_select_attend_noalloc: the call needs more
                                than SKV_NOALLOC_SCRATCH_BYTES of scratch */
} skv_status;

/* Size of the static device scratch of sparse_kv_select_attend_noalloc. */
#define SKV_NOALLOC_SCRATCH_BYTES (8u << 20)

typedef enum skv_dtype { SKV_F32 = 0, SKV_BF16 = 1 } skv_dtype;

typedef enum skv_score_mode {
    SKV_SCORE_BLOCKMAX = 0, /* exact: max over the block's tokens of q.k */
    SKV_SCORE_QUEST = 1     /* bound from per-block element-wise key min/max */
} skv_score_mode;

typedef enum skv_src_kind {
    SKV_SRC_DEVICE = 0,     /* the full K/V source is in HBM */
    SKV_SRC_HOST_MAPPED = 1 /* the source is pinned host memory mapped into the
                               device address space (sparse_kv_host_alloc);
                               misses are read over PCIe by the kernel itself */
} skv_src_kind;

typedef struct skv_shape {
    int32_t batch;      /* B >= 1 */
    int32_t n_q_heads;  /* Hq >= 1 */
    int32_t n_kv_heads; /* Hkv >= 1, Hq % Hkv == 0 */
    int32_t head_dim;   /* D: 64 or 128 */
    int32_t block_size; /* tokens per block: must be 16 */
    int32_t max_ctx;    /* T: tokens allocated per row, a multiple of 16, >= 16 */
    int32_t dtype;      /* skv_dtype */
} skv_shape;

/*
 * Stage 1: block scores.
 *
 * SKV_SCORE_BLOCKMAX:
 *   scores[b,j,n] = scale * max over r < n_queries, over the G heads h of
 *   group j and over the valid tokens t of block n (16n <= t < seq_lens[b])
 *   of <q[b,r,h,:], keys[b,j,t,:]>.
 *   The group max is the element-wise max within a GQA group ("KV Cache 塞不进
 *   HBM 了" §3 step 3); with n_queries > 1 the queries are lookahead drafts
 *   and the block importance is their max (OasisKV summary, key module 2).
 * SKV_SCORE_QUEST:
 *   scores[b,j,n] = scale * max over r, h of
 *                   sum_d max(q_d * meta[b,j,n,0,d], q_d * meta[b,j,n,1,d])
 *   an upper bound of every q.k in the block from its element-wise key box
 *   (Quest, named among query-driven selectors in "KV Cache Sparsity
 *   稀疏化方法", second truth); meta comes from sparse_kv_quest_meta.
 * Blocks with no valid token get -inf.
 *
 * q             [B, n_queries, Hq, D]            dtype
 * keys_or_meta  BLOCKMAX: keys [B, Hkv, T, D]    dtype
 *               QUEST:    meta [B, Hkv, NB, 2, D] dtype
 * seq_lens      [B] int32, each in [0, T]
 * scores        [B, Hkv, NB] float32 (output)
 * n_queries     1..4 (the G * n_queries query rows per kv head must be <= 32)
 */
skv_status sparse_kv_score(const skv_shape *shape, int32_t mode, const void *q, int32_t n_queries,
                           const void *keys_or_meta, const int32_t *seq_lens, float scale,
                           float *scores, void *stream);

/*
 * Stage 2: per-row top-k under the budget.
 *
 * Each row keeps at most k_blocks blocks (the budget is a per-head,
 * per-step cap: "KV Cache 塞不进 HBM 了" §3 step 2).  The blocks covering
 * tokens [0, sink_tokens) and the last recent_tokens valid tokens are
 * always kept and count inside the budget (sink + recent + top-scored, same
 * page §2.3); the rest go to the best remaining valid blocks in the order
 * (score descending, block id ascending).  A row with at most k_blocks
 * valid blocks keeps all of them.
 *
 * scores      [B, Hkv, NB] float32
 * seq_lens    [B] int32
 * sel_blocks  [B, Hkv, k_blocks] int32 (output): ascending block ids,
 *             padded with -1 after sel_count entries
 * sel_count   [B, Hkv] int32 (output)
 * workspace   >= sparse_kv_topk_workspace_bytes(shape, k_blocks) bytes of
 *             device memory, 256-byte aligned; may be NULL when that size is
 *             0 (NB <= 16384).  Rows over 16384 blocks are selected by many
 *             workgroups per row in two launches: the first keeps each
 *             1024- (or 4096-) block chunk's best blocks there, the second
 *             picks the row's selection from them.  Nothing in it needs
 *             clearing; calls that share a workspace must not overlap in
 *             time (enqueue them on one stream).
 * Limits: 1 <= k_blocks <= min(NB, 1024); NB <= 65536;
 *         ceil(sink/16) + ceil(recent/16) + 1 <= k_blocks when either is > 0.
 */
skv_status sparse_kv_topk(const skv_shape *shape, const float *scores, const int32_t *seq_lens,
                          int32_t k_blocks, int32_t sink_tokens, int32_t recent_tokens,
                          int32_t *sel_blocks, int32_t *sel_count, void *workspace, size_t workspace_bytes,
                          void *stream);

/*
 * Stage 3: delta / working-set manager and miss fetch.
 *
 * Each row owns `capacity` slots.  With R the row's resident blocks and S
 * its selection (ascending, sel_count entries):
 *   hits   = S and R: keep their slot;
 *   misses = S - R in ascending block order (only the delta moves:
 *            "KV Cache 塞不进 HBM 了" §2.1 / §3 step 1, OasisKV summary key
 *            module 3);
 *   victims: empty slots in ascending slot order, then occupied slots whose
 *            block is not in S, least recently used first, ordered by
 *            (stamp, block id); miss i takes victim i;
 *   the row's clock is advanced by one with a device atomic and every slot
 *   of S gets the new value as its stamp (LRU updated in-kernel, no host
 *   synchronisation: HiSparse promo, insight 2).
 * Touching the blocks of a step in ascending id order makes this exactly a
 * linked-list LRU.  Evicted slots are overwritten in place.
 *
 * In/out state: slot_block [B,Hkv,capacity] int32 (-1 = empty),
 *               slot_stamp [B,Hkv,capacity] uint32, clock [B,Hkv] uint32.
 *               Initialise slot_block to -1 and clock to 0 once.
 * Outputs:      sel_slot  [B,Hkv,k_blocks] int32 (slot of S[i]; -1 pad)
 *               sel_hit   [B,Hkv,k_blocks] uint8 (1 = was resident; 0 pad)
 *               miss_block, miss_slot [B,Hkv,k_blocks] int32 (-1 pad)
 *               miss_count [B,Hkv] int32
 * Fetch:        when src_k/src_v are non-NULL, K and V rows
 *               [16*blk, 16*blk+16) of each miss are copied from
 *               src [B,Hkv,T,D] into pool [B,Hkv,capacity,16,D].  With
 *               src_kind SKV_SRC_HOST_MAPPED, src is the device pointer of
 *               mapped pinned host memory and the copy crosses PCIe.  NULL
 *               sources build the lists only (the "no-IO" control).
 * Bad input seen on the device (a selection not strictly ascending, an id
 * outside [0, NB), a count outside [0, k_blocks], or a corrupt slot table:
 * an id outside [-1, NB), or one block held by two slots, selected or not --
 * the table maps each resident block to one slot, a block table as in
 * KV-Cache 压缩技术的工程原理 §5.2) refuses the row: its slot table, stamps,
 * clock and pool stay untouched, miss_count = -1, and its lists are padded
 * (sel_slot -1, sel_hit 0, miss_block / miss_slot -1), so an attention call
 * over them reads nothing for that row.
 * Cross-layer prefetch (HiSparse promo, insight 3: picks overlap between
 * layers, so the previous layer's picks are fetched for the next layer
 * before its own are known): call this for layer l+1's state and source with
 * layer l's sel_blocks / sel_count, on a second stream while layer l
 * attends, with separate list outputs.  It is an ordinary update (clock tick
 * and stamps included); layer l+1's own update then finds the shared blocks
 * resident.  The two calls on one layer's state must not overlap in time.
 * Limits: 1 <= k_blocks <= capacity <= 1024; NB <= 2^21 (else
 * SKV_ERR_UNSUPPORTED).
 */
skv_status sparse_kv_cache_update(const skv_shape *shape, int32_t k_blocks, int32_t capacity,
                                  const int32_t *sel_blocks, const int32_t *sel_count,
                                  int32_t *slot_block, uint32_t *slot_stamp, uint32_t *clock,
                                  int32_t *sel_slot, uint8_t *sel_hit, int32_t *miss_block,
                                  int32_t *miss_slot, int32_t *miss_count, const void *src_k,
                                  const void *src_v, int32_t src_kind, void *pool_k, void *pool_v,
                                  void *stream);

/*
 * Stages 2 and 3 in one launch: sparse_kv_topk followed by
 * sparse_kv_cache_update (LRU), with the selection kept on chip between the
 * two and the plan committed by the same workgroup.  Same arguments, same
 * outputs and the same results bit for bit as the two calls in that order
 * (the selection goes to sel_blocks / sel_count as well); with src_k/src_v
 * the misses are gathered into the pool afterwards, else only the lists are
 * built (as sparse_kv_cache_update with NULL sources).  For pipelines that
 * attend separately, e.g. one step behind ("KV Cache 塞不进 HBM 了" §2.1:
 * the next step's retrieval runs while the forward uses the KV already
 * resident).  The workspace is sparse_kv_topk's (rows over 16384 blocks
 * run that call's first launch, then one launch that selects and updates).
 * Limits: those of the two calls.
 */
skv_status sparse_kv_select(const skv_shape *shape, const float *scores, const int32_t *seq_lens,
                            int32_t k_blocks, int32_t sink_tokens, int32_t recent_tokens, int32_t capacity,
                            int32_t *sel_blocks, int32_t *sel_count, int32_t *slot_block, uint32_t *slot_stamp,
                            uint32_t *clock, int32_t *sel_slot, uint8_t *sel_hit, int32_t *miss_block,
                            int32_t *miss_slot, int32_t *miss_count, const void *src_k, const void *src_v,
                            int32_t src_kind, void *pool_k, void *pool_v, void *workspace, size_t workspace_bytes,
                            void *stream);

/*
 * Stage 3 with importance-capped eviction instead of LRU (OasisKV summary,
 * key module 3: only the delta moves, and when the capped cache has no room
 * the least important blocks are evicted).  Everything as in
 * sparse_kv_cache_update except the order of the victims after the empty
 * slots: occupied slots whose block is not in S, least important first,
 * ordered by (scores[b,j,block], block id), where scores [B,Hkv,NB] float32
 * are this step's block scores (from sparse_kv_score; not modified).  Stamps
 * and the clock are still advanced, so a row may switch policies between
 * steps.  scores == NULL returns SKV_ERR_NULL.
 */
skv_status sparse_kv_cache_update_importance(const skv_shape *shape, int32_t k_blocks, int32_t capacity,
                                             const int32_t *sel_blocks, const int32_t *sel_count,
                                             const float *scores, int32_t *slot_block, uint32_t *slot_stamp,
                                             uint32_t *clock, int32_t *sel_slot, uint8_t *sel_hit,
                                             int32_t *miss_block, int32_t *miss_slot, int32_t *miss_count,
                                             const void *src_k, const void *src_v, int32_t src_kind, void *pool_k,
                                             void *pool_v, void *stream);

/*
 * Decode-time append (the method's gains come where the KV grows during
 * decoding: "KV Cache 塞不进 HBM 了", intro and §1).  For every sequence b
 * with 0 <= seq_lens[b] < T, the new rows new_k[b,j,:], new_v[b,j,:] of each
 * kv head j are stored at token seq_lens[b] of keys/values [B,Hkv,T,D], and
 * seq_lens[b] grows by one (device-side; a full sequence is left as it is).
 *   meta (nullable) [B,Hkv,NB,2,D]: the Quest box of the token's block is
 *     kept exact: a token that opens a block sets min = max = its row, else
 *     min/max take the element-wise minimum/maximum with it (the result
 *     equals sparse_kv_quest_meta over the grown cache);
 *   slot_block (nullable) [B,Hkv,capacity]: if the token's block is resident
 *     in a slot, the rows are also stored in pool_k/pool_v [B,Hkv,capacity,
 *     16,D], so every resident slot keeps its block's bytes.
 * new_k, new_v [B,Hkv,D] in shape->dtype.  Call it between steps on the
 * step's stream; every later call sees the grown length.
 */
skv_status sparse_kv_append(const skv_shape *shape, const void *new_k, const void *new_v, int32_t *seq_lens,
                            void *keys, void *values, void *meta, const int32_t *slot_block, int32_t capacity,
                            void *pool_k, void *pool_v, void *stream);

/*
 * Stage 4: GQA decode attention over the selected blocks.
 *
 * For query head h (kv head j = h / G) and the valid tokens t of the
 * selected blocks (read from the pool through sel_slot):
 *   out[b,h,:] = sum_t softmax_t(scale * <q[b,h], k_t>) v_t
 *   lse[b,h]   = log sum_t exp(scale * <q[b,h], k_t>)
 * Exact attention over the kept KV (OasisKV summary, key module 1).  Each
 * row's selection is cut into num_splits contiguous parts, each part is
 * reduced by one workgroup to (max, sum, unnormalised output) and the parts
 * are merged with the usual log-sum-exp rescaling.  A row with no valid
 * token gives out = 0 and lse = -inf.
 *
 * Fetch on attend: when src_k/src_v are given (device or host-mapped, as
 * in sparse_kv_cache_update), every selected block with sel_hit == 0 is
 * read from the source by its block id instead of from the pool, and is
 * also written into its pool slot.  Use it with a list-only cache update
 * (NULL sources there) to move each miss once; with NULL sources here the
 * pool must already hold every selected block.
 *
 * q           [B, Hq, D] dtype
 * pool_k/v    [B, Hkv, capacity, 16, D] dtype (written only for fetched misses)
 * sel_blocks, sel_slot [B, Hkv, k_blocks] int32; sel_hit [B, Hkv, k_blocks]
 *             uint8 (only read with sources, may be NULL otherwise);
 *             sel_count [B, Hkv] int32; seq_lens [B] int32
 * out         [B, Hq, D] float32; lse [B, Hq] float32 or NULL
 * num_splits  0 = choose (sparse_decode_attention_splits), else
 *             1..min(k_blocks, 128)
 * workspace   >= sparse_decode_attention_workspace_bytes(shape, k_blocks,
 *             num_splits) bytes of device memory, 256-byte aligned (the
 *             per-split partials); calls that share a workspace must not
 *             overlap in time (enqueue them on one stream).
 * Entries with a slot outside [0, capacity) or a negative block are skipped.
 */
skv_status sparse_decode_attention(const skv_shape *shape, const void *q, void *pool_k, void *pool_v,
                                   int32_t capacity, const int32_t *sel_blocks, const int32_t *sel_slot,
                                   const uint8_t *sel_hit, const int32_t *sel_count, const int32_t *seq_lens,
                                   int32_t k_blocks, float scale, int32_t num_splits, const void *src_k,
                                   const void *src_v, int32_t src_kind, float *out, float *lse, void *workspace,
                                   size_t workspace_bytes, void *stream);

/*
 * Stages 2-4 in one call: sparse_kv_topk, then sparse_kv_cache_update with
 * NULL sources (lists only), then sparse_decode_attention with the given
 * sources (fetch on attend) -- the same results bit for bit, with every
 * argument as in those calls (the workspace is sized by
 * sparse_decode_attention_workspace_bytes).  Each workgroup of a row
 * recomputes the row's top-k and working-set plan in on-chip memory before
 * attending its share, so the three stages cost one pass over the scores
 * and slot table instead of three launches with global round trips in
 * between; the plan is committed to the slot table, stamps and clock at the
 * end of the call.  A row refused as in sparse_kv_cache_update (a corrupt
 * slot table) gets miss_count = -1, padded lists, an untouched table,
 * out = 0 and lse = -inf.
 * num_splits = 0 resolves to sparse_kv_select_attend_splits (fewer, larger
 * parts than the attention call's default: the fused call prefers one
 * resident workgroup per CU); results equal the separate calls' bit for bit
 * when both use the same num_splits.  The workspace must hold
 * sparse_decode_attention_workspace_bytes(shape, k_blocks, splits) bytes for
 * the resolved split count (the partials) plus, when NB > 16384,
 * sparse_kv_topk_workspace_bytes(shape, k_blocks) (the top-k's chunk
 * candidates, placed right after the partials: such rows first run
 * sparse_kv_topk's chunk launch, then every workgroup of a row selects from
 * the candidates); sparse_kv_workspace_bytes covers both.
 * Limits: those of the three calls.
 */
skv_status sparse_kv_select_attend(const skv_shape *shape, const float *scores, const int32_t *seq_lens,
                                   int32_t k_blocks, int32_t sink_tokens, int32_t recent_tokens, int32_t capacity,
                                   int32_t *sel_blocks, int32_t *sel_count, int32_t *slot_block,
                                   uint32_t *slot_stamp, uint32_t *clock, int32_t *sel_slot, uint8_t *sel_hit,
                                   int32_t *miss_block, int32_t *miss_slot, int32_t *miss_count, const void *q,
                                   void *pool_k, void *pool_v, const void *src_k, const void *src_v,
                                   int32_t src_kind, float scale, int32_t num_splits, float *out, float *lse,
                                   void *workspace, size_t workspace_bytes, void *stream);

/*
 * sparse_kv_select_attend without a workspace argument and without any
 * allocation, for callers that cannot allocate device memory: code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc.
 * Same arguments (minus workspace / workspace_bytes), same kernels and the
 * same results bit for bit as sparse_kv_select_attend with the same
 * num_splits.  The per-split partials (and, past 16384 blocks, the top-k's
 * chunk candidates) go to a static device array of
 * SKV_NOALLOC_SCRATCH_BYTES (8 MiB) that each GPU the library runs on holds
 * until the process ends; its address is looked up once per device on the
 * first call with that device current.  A call that needs more (the
 * workspace size sparse_kv_select_attend would need) returns
 * SKV_ERR_SCRATCH before launching anything.  Nothing in the scratch needs
 * clearing (every workgroup writes its whole partial before the merge reads
 * it, every chunk its candidates before they are read).  All calls on one GPU share that GPU's array: calls that overlap in
 * time on one GPU (other streams, other host threads) race; enqueue them on
 * one stream.
 */
skv_status sparse_kv_select_attend_noalloc(const skv_shape *shape, const float *scores, const int32_t *seq_lens,
                                           int32_t k_blocks, int32_t sink_tokens, int32_t recent_tokens,
                                           int32_t capacity, int32_t *sel_blocks, int32_t *sel_count,
                                           int32_t *slot_block, uint32_t *slot_stamp, uint32_t *clock,
                                           int32_t *sel_slot, uint8_t *sel_hit, int32_t *miss_block,
                                           int32_t *miss_slot, int32_t *miss_count, const void *q, void *pool_k,
                                           void *pool_v, const void *src_k, const void *src_v, int32_t src_kind,
                                           float scale, int32_t num_splits, float *out, float *lse, void *stream);

/* Number of splits num_splits = 0 resolves to (attention / fused call). */
int32_t sparse_decode_attention_splits(const skv_shape *shape, int32_t k_blocks);
int32_t sparse_kv_select_attend_splits(const skv_shape *shape, int32_t k_blocks);

/* Workspace bytes sparse_decode_attention needs (0 on invalid arguments). */
size_t sparse_decode_attention_workspace_bytes(const skv_shape *shape, int32_t k_blocks,
                                               int32_t num_splits);

/* Workspace bytes sparse_kv_topk and sparse_kv_select need: 0 when
 * NB <= 16384, else B*Hkv * chunks * k_blocks * 8 with chunks = ceil(NB /
 * 1024), or ceil(NB / 4096) when ceil(NB / 1024) * k_blocks > 16384
 * (0 on invalid arguments). */
size_t sparse_kv_topk_workspace_bytes(const skv_shape *shape, int32_t k_blocks);

/* One workspace size that serves every call of a step with these k_blocks
 * and num_splits (0 = each call's own default): the larger of the two
 * sizes above and the fused call's partials.  0 on invalid arguments. */
size_t sparse_kv_workspace_bytes(const skv_shape *shape, int32_t k_blocks, int32_t num_splits);

/*
 * Helper (failure detection, not part of the step): checks a working-set
 * state on the device and writes per row flags [B,Hkv] int32, the OR of
 *   1: a slot id outside [-1, NB),
 *   2: one block held by two slots (a block table maps each resident block
 *      to one slot: KV-Cache 压缩技术的工程原理 §5.2),
 *   4: an occupied slot whose stamp is ahead of the row's clock (every
 *      update stamps the slots it touches with the clock value it has just
 *      advanced to).
 * 0 means consistent.  Use it after restoring a snapshot or when a row came
 * back refused (miss_count = -1) to see what is wrong; the update calls
 * refuse rows with flags 1 or 2 on their own.  Reads the state only.
 * Limits: 1 <= capacity <= 1024.
 */
skv_status sparse_kv_check_state(const skv_shape *shape, int32_t capacity, const int32_t *slot_block,
                                 const uint32_t *slot_stamp, const uint32_t *clock, int32_t *flags, void *stream);

/*
 * Helper (prefill time, not part of the step): per-block element-wise key
 * minimum and maximum over the valid tokens, meta [B,Hkv,NB,2,D] in the key
 * dtype (min at [...,0,:], max at [...,1,:]); blocks past seq_lens get
 * zeros.  These are exact (min/max of stored values).
 */
skv_status sparse_kv_quest_meta(const skv_shape *shape, const void *keys, const int32_t *seq_lens,
                                void *meta, void *stream);

/*
 * Helper (measurement only, not part of the step): reads keys [B,Hkv,T,D]
 * once, whole, in the launch shape and 16-byte load form of the exact block
 * scan of sparse_kv_score, with no arithmetic beyond folding what it reads
 * into one word.  It writes sink[0] only when that word equals one fixed
 * value, which real data almost never produce (so the reads cannot be
 * dropped).  Its duration gives the HBM read rate the scan's access pattern
 * can reach: the measured anchor of the scan's roofline beside the
 * nameplate peak.  sink: one uint32 of device memory.
 */
skv_status sparse_kv_stream_read(const skv_shape *shape, const void *keys, uint32_t *sink, void *stream);

/*
 * Helper: pinned host memory mapped into the device address space, for a
 * host-resident K/V source.  *host_ptr is for the CPU, *device_ptr for the
 * kernels.  Free with sparse_kv_host_free(host_ptr).
 */
skv_status sparse_kv_host_alloc(size_t bytes, void **host_ptr, void **device_ptr);
skv_status sparse_kv_host_free(void *host_ptr);

/* Static English text for a status code. */
const char *sparse_kv_status_string(skv_status status);

#ifdef __cplusplus
}
#endif

#endif /* SPARSE_KV_H */
