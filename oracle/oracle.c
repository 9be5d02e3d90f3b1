/*
 * CPU oracle for the sparse KV-cache decode step.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the CPU
 * baseline leg of the benchmark load this library.  It shares no code with
 * the HIP path and never sees its outputs except as values to compare.
 *
 * Plain C99, fp64 arithmetic on the exact input values (fp32 inputs widen
 * exactly; bf16 inputs are widened from their 16 bits), scalar loops, no
 * blocking, no fast math.  OpenMP only runs independent rows in parallel.
 *
 * Conventions (all arrays row-major, caller-owned):
 *   dtype 0 = float32, 1 = bfloat16 given as uint16 bits, 2 = float64.
 *   q       [B, NQ, Hq, D]          scoring queries (NQ = 1, or the drafts)
 *   K, V    [B, Hkv, T_max, D]      full per-layer cache ("source")
 *   meta    [B, Hkv, NB_max, 2, D]  per-block element-wise key min / max
 *   scores  [B, Hkv, NB_max]        one per (row, block); -inf past the end
 *   sel     [B, Hkv, k_max]         selected block ids, ascending, -1 pad
 *   pool    [B, Hkv, C, block, D]   working-set slots
 * Query head h belongs to kv head j = h / G with G = Hq / Hkv (contiguous
 * groups, the usual GQA layout).
 *
 * Page citations below name each page by its title.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORC_OK 0
#define ORC_BAD 1

static double widen(const void *base, int dtype, size_t i)
{
    if (dtype == 0)
        return (double)((const float *)base)[i];
    if (dtype == 2)
        return ((const double *)base)[i];
    uint32_t bits = (uint32_t)((const uint16_t *)base)[i] << 16;
    float f;
    memcpy(&f, &bits, sizeof f);
    return (double)f;
}

static int nb_of(int len, int block) { return (len + block - 1) / block; }

/*
 * Exact block score.  For every (b, j, n):
 *   s = scale * max over scoring queries r, over the heads h of group j and
 *       over the valid tokens t of block n of  <q[b,r,h], k[b,j,t]>.
 * The max over heads of a GQA group follows "KV Cache 塞不进 HBM 了" §3 (step
 * 3: element-wise max of the group's scores, then top-k per group); the
 * block-granular importance from the draft tokens' attention follows the
 * OasisKV summary (method, key module 2); with one query it is the current
 * query's block importance.  Blocks with no valid token score -inf.
 */
int oracle_score_blockmax(int B, int NQ, int Hq, int Hkv, int D, int T_max, int block,
                          int dtype, const void *q, const void *k, const int32_t *seq_lens,
                          double scale, int nb_max, double *scores)
{
    if (B <= 0 || NQ <= 0 || Hq <= 0 || Hkv <= 0 || Hq % Hkv || D <= 0 || block <= 0)
        return ORC_BAD;
    const int G = Hq / Hkv;
#pragma omp parallel for collapse(2) schedule(dynamic)
    for (int b = 0; b < B; ++b)
        for (int j = 0; j < Hkv; ++j) {
            int len = seq_lens[b] < T_max ? seq_lens[b] : T_max;
            int nvalid = nb_of(len, block);
            double *qd = (double *)malloc(sizeof(double) * (size_t)NQ * G * D);
            for (int r = 0; r < NQ; ++r)
                for (int g = 0; g < G; ++g)
                    for (int d = 0; d < D; ++d)
                        qd[((size_t)r * G + g) * D + d] =
                            widen(q, dtype, (((size_t)b * NQ + r) * Hq + (size_t)j * G + g) * D + d);
            double *out = scores + ((size_t)b * Hkv + j) * nb_max;
            for (int n = 0; n < nb_max; ++n) {
                if (n >= nvalid) {
                    out[n] = -INFINITY;
                    continue;
                }
                int t0 = n * block, t1 = t0 + block < len ? t0 + block : len;
                double best = -INFINITY;
                for (int t = t0; t < t1; ++t) {
                    size_t kbase = (((size_t)b * Hkv + j) * T_max + t) * D;
                    for (int rg = 0; rg < NQ * G; ++rg) {
                        double dot = 0.0;
                        for (int d = 0; d < D; ++d)
                            dot += qd[(size_t)rg * D + d] * widen(k, dtype, kbase + d);
                        if (dot > best)
                            best = dot;
                    }
                }
                out[n] = scale * best;
            }
            free(qd);
        }
    return ORC_OK;
}

/*
 * Per-block element-wise minimum and maximum of the valid keys (the block
 * summary a Quest-style selector keeps; the pages name Quest among the
 * query-driven selectors: KV Cache Sparsity 稀疏化方法, second truth; HiSparse
 * promo, intro).  meta[b,j,n,0,:] = min, meta[b,j,n,1,:] = max.  Blocks past
 * the end get zeros.
 */
int oracle_quest_meta(int B, int Hkv, int D, int T_max, int block, int dtype, const void *k,
                      const int32_t *seq_lens, int nb_max, double *meta)
{
#pragma omp parallel for collapse(2)
    for (int b = 0; b < B; ++b)
        for (int j = 0; j < Hkv; ++j) {
            int len = seq_lens[b] < T_max ? seq_lens[b] : T_max;
            int nvalid = nb_of(len, block);
            for (int n = 0; n < nb_max; ++n) {
                double *mn = meta + ((((size_t)b * Hkv + j) * nb_max + n) * 2) * D;
                double *mx = mn + D;
                if (n >= nvalid) {
                    for (int d = 0; d < D; ++d)
                        mn[d] = mx[d] = 0.0;
                    continue;
                }
                int t0 = n * block, t1 = t0 + block < len ? t0 + block : len;
                for (int d = 0; d < D; ++d) {
                    double lo = INFINITY, hi = -INFINITY;
                    for (int t = t0; t < t1; ++t) {
                        double x = widen(k, dtype, (((size_t)b * Hkv + j) * T_max + t) * D + d);
                        if (x < lo)
                            lo = x;
                        if (x > hi)
                            hi = x;
                    }
                    mn[d] = lo;
                    mx[d] = hi;
                }
            }
        }
    return ORC_OK;
}

/*
 * Quest-style upper bound of the block's q.k:
 *   s = scale * max over r, h of  sum_d max(q_d * min_d, q_d * max_d)
 * Each term is the largest value q_d * k_d can take for any key inside the
 * block's box, so the sum bounds every key's dot product from above.
 * meta may be given in the keys' dtype or in float64 (min/max of stored
 * values are stored values, so either form is exact).
 */
int oracle_score_quest(int B, int NQ, int Hq, int Hkv, int D, int block, int dtype,
                       const void *q, const void *meta, int meta_dtype, const int32_t *seq_lens,
                       int T_max, double scale, int nb_max, double *scores)
{
    if (Hq % Hkv)
        return ORC_BAD;
    const int G = Hq / Hkv;
#pragma omp parallel for collapse(2) schedule(dynamic)
    for (int b = 0; b < B; ++b)
        for (int j = 0; j < Hkv; ++j) {
            int len = seq_lens[b] < T_max ? seq_lens[b] : T_max;
            int nvalid = nb_of(len, block);
            double *out = scores + ((size_t)b * Hkv + j) * nb_max;
            for (int n = 0; n < nb_max; ++n) {
                if (n >= nvalid) {
                    out[n] = -INFINITY;
                    continue;
                }
                size_t mbase = ((((size_t)b * Hkv + j) * nb_max + n) * 2) * D;
                double best = -INFINITY;
                for (int r = 0; r < NQ; ++r)
                    for (int g = 0; g < G; ++g) {
                        double bound = 0.0;
                        for (int d = 0; d < D; ++d) {
                            double qv = widen(q, dtype, (((size_t)b * NQ + r) * Hq + (size_t)j * G + g) * D + d);
                            double lo = qv * widen(meta, meta_dtype, mbase + d);
                            double hi = qv * widen(meta, meta_dtype, mbase + D + d);
                            bound += lo > hi ? lo : hi;
                        }
                        if (bound > best)
                            best = bound;
                    }
                out[n] = scale * best;
            }
        }
    return ORC_OK;
}

/* ------------------------------------------------------------------ top-k */
typedef struct {
    double s;
    int32_t id;
} scored_t;

/* score descending, then block id ascending: a strict total order */
static int by_score_desc_id_asc(const void *a, const void *b)
{
    const scored_t *x = (const scored_t *)a, *y = (const scored_t *)b;
    if (x->s > y->s)
        return -1;
    if (x->s < y->s)
        return 1;
    return (x->id > y->id) - (x->id < y->id);
}

static int by_int_asc(const void *a, const void *b)
{
    int32_t x = *(const int32_t *)a, y = *(const int32_t *)b;
    return (x > y) - (x < y);
}

/*
 * Per-row block selection under the KV budget.
 *
 * Each (sequence, kv-head) row keeps at most k_blocks blocks per step (the
 * budget is a per-head per-step cap: "KV Cache 塞不进 HBM 了" §3 step 2, and
 * the per-head top-k of §1 / §3 step 1).  Blocks covering the first
 * sink_tokens tokens and the last recent_tokens valid tokens are always kept
 * (sink + recent + top-scored tokens, as in SparseSpec-L, same page §2.3);
 * they count inside the budget.  The rest of the budget goes to the
 * best-scored remaining valid blocks in the order (score desc, id asc).  If
 * the row has no more valid blocks than the budget, all are selected.
 * Output is ascending by block id and padded with -1.
 */
int oracle_topk(int B, int Hkv, int nb_max, const double *scores, const int32_t *seq_lens,
                int T_max, int block, int k_blocks, int sink_tokens, int recent_tokens,
                int32_t *sel, int32_t *sel_count)
{
    int bad = 0;
#pragma omp parallel for collapse(2) reduction(| : bad)
    for (int b = 0; b < B; ++b)
        for (int j = 0; j < Hkv; ++j) {
            int len = seq_lens[b] < T_max ? seq_lens[b] : T_max;
            int nvalid = nb_of(len, block);
            if (nvalid > nb_max)
                nvalid = nb_max;
            const double *s = scores + ((size_t)b * Hkv + j) * nb_max;
            int32_t *out = sel + ((size_t)b * Hkv + j) * k_blocks;
            char *forced = (char *)calloc((size_t)nvalid + 1, 1);
            scored_t *cand = (scored_t *)malloc(sizeof(scored_t) * ((size_t)nvalid + 1));
            int nf = 0, nc = 0, n = 0;
            if (nvalid <= k_blocks) {
                for (int i = 0; i < nvalid; ++i)
                    out[n++] = i;
            } else {
                if (sink_tokens > 0) {
                    int last = nb_of(sink_tokens < len ? sink_tokens : len, block);
                    for (int i = 0; i < last; ++i)
                        forced[i] = 1;
                }
                if (recent_tokens > 0) {
                    int first_tok = len - recent_tokens > 0 ? len - recent_tokens : 0;
                    for (int i = first_tok / block; i < nvalid; ++i)
                        forced[i] = 1;
                }
                for (int i = 0; i < nvalid; ++i) {
                    if (forced[i])
                        out[nf++] = i;
                    else {
                        cand[nc].s = s[i];
                        cand[nc].id = i;
                        ++nc;
                    }
                }
                if (nf > k_blocks)
                    bad = 1;
                n = nf;
                int take = k_blocks - nf;
                if (take > nc)
                    take = nc;
                if (take > 0) {
                    qsort(cand, (size_t)nc, sizeof(scored_t), by_score_desc_id_asc);
                    for (int i = 0; i < take; ++i)
                        out[n++] = cand[i].id;
                }
                qsort(out, (size_t)n, sizeof(int32_t), by_int_asc);
            }
            for (int i = n; i < k_blocks; ++i)
                out[i] = -1;
            sel_count[(size_t)b * Hkv + j] = n;
            free(forced);
            free(cand);
        }
    return bad ? ORC_BAD : ORC_OK;
}

/* ------------------------------------------------------- working set (LRU) */
/*
 * A fixed-size working set of `cap` slots per row, managed least-recently
 * used (HiSparse promo, insight 1: a fixed GPU cache under LRU; insight 2:
 * hit detection + LRU replacement + fetch in one pass).  Only the delta
 * between the selection and what is resident moves ("KV Cache 塞不进 HBM 了"
 * §2.1 and §3 step 1: to_load = selected - resident; OasisKV summary, key
 * module 3).  Evicted slots are overwritten in place (soft marking; KV-Cache
 * 压缩技术的工程原理 §4.3); the slot table is a block table (same page §5.2).
 *
 * This form keeps an explicit doubly linked list of occupied slots per row,
 * least recent at the head.  One step with selection S (ascending):
 *   hits    = blocks of S already resident (keep their slot)
 *   misses  = blocks of S not resident, ascending
 *   victims = empty slots in ascending slot order, then occupied slots taken
 *             from the least-recent end, skipping slots that hold a block of S
 *   miss i goes to victim i; then every block of S is touched in ascending
 *   block order (moved or appended to the most-recent end).
 * An invalid row leaves its state untouched, reports miss_count = -1 and
 * gets padded lists (sel_slot -1, sel_hit 0, miss_block / miss_slot -1).  A
 * row is invalid when its selection is (count outside [0, min(k, cap)], not
 * strictly ascending, or an id outside [0, nb_limit)) or when its slot table
 * is: an id outside [-1, nb_limit), or one block held by two slots, selected
 * or not.  The slot table is a block table (KV-Cache 压缩技术的工程原理
 * §5.2): it maps each resident block to the one slot holding its bytes, so
 * a block that appears twice is a broken mapping whatever this step picks.
 *
 * oracle_lru_load starts the rows from a given table: slot_block as given,
 * and the occupied slots linked least recent first in the order of
 * (stamp, block id, slot) -- the stamp of a slot being the step at which it
 * was last touched, and blocks touched in one step counting in ascending id
 * order, as the step below touches them.
 */
typedef struct {
    int rows, cap;
    int32_t *slot_block, *prev, *next, *head, *tail;
} oracle_lru;

oracle_lru *oracle_lru_create(int rows, int cap)
{
    oracle_lru *h = (oracle_lru *)calloc(1, sizeof *h);
    h->rows = rows;
    h->cap = cap;
    size_t n = (size_t)rows * cap;
    h->slot_block = (int32_t *)malloc(n * sizeof(int32_t));
    h->prev = (int32_t *)malloc(n * sizeof(int32_t));
    h->next = (int32_t *)malloc(n * sizeof(int32_t));
    h->head = (int32_t *)malloc((size_t)rows * sizeof(int32_t));
    h->tail = (int32_t *)malloc((size_t)rows * sizeof(int32_t));
    for (size_t i = 0; i < n; ++i)
        h->slot_block[i] = h->prev[i] = h->next[i] = -1;
    for (int r = 0; r < rows; ++r)
        h->head[r] = h->tail[r] = -1;
    return h;
}

void oracle_lru_destroy(oracle_lru *h)
{
    if (!h)
        return;
    free(h->slot_block);
    free(h->prev);
    free(h->next);
    free(h->head);
    free(h->tail);
    free(h);
}

/* drop every resident block (slots become empty, order forgotten) */
void oracle_lru_flush(oracle_lru *h)
{
    size_t n = (size_t)h->rows * h->cap;
    for (size_t i = 0; i < n; ++i)
        h->slot_block[i] = h->prev[i] = h->next[i] = -1;
    for (int r = 0; r < h->rows; ++r)
        h->head[r] = h->tail[r] = -1;
}

void oracle_lru_get(const oracle_lru *h, int32_t *slot_block_out)
{
    memcpy(slot_block_out, h->slot_block, (size_t)h->rows * h->cap * sizeof(int32_t));
}

/* LRU order of occupied slots, least recent first, -1 padded: [rows, cap] */
void oracle_lru_order(const oracle_lru *h, int32_t *order_out)
{
    for (int r = 0; r < h->rows; ++r) {
        int32_t *o = order_out + (size_t)r * h->cap;
        int n = 0;
        for (int s = h->head[r]; s >= 0; s = h->next[(size_t)r * h->cap + s])
            o[n++] = s;
        for (; n < h->cap; ++n)
            o[n] = -1;
    }
}

static void unlink_slot(oracle_lru *h, int r, int s)
{
    int32_t *pv = h->prev + (size_t)r * h->cap, *nx = h->next + (size_t)r * h->cap;
    if (pv[s] >= 0)
        nx[pv[s]] = nx[s];
    else if (h->head[r] == s)
        h->head[r] = nx[s];
    if (nx[s] >= 0)
        pv[nx[s]] = pv[s];
    else if (h->tail[r] == s)
        h->tail[r] = pv[s];
    pv[s] = nx[s] = -1;
}

static void append_slot(oracle_lru *h, int r, int s)
{
    int32_t *pv = h->prev + (size_t)r * h->cap, *nx = h->next + (size_t)r * h->cap;
    pv[s] = h->tail[r];
    nx[s] = -1;
    if (h->tail[r] >= 0)
        nx[h->tail[r]] = s;
    else
        h->head[r] = s;
    h->tail[r] = s;
}

static int in_sorted(const int32_t *S, int n, int32_t x)
{
    int lo = 0, hi = n - 1;
    while (lo <= hi) {
        int mid = (lo + hi) / 2;
        if (S[mid] == x)
            return 1;
        if (S[mid] < x)
            lo = mid + 1;
        else
            hi = mid - 1;
    }
    return 0;
}

/* 1 if the row's selection S[0, n) and slot table sb[0, C) are valid input
 * for a working-set step (see the rules above), else 0. */
static int row_input_ok(const int32_t *S, int n, int k_max, int nb_limit, const int32_t *sb, int C)
{
    if (n < 0 || n > k_max || n > C)
        return 0;
    for (int i = 0; i < n; ++i)
        if (S[i] < 0 || S[i] >= nb_limit || (i > 0 && S[i] <= S[i - 1]))
            return 0;
    for (int s = 0; s < C; ++s) {
        if (sb[s] < -1 || sb[s] >= nb_limit)
            return 0;
        for (int t = 0; t < s; ++t)
            if (sb[s] >= 0 && sb[t] == sb[s])
                return 0;
    }
    return 1;
}

/* the lists of an invalid row: nothing selected, nothing missed */
static void pad_invalid_row(int k_max, int32_t *ss, uint8_t *sh, int32_t *mb, int32_t *ms, int32_t *mc)
{
    for (int i = 0; i < k_max; ++i) {
        ss[i] = -1;
        sh[i] = 0;
        mb[i] = ms[i] = -1;
    }
    *mc = -1;
}

typedef struct {
    uint32_t stamp;
    int32_t blk, slot;
} orc_touch;

static int by_touch(const void *a, const void *b)
{
    const orc_touch *x = (const orc_touch *)a, *y = (const orc_touch *)b;
    if (x->stamp != y->stamp)
        return x->stamp < y->stamp ? -1 : 1;
    if (x->blk != y->blk)
        return x->blk < y->blk ? -1 : 1;
    return (x->slot > y->slot) - (x->slot < y->slot);
}

void oracle_lru_load(oracle_lru *h, const int32_t *slot_block, const uint32_t *slot_stamp)
{
    const int C = h->cap;
    orc_touch *t = (orc_touch *)malloc(sizeof(orc_touch) * (size_t)(C > 0 ? C : 1));
    for (int r = 0; r < h->rows; ++r) {
        int32_t *sb = h->slot_block + (size_t)r * C;
        int n = 0;
        for (int s = 0; s < C; ++s) {
            sb[s] = slot_block[(size_t)r * C + s];
            h->prev[(size_t)r * C + s] = h->next[(size_t)r * C + s] = -1;
            if (sb[s] >= 0) {
                t[n].stamp = slot_stamp[(size_t)r * C + s];
                t[n].blk = sb[s];
                t[n].slot = s;
                ++n;
            }
        }
        h->head[r] = h->tail[r] = -1;
        qsort(t, (size_t)n, sizeof(orc_touch), by_touch);
        for (int i = 0; i < n; ++i)
            append_slot(h, r, t[i].slot);
    }
    free(t);
}

int oracle_lru_step(oracle_lru *h, int k_max, int nb_limit, const int32_t *sel, const int32_t *sel_count,
                    int32_t *sel_slot, uint8_t *sel_hit, int32_t *miss_block, int32_t *miss_slot,
                    int32_t *miss_count)
{
    const int C = h->cap;
#pragma omp parallel for schedule(dynamic)
    for (int r = 0; r < h->rows; ++r) {
        const int32_t *S = sel + (size_t)r * k_max;
        const int n = sel_count[r];
        int32_t *sb = h->slot_block + (size_t)r * C;
        int32_t *ss = sel_slot + (size_t)r * k_max;
        uint8_t *sh = sel_hit + (size_t)r * k_max;
        int32_t *mb = miss_block + (size_t)r * k_max, *ms = miss_slot + (size_t)r * k_max;
        if (!row_input_ok(S, n, k_max, nb_limit, sb, C)) {
            pad_invalid_row(k_max, ss, sh, mb, ms, miss_count + r);
            continue;
        }
        int32_t *victim = (int32_t *)malloc(sizeof(int32_t) * (size_t)(C > 0 ? C : 1));
        int nm = 0;
        for (int i = 0; i < n; ++i) {
            int found = -1;
            for (int s = 0; s < C; ++s)
                if (sb[s] == S[i]) {
                    found = s;
                    break;
                }
            ss[i] = found;
            sh[i] = (uint8_t)(found >= 0);
            if (found < 0)
                mb[nm++] = S[i];
        }
        int nv = 0;
        for (int s = 0; s < C && nv < nm; ++s)
            if (sb[s] < 0)
                victim[nv++] = s;
        for (int s = h->head[r]; s >= 0 && nv < nm; s = h->next[(size_t)r * C + s])
            if (!in_sorted(S, n, sb[s]))
                victim[nv++] = s;
        /* nv == nm always holds here because n <= C */
        for (int i = 0, m = 0; i < n; ++i)
            if (!sh[i]) {
                int v = victim[m];
                if (sb[v] >= 0)
                    unlink_slot(h, r, v);
                sb[v] = S[i];
                ss[i] = v;
                ms[m] = v;
                ++m;
            }
        for (int i = 0; i < n; ++i) {
            int s = ss[i];
            if (sh[i])
                unlink_slot(h, r, s);
            append_slot(h, r, s);
        }
        for (int i = n; i < k_max; ++i) {
            ss[i] = -1;
            sh[i] = 0;
        }
        for (int i = nm; i < k_max; ++i)
            mb[i] = ms[i] = -1;
        miss_count[r] = nm;
        free(victim);
    }
    return ORC_OK;
}

/*
 * Importance-capped eviction (OasisKV summary, key module 3: the important
 * blocks are compared with the resident ones, only the delta moves, and
 * when the capped HBM cache has no room the least important blocks are
 * evicted).  Reading: a block's importance is its score of the current step.
 * Hits and misses as for the LRU form; the victims are the empty slots in
 * ascending slot order, then the occupied slots whose block is not
 * selected, least important first: score ascending, then block id
 * ascending.  Miss i goes to victim i.
 *
 * The slot table [rows, cap] is the caller's and is updated in place.  An
 * invalid row (the same rules as the LRU step: a bad selection, a table id
 * outside [-1, nb_limit), or a block held by two slots) is left untouched
 * with miss_count = -1 and padded lists.
 */
typedef struct {
    double score;
    int32_t blk, slot;
} orc_cand;

static int by_score_then_block(const void *a, const void *b)
{
    const orc_cand *x = (const orc_cand *)a, *y = (const orc_cand *)b;
    if (x->score != y->score)
        return x->score < y->score ? -1 : 1;
    return (x->blk > y->blk) - (x->blk < y->blk);
}

int oracle_capped_step(int rows, int cap, int k_max, int nb_limit, int nb_max, const int32_t *sel,
                       const int32_t *sel_count, const double *scores, int32_t *slot_block, int32_t *sel_slot,
                       uint8_t *sel_hit, int32_t *miss_block, int32_t *miss_slot, int32_t *miss_count)
{
    const int C = cap;
#pragma omp parallel for schedule(dynamic)
    for (int r = 0; r < rows; ++r) {
        const int32_t *S = sel + (size_t)r * k_max;
        int32_t *sb = slot_block + (size_t)r * C;
        const int n = sel_count[r];
        int32_t *ss = sel_slot + (size_t)r * k_max;
        uint8_t *sh = sel_hit + (size_t)r * k_max;
        int32_t *mb = miss_block + (size_t)r * k_max, *ms = miss_slot + (size_t)r * k_max;
        if (!row_input_ok(S, n, k_max, nb_limit, sb, C)) {
            pad_invalid_row(k_max, ss, sh, mb, ms, miss_count + r);
            continue;
        }
        orc_cand *cand = (orc_cand *)malloc(sizeof(orc_cand) * (size_t)(C > 0 ? C : 1));
        int32_t *victim = (int32_t *)malloc(sizeof(int32_t) * (size_t)(C > 0 ? C : 1));
        int nm = 0;
        for (int i = 0; i < n; ++i) {
            int found = -1;
            for (int s = 0; s < C; ++s)
                if (sb[s] == S[i]) {
                    found = s;
                    break;
                }
            ss[i] = found;
            sh[i] = (uint8_t)(found >= 0);
            if (found < 0)
                mb[nm++] = S[i];
        }
        int nv = 0, nc = 0;
        for (int s = 0; s < C; ++s)
            if (sb[s] < 0)
                victim[nv++] = s;
        for (int s = 0; s < C; ++s)
            if (sb[s] >= 0 && !in_sorted(S, n, sb[s])) {
                cand[nc].score = scores[(size_t)r * nb_max + sb[s]];
                cand[nc].blk = sb[s];
                cand[nc].slot = s;
                ++nc;
            }
        qsort(cand, (size_t)nc, sizeof(orc_cand), by_score_then_block);
        for (int c = 0; c < nc; ++c)
            victim[nv++] = cand[c].slot;
        for (int i = 0, m = 0; i < n; ++i)
            if (!sh[i]) {
                int v = victim[m];
                sb[v] = S[i];
                ss[i] = v;
                ms[m] = v;
                ++m;
            }
        for (int i = n; i < k_max; ++i) {
            ss[i] = -1;
            sh[i] = 0;
        }
        for (int i = nm; i < k_max; ++i)
            mb[i] = ms[i] = -1;
        miss_count[r] = nm;
        free(cand);
        free(victim);
    }
    return ORC_OK;
}

/*
 * Decode-time append (the gains of the method concentrate where the KV grows
 * during decoding: "KV Cache 塞不进 HBM 了", intro and §1).  For every
 * sequence b with seq_lens[b] < T_max, the new key and value rows of each kv
 * head are stored at token seq_lens[b]; if the block holding that token is
 * resident in a slot of the row's working set (slot_block may be NULL), the
 * row is also stored in that slot, so every resident slot keeps the bytes of
 * its block.  Then seq_lens[b] grows by one.  A full sequence (seq_lens[b]
 * >= T_max) is left as it is.  Plain byte copies.
 */
/*
 * Consistency check of a working-set state (failure detection: a block
 * table must map each resident block to one slot, KV-Cache 压缩技术的工程原理
 * §5.2; a corrupted or mis-restored table is what its rollback / resync
 * guards against, same page §6.1).  Per row, flags[r] is the OR of
 *   1: a slot id outside [-1, nb_limit),
 *   2: one block held by two slots,
 *   4: an occupied slot whose stamp is ahead of the row's clock (every
 *      update stamps the slots it touches with the clock value it has just
 *      advanced to, so no stamp can exceed the clock).
 * Returns the number of rows with a nonzero flag.
 */
int oracle_check_state(int rows, int cap, int nb_limit, const int32_t *slot_block, const uint32_t *slot_stamp,
                       const uint32_t *clock, int32_t *flags)
{
    int bad_rows = 0;
    for (int r = 0; r < rows; ++r) {
        const int32_t *sb = slot_block + (size_t)r * cap;
        const uint32_t *st = slot_stamp + (size_t)r * cap;
        int f = 0;
        for (int s = 0; s < cap; ++s) {
            if (sb[s] < -1 || sb[s] >= nb_limit)
                f |= 1;
            for (int t = 0; t < s; ++t)
                if (sb[s] >= 0 && sb[t] == sb[s])
                    f |= 2;
            if (sb[s] >= 0 && st[s] > clock[r])
                f |= 4;
        }
        flags[r] = f;
        bad_rows += f != 0;
    }
    return bad_rows;
}

int oracle_append(int B, int Hkv, int D, int T_max, int block, int elem_bytes, const void *new_k,
                  const void *new_v, int32_t *seq_lens, void *k, void *v, const int32_t *slot_block, int cap,
                  void *pool_k, void *pool_v)
{
    const size_t rowb = (size_t)D * elem_bytes;
    for (int b = 0; b < B; ++b) {
        const int len = seq_lens[b];
        if (len < 0 || len >= T_max)
            continue;
        for (int j = 0; j < Hkv; ++j) {
            const size_t r = (size_t)b * Hkv + j;
            memcpy((char *)k + (r * T_max + len) * rowb, (const char *)new_k + r * rowb, rowb);
            memcpy((char *)v + (r * T_max + len) * rowb, (const char *)new_v + r * rowb, rowb);
            if (!slot_block)
                continue;
            for (int s = 0; s < cap; ++s)
                if (slot_block[r * cap + s] == len / block) {
                    const size_t po = ((r * cap + s) * block + len % block) * rowb;
                    memcpy((char *)pool_k + po, (const char *)new_k + r * rowb, rowb);
                    memcpy((char *)pool_v + po, (const char *)new_v + r * rowb, rowb);
                }
        }
        seq_lens[b] = len + 1;
    }
    return ORC_OK;
}

/*
 * Fetch: copy the rows of every missed block from the source cache into its
 * slot (hit detection, replacement and fetch are one pass in HiSparse;
 * "to_load" blocks are what moves in "KV Cache 塞不进 HBM 了" §3 step 1).
 * Byte copy, so bit-exact by construction.
 */
int oracle_gather(int rows, int cap, int T_max, int D, int elem_bytes, int block, int k_max,
                  const int32_t *miss_block, const int32_t *miss_slot, const int32_t *miss_count,
                  const void *src_k, const void *src_v, void *pool_k, void *pool_v)
{
    size_t rowb = (size_t)D * elem_bytes, blkb = rowb * block;
    for (int r = 0; r < rows; ++r) {
        int n = miss_count[r];
        for (int i = 0; i < n; ++i) {
            int blk = miss_block[(size_t)r * k_max + i], s = miss_slot[(size_t)r * k_max + i];
            size_t so = ((size_t)r * T_max + (size_t)blk * block) * rowb;
            size_t po = ((size_t)r * cap + s) * blkb;
            memcpy((char *)pool_k + po, (const char *)src_k + so, blkb);
            memcpy((char *)pool_v + po, (const char *)src_v + so, blkb);
        }
    }
    return ORC_OK;
}

/*
 * Attention over the selected blocks, read straight from the source cache
 * by block id.  For query head h (kv head j = h / G):
 *   z_t  = scale * <q[b,h], k[b,j,t]>   for the valid tokens t of the
 *          selected blocks (t < seq_len)
 *   out  = sum_t softmax(z)_t * v[b,j,t],  lse = log sum_t exp(z_t)
 * Exact attention over the kept KV (OasisKV summary, key module 1); the
 * result does not depend on which memory tier held the blocks (HiSparse
 * promo, insight 1).  No valid token: out = 0, lse = -inf.
 */
int oracle_attention(int B, int Hq, int Hkv, int D, int T_max, int block, int dtype,
                     const void *q, const void *k, const void *v, const int32_t *sel,
                     const int32_t *sel_count, int k_max, const int32_t *seq_lens, double scale,
                     double *out, double *lse)
{
    if (Hq % Hkv)
        return ORC_BAD;
    const int G = Hq / Hkv;
#pragma omp parallel for collapse(2) schedule(dynamic)
    for (int b = 0; b < B; ++b)
        for (int h = 0; h < Hq; ++h) {
            int j = h / G;
            int len = seq_lens[b] < T_max ? seq_lens[b] : T_max;
            const int32_t *S = sel + ((size_t)b * Hkv + j) * k_max;
            int n = sel_count[(size_t)b * Hkv + j];
            double *o = out + ((size_t)b * Hq + h) * D;
            double *qd = (double *)malloc(sizeof(double) * D);
            for (int d = 0; d < D; ++d)
                qd[d] = widen(q, dtype, ((size_t)b * Hq + h) * D + d);
            /* pass 1: logits and their maximum */
            int ntok = 0;
            for (int i = 0; i < n; ++i) {
                int t0 = S[i] * block, t1 = t0 + block < len ? t0 + block : len;
                if (t1 > t0)
                    ntok += t1 - t0;
            }
            double *z = (double *)malloc(sizeof(double) * (size_t)(ntok > 0 ? ntok : 1));
            int32_t *tok = (int32_t *)malloc(sizeof(int32_t) * (size_t)(ntok > 0 ? ntok : 1));
            int m = 0;
            double zmax = -INFINITY;
            for (int i = 0; i < n; ++i) {
                int t0 = S[i] * block, t1 = t0 + block < len ? t0 + block : len;
                for (int t = t0; t < t1; ++t) {
                    size_t kb = (((size_t)b * Hkv + j) * T_max + t) * D;
                    double dot = 0.0;
                    for (int d = 0; d < D; ++d)
                        dot += qd[d] * widen(k, dtype, kb + d);
                    z[m] = scale * dot;
                    tok[m] = t;
                    if (z[m] > zmax)
                        zmax = z[m];
                    ++m;
                }
            }
            for (int d = 0; d < D; ++d)
                o[d] = 0.0;
            if (m == 0) {
                if (lse)
                    lse[(size_t)b * Hq + h] = -INFINITY;
            } else {
                double l = 0.0;
                for (int i = 0; i < m; ++i)
                    l += exp(z[i] - zmax);
                for (int i = 0; i < m; ++i) {
                    double p = exp(z[i] - zmax) / l;
                    size_t vb = (((size_t)b * Hkv + j) * T_max + tok[i]) * D;
                    for (int d = 0; d < D; ++d)
                        o[d] += p * widen(v, dtype, vb + d);
                }
                if (lse)
                    lse[(size_t)b * Hq + h] = zmax + log(l);
            }
            free(z);
            free(tok);
            free(qd);
        }
    return ORC_OK;
}

/*
 * The same attention read through the slot table instead of from the
 * source: block S[i] is taken from pool[b, j, slot[i]].  Used to check that
 * the tier holding a block does not change the result.
 */
int oracle_attention_pool(int B, int Hq, int Hkv, int D, int cap, int block, int dtype,
                          const void *q, const void *pool_k, const void *pool_v, const int32_t *sel,
                          const int32_t *sel_slot, const int32_t *sel_count, int k_max,
                          const int32_t *seq_lens, double scale, double *out, double *lse)
{
    if (Hq % Hkv)
        return ORC_BAD;
    const int G = Hq / Hkv;
#pragma omp parallel for collapse(2) schedule(dynamic)
    for (int b = 0; b < B; ++b)
        for (int h = 0; h < Hq; ++h) {
            int j = h / G;
            int len = seq_lens[b];
            size_t row = (size_t)b * Hkv + j;
            const int32_t *S = sel + row * k_max, *SL = sel_slot + row * k_max;
            int n = sel_count[row];
            double *o = out + ((size_t)b * Hq + h) * D;
            double zmax = -INFINITY;
            for (int pass = 0; pass < 2; ++pass) {
                double l = 0.0;
                if (pass == 1)
                    for (int d = 0; d < D; ++d)
                        o[d] = 0.0;
                for (int i = 0; i < n; ++i) {
                    int t0 = S[i] * block, t1 = t0 + block < len ? t0 + block : len;
                    for (int t = t0; t < t1; ++t) {
                        size_t kb = ((row * cap + SL[i]) * block + (t - t0)) * D;
                        double dot = 0.0;
                        for (int d = 0; d < D; ++d)
                            dot += widen(q, dtype, ((size_t)b * Hq + h) * D + d) * widen(pool_k, dtype, kb + d);
                        double zz = scale * dot;
                        if (pass == 0) {
                            if (zz > zmax)
                                zmax = zz;
                        } else {
                            double p = exp(zz - zmax);
                            l += p;
                            for (int d = 0; d < D; ++d)
                                o[d] += p * widen(pool_v, dtype, kb + d);
                        }
                    }
                }
                if (pass == 1) {
                    if (l > 0.0) {
                        for (int d = 0; d < D; ++d)
                            o[d] /= l;
                        if (lse)
                            lse[(size_t)b * Hq + h] = zmax + log(l);
                    } else if (lse)
                        lse[(size_t)b * Hq + h] = -INFINITY;
                }
            }
        }
    return ORC_OK;
}
