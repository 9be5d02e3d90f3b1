// C ABI of the sparse KV-cache decode step: argument validation on the host,
// then stream-ordered kernel launches.  Nothing here allocates, synchronises
// or keeps state between calls.
#include "sparse_kv.h"
#include "skv_launch.h"

#include <hip/hip_runtime.h>

#include <mutex>

#define SKV_API extern "C" __attribute__((visibility("default")))

// Scratch of sparse_kv_select_attend_noalloc: the per-split partials of the
// fused call, in a device array that every GPU the library runs on holds
// from module load to the end of the process.  Host code uses the address
// hipGetSymbolAddress gives for the current device, never the array's name.
static __device__ __align__(256) uint8_t scratch[SKV_NOALLOC_SCRATCH_BYTES];

namespace {

using skv::Dims;

skv_status check_shape(const skv_shape *s, Dims &d) {
    if (!s)
        return SKV_ERR_NULL;
    if (s->dtype != SKV_F32 && s->dtype != SKV_BF16)
        return SKV_ERR_DTYPE;
    if (s->batch < 1 || s->n_q_heads < 1 || s->n_kv_heads < 1 || s->n_q_heads % s->n_kv_heads != 0)
        return SKV_ERR_SHAPE;
    if (s->head_dim != 64 && s->head_dim != 128)
        return SKV_ERR_SHAPE;
    if (s->block_size != 16 || s->max_ctx < 16 || s->max_ctx % 16 != 0)
        return SKV_ERR_SHAPE;
    if ((long long)s->batch * s->n_kv_heads > 65535)
        return SKV_ERR_SHAPE;
    d.B = s->batch;
    d.Hq = s->n_q_heads;
    d.Hkv = s->n_kv_heads;
    d.D = s->head_dim;
    d.T = s->max_ctx;
    d.NB = s->max_ctx / 16;
    d.dtype = s->dtype;
    return SKV_OK;
}

skv_status hip_status(hipError_t e) { return e == hipSuccess ? SKV_OK : SKV_ERR_HIP; }

int nb_blocks(int tokens) { return (tokens + 15) / 16; }

// The top-k's workspace: only rows over 16384 blocks need one.
bool topk_workspace_ok(const Dims &d, int k, const void *ws, size_t bytes) {
    const size_t need = skv::long_row_ws_bytes(d, k);
    return need == 0 || (ws && bytes >= need && ((uintptr_t)ws & 255u) == 0);
}

}  // namespace

SKV_API skv_status sparse_kv_score(const skv_shape *shape, int32_t mode, const void *q, int32_t n_queries,
                                   const void *keys_or_meta, const int32_t *seq_lens, float scale, float *scores,
                                   void *stream) {
    Dims d;
    skv_status st = check_shape(shape, d);
    if (st != SKV_OK)
        return st;
    if (!q || !keys_or_meta || !seq_lens || !scores)
        return SKV_ERR_NULL;
    if (n_queries < 1 || n_queries > 4 || n_queries * d.G() > skv::kMaxQueryRows)
        return SKV_ERR_SHAPE;
    hipStream_t s = (hipStream_t)stream;
    if (mode == SKV_SCORE_BLOCKMAX)
        return hip_status(skv::launch_score_blockmax(d, q, n_queries, keys_or_meta, seq_lens, scale, scores, s));
    if (mode == SKV_SCORE_QUEST)
        return hip_status(skv::launch_score_quest(d, q, n_queries, keys_or_meta, seq_lens, scale, scores, s));
    return SKV_ERR_UNSUPPORTED;
}

SKV_API skv_status sparse_kv_topk(const skv_shape *shape, const float *scores, const int32_t *seq_lens,
                                  int32_t k_blocks, int32_t sink_tokens, int32_t recent_tokens, int32_t *sel_blocks,
                                  int32_t *sel_count, void *workspace, size_t workspace_bytes, void *stream) {
    Dims d;
    skv_status st = check_shape(shape, d);
    if (st != SKV_OK)
        return st;
    if (!scores || !seq_lens || !sel_blocks || !sel_count)
        return SKV_ERR_NULL;
    if (d.NB > skv::kMaxTopkBlocks)
        return SKV_ERR_UNSUPPORTED;
    if (k_blocks < 1 || k_blocks > d.NB || k_blocks > skv::kMaxK || sink_tokens < 0 || recent_tokens < 0)
        return SKV_ERR_SHAPE;
    if (sink_tokens > 0 || recent_tokens > 0) {
        const long long forced_max = (long long)nb_blocks(sink_tokens) + nb_blocks(recent_tokens) + 1;
        if (forced_max > k_blocks)
            return SKV_ERR_CAPACITY;
    }
    if (!topk_workspace_ok(d, k_blocks, workspace, workspace_bytes))
        return SKV_ERR_WORKSPACE;
    return hip_status(skv::launch_topk(d, scores, seq_lens, k_blocks, sink_tokens, recent_tokens, sel_blocks,
                                       sel_count, workspace, (hipStream_t)stream));
}

static skv_status cache_update_impl(const skv_shape *shape, int32_t k_blocks, int32_t capacity,
                                    const int32_t *sel_blocks, const int32_t *sel_count, const float *scores,
                                    int32_t *slot_block, uint32_t *slot_stamp, uint32_t *clock, int32_t *sel_slot,
                                    uint8_t *sel_hit, int32_t *miss_block, int32_t *miss_slot, int32_t *miss_count,
                                    const void *src_k, const void *src_v, int32_t src_kind, void *pool_k,
                                    void *pool_v, void *stream) {
    Dims d;
    skv_status st = check_shape(shape, d);
    if (st != SKV_OK)
        return st;
    if (!sel_blocks || !sel_count || !slot_block || !slot_stamp || !clock || !sel_slot || !sel_hit || !miss_block ||
        !miss_slot || !miss_count)
        return SKV_ERR_NULL;
    if (k_blocks < 1 || k_blocks > skv::kMaxK || capacity < 1)
        return SKV_ERR_SHAPE;
    if (capacity < k_blocks)
        return SKV_ERR_CAPACITY;
    if (capacity > skv::kMaxCapacity || d.NB > skv::kMaxUpdateBlocks)
        return SKV_ERR_UNSUPPORTED;
    if (src_kind != SKV_SRC_DEVICE && src_kind != SKV_SRC_HOST_MAPPED)
        return SKV_ERR_SHAPE;
    const bool fetch = src_k || src_v;
    if (fetch && (!src_k || !src_v || !pool_k || !pool_v))
        return SKV_ERR_NULL;
    hipStream_t s = (hipStream_t)stream;
    hipError_t e = skv::launch_cache_update(d, k_blocks, capacity, sel_blocks, sel_count, slot_block, slot_stamp,
                                            clock, sel_slot, sel_hit, miss_block, miss_slot, miss_count, scores, s);
    if (e != hipSuccess || !fetch)
        return hip_status(e);
    return hip_status(
        skv::launch_gather(d, k_blocks, capacity, miss_block, miss_slot, miss_count, src_k, src_v, pool_k, pool_v, s));
}

SKV_API skv_status sparse_kv_cache_update(const skv_shape *shape, int32_t k_blocks, int32_t capacity,
                                          const int32_t *sel_blocks, const int32_t *sel_count, int32_t *slot_block,
                                          uint32_t *slot_stamp, uint32_t *clock, int32_t *sel_slot,
                                          uint8_t *sel_hit, int32_t *miss_block, int32_t *miss_slot,
                                          int32_t *miss_count, const void *src_k, const void *src_v,
                                          int32_t src_kind, void *pool_k, void *pool_v, void *stream) {
    return cache_update_impl(shape, k_blocks, capacity, sel_blocks, sel_count, nullptr, slot_block, slot_stamp,
                             clock, sel_slot, sel_hit, miss_block, miss_slot, miss_count, src_k, src_v, src_kind,
                             pool_k, pool_v, stream);
}

SKV_API skv_status sparse_kv_cache_update_importance(const skv_shape *shape, int32_t k_blocks, int32_t capacity,
                                                     const int32_t *sel_blocks, const int32_t *sel_count,
                                                     const float *scores, int32_t *slot_block, uint32_t *slot_stamp,
                                                     uint32_t *clock, int32_t *sel_slot, uint8_t *sel_hit,
                                                     int32_t *miss_block, int32_t *miss_slot, int32_t *miss_count,
                                                     const void *src_k, const void *src_v, int32_t src_kind,
                                                     void *pool_k, void *pool_v, void *stream) {
    if (!scores)
        return SKV_ERR_NULL;
    return cache_update_impl(shape, k_blocks, capacity, sel_blocks, sel_count, scores, slot_block, slot_stamp, clock,
                             sel_slot, sel_hit, miss_block, miss_slot, miss_count, src_k, src_v, src_kind, pool_k,
                             pool_v, stream);
}

SKV_API skv_status sparse_kv_select(const skv_shape *shape, const float *scores, const int32_t *seq_lens,
                                    int32_t k_blocks, int32_t sink_tokens, int32_t recent_tokens, int32_t capacity,
                                    int32_t *sel_blocks, int32_t *sel_count, int32_t *slot_block,
                                    uint32_t *slot_stamp, uint32_t *clock, int32_t *sel_slot, uint8_t *sel_hit,
                                    int32_t *miss_block, int32_t *miss_slot, int32_t *miss_count,
                                    const void *src_k, const void *src_v, int32_t src_kind, void *pool_k,
                                    void *pool_v, void *workspace, size_t workspace_bytes, void *stream) {
    Dims d;
    skv_status st = check_shape(shape, d);
    if (st != SKV_OK)
        return st;
    if (!scores || !seq_lens || !sel_blocks || !sel_count || !slot_block || !slot_stamp || !clock || !sel_slot ||
        !sel_hit || !miss_block || !miss_slot || !miss_count)
        return SKV_ERR_NULL;
    if (d.NB > skv::kMaxTopkBlocks)
        return SKV_ERR_UNSUPPORTED;
    if (k_blocks < 1 || k_blocks > d.NB || k_blocks > skv::kMaxK || sink_tokens < 0 || recent_tokens < 0 ||
        capacity < 1)
        return SKV_ERR_SHAPE;
    if (capacity < k_blocks)
        return SKV_ERR_CAPACITY;
    if (capacity > skv::kMaxCapacity)
        return SKV_ERR_UNSUPPORTED;
    if (sink_tokens > 0 || recent_tokens > 0) {
        const long long forced_max = (long long)nb_blocks(sink_tokens) + nb_blocks(recent_tokens) + 1;
        if (forced_max > k_blocks)
            return SKV_ERR_CAPACITY;
    }
    if (src_kind != SKV_SRC_DEVICE && src_kind != SKV_SRC_HOST_MAPPED)
        return SKV_ERR_SHAPE;
    const bool fetch = src_k || src_v;
    if (fetch && (!src_k || !src_v || !pool_k || !pool_v))
        return SKV_ERR_NULL;
    if (!topk_workspace_ok(d, k_blocks, workspace, workspace_bytes))
        return SKV_ERR_WORKSPACE;
    hipStream_t s = (hipStream_t)stream;
    hipError_t e = skv::launch_select(d, scores, seq_lens, k_blocks, sink_tokens, recent_tokens, capacity, sel_blocks,
                                      sel_count, slot_block, slot_stamp, clock, sel_slot, sel_hit, miss_block,
                                      miss_slot, miss_count, workspace, s);
    if (e != hipSuccess || !fetch)
        return hip_status(e);
    return hip_status(skv::launch_gather(d, k_blocks, capacity, miss_block, miss_slot, miss_count, src_k, src_v,
                                         pool_k, pool_v, s));
}

SKV_API skv_status sparse_kv_append(const skv_shape *shape, const void *new_k, const void *new_v, int32_t *seq_lens,
                                    void *keys, void *values, void *meta, const int32_t *slot_block, int32_t capacity,
                                    void *pool_k, void *pool_v, void *stream) {
    Dims d;
    skv_status st = check_shape(shape, d);
    if (st != SKV_OK)
        return st;
    if (!new_k || !new_v || !seq_lens || !keys || !values)
        return SKV_ERR_NULL;
    if (slot_block) {
        if (!pool_k || !pool_v)
            return SKV_ERR_NULL;
        if (capacity < 1)
            return SKV_ERR_SHAPE;
        if (capacity > skv::kMaxCapacity)
            return SKV_ERR_UNSUPPORTED;
    }
    return hip_status(skv::launch_append(d, new_k, new_v, seq_lens, keys, values, meta, slot_block,
                                         slot_block ? capacity : 0, pool_k, pool_v, (hipStream_t)stream));
}

SKV_API int32_t sparse_decode_attention_splits(const skv_shape *shape, int32_t k_blocks) {
    Dims d;
    if (check_shape(shape, d) != SKV_OK || k_blocks < 1)
        return 0;
    return skv::attention_auto_splits(d.rows(), k_blocks);
}

SKV_API int32_t sparse_kv_select_attend_splits(const skv_shape *shape, int32_t k_blocks) {
    Dims d;
    if (check_shape(shape, d) != SKV_OK || k_blocks < 1)
        return 0;
    return skv::fused_auto_splits(d, k_blocks);
}

SKV_API size_t sparse_decode_attention_workspace_bytes(const skv_shape *shape, int32_t k_blocks, int32_t num_splits) {
    Dims d;
    if (check_shape(shape, d) != SKV_OK || k_blocks < 1 || num_splits < 0 || num_splits > k_blocks ||
        num_splits > skv::kMaxSplits)
        return 0;
    const int splits = num_splits == 0 ? skv::attention_auto_splits(d.rows(), k_blocks) : num_splits;
    return skv::attention_ws_bytes(d.rows(), d.G(), d.D, splits);
}

SKV_API size_t sparse_kv_topk_workspace_bytes(const skv_shape *shape, int32_t k_blocks) {
    Dims d;
    if (check_shape(shape, d) != SKV_OK || k_blocks < 1 || k_blocks > d.NB || k_blocks > skv::kMaxK ||
        d.NB > skv::kMaxTopkBlocks)
        return 0;
    return skv::long_row_ws_bytes(d, k_blocks);
}

SKV_API size_t sparse_kv_workspace_bytes(const skv_shape *shape, int32_t k_blocks, int32_t num_splits) {
    Dims d;
    if (check_shape(shape, d) != SKV_OK || k_blocks < 1 || k_blocks > skv::kMaxK || num_splits < 0 ||
        num_splits > k_blocks || num_splits > skv::kMaxSplits)
        return 0;
    const int att = num_splits == 0 ? skv::attention_auto_splits(d.rows(), k_blocks) : num_splits;
    const int fused = num_splits == 0 ? skv::fused_auto_splits(d, k_blocks) : num_splits;
    size_t need = skv::attention_ws_bytes(d.rows(), d.G(), d.D, att);
    if (k_blocks <= d.NB && d.NB <= skv::kMaxTopkBlocks) {
        // the fused call's (partials, then the top-k's candidates) covers the top-k's own
        const size_t f = skv::fused_ws_bytes(d, k_blocks, fused);
        need = f > need ? f : need;
    }
    return need;
}

SKV_API skv_status sparse_decode_attention(const skv_shape *shape, const void *q, void *pool_k, void *pool_v,
                                           int32_t capacity, const int32_t *sel_blocks, const int32_t *sel_slot,
                                           const uint8_t *sel_hit, const int32_t *sel_count, const int32_t *seq_lens,
                                           int32_t k_blocks, float scale, int32_t num_splits, const void *src_k,
                                           const void *src_v, int32_t src_kind, float *out, float *lse,
                                           void *workspace, size_t workspace_bytes, void *stream) {
    Dims d;
    skv_status st = check_shape(shape, d);
    if (st != SKV_OK)
        return st;
    if (!q || !pool_k || !pool_v || !sel_blocks || !sel_slot || !sel_count || !seq_lens || !out)
        return SKV_ERR_NULL;
    if (k_blocks < 1 || k_blocks > skv::kMaxK || capacity < 1 || num_splits < 0 || num_splits > k_blocks ||
        num_splits > skv::kMaxSplits)
        return SKV_ERR_SHAPE;
    if (src_kind != SKV_SRC_DEVICE && src_kind != SKV_SRC_HOST_MAPPED)
        return SKV_ERR_SHAPE;
    const bool fetch = src_k || src_v;
    if (fetch && (!src_k || !src_v || !sel_hit))
        return SKV_ERR_NULL;
    if (d.G() > skv::kMaxGroup)
        return SKV_ERR_UNSUPPORTED;
    const int splits = num_splits == 0 ? skv::attention_auto_splits(d.rows(), k_blocks) : num_splits;
    const size_t need = skv::attention_ws_bytes(d.rows(), d.G(), d.D, splits);
    if (!workspace || workspace_bytes < need || ((uintptr_t)workspace & 255u) != 0)
        return SKV_ERR_WORKSPACE;
    skv::AttnArgs a{q,         pool_k, pool_v,       capacity, sel_blocks, sel_slot, sel_hit, sel_count,
                    seq_lens,  k_blocks, scale,      splits,   src_k,      src_v,    out,     lse,
                    workspace};
    return hip_status(skv::launch_attention(d, a, (hipStream_t)stream));
}

namespace {

// Argument checks of the fused call (everything but the workspace); on
// success d holds the dims and splits the resolved split count.
skv_status check_select_attend(const skv_shape *shape, const float *scores, const int32_t *seq_lens,
                               int32_t k_blocks, int32_t sink_tokens, int32_t recent_tokens, int32_t capacity,
                               const int32_t *sel_blocks, const int32_t *sel_count, const int32_t *slot_block,
                               const uint32_t *slot_stamp, const uint32_t *clock, const int32_t *sel_slot,
                               const uint8_t *sel_hit, const int32_t *miss_block, const int32_t *miss_slot,
                               const int32_t *miss_count, const void *q, const void *pool_k, const void *pool_v,
                               const void *src_k, const void *src_v, int32_t src_kind, int32_t num_splits,
                               const float *out, Dims &d, int &splits) {
    skv_status st = check_shape(shape, d);
    if (st != SKV_OK)
        return st;
    if (!scores || !seq_lens || !sel_blocks || !sel_count || !slot_block || !slot_stamp || !clock || !sel_slot ||
        !sel_hit || !miss_block || !miss_slot || !miss_count || !q || !pool_k || !pool_v || !src_k || !src_v || !out)
        return SKV_ERR_NULL;
    if (d.NB > skv::kMaxTopkBlocks)
        return SKV_ERR_UNSUPPORTED;
    if (k_blocks < 1 || k_blocks > d.NB || k_blocks > skv::kMaxK || sink_tokens < 0 || recent_tokens < 0 ||
        capacity < 1 || num_splits < 0 || num_splits > k_blocks || num_splits > skv::kMaxSplits)
        return SKV_ERR_SHAPE;
    if (capacity < k_blocks)
        return SKV_ERR_CAPACITY;
    if (capacity > skv::kMaxCapacity || d.G() > skv::kMaxGroup)
        return SKV_ERR_UNSUPPORTED;
    if (sink_tokens > 0 || recent_tokens > 0) {
        const long long forced_max = (long long)nb_blocks(sink_tokens) + nb_blocks(recent_tokens) + 1;
        if (forced_max > k_blocks)
            return SKV_ERR_CAPACITY;
    }
    if (src_kind != SKV_SRC_DEVICE && src_kind != SKV_SRC_HOST_MAPPED)
        return SKV_ERR_SHAPE;
    splits = num_splits == 0 ? skv::fused_auto_splits(d, k_blocks) : num_splits;
    return SKV_OK;
}

// The address of this process's scratch array on the current device,
// looked up once per device (hipGetSymbolAddress, with that device
// current) and kept.
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxDevices] = {};

hipError_t scratch_on_current_device(void **ptr) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess)
        return e;
    if (dev < 0 || dev >= kMaxDevices)
        return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess)
            return e;
        g_scratch_ptr[dev] = p;
    }
    *ptr = g_scratch_ptr[dev];
    return hipSuccess;
}

}  // namespace

SKV_API skv_status sparse_kv_select_attend(const skv_shape *shape, const float *scores, const int32_t *seq_lens,
                                           int32_t k_blocks, int32_t sink_tokens, int32_t recent_tokens,
                                           int32_t capacity, int32_t *sel_blocks, int32_t *sel_count,
                                           int32_t *slot_block, uint32_t *slot_stamp, uint32_t *clock,
                                           int32_t *sel_slot, uint8_t *sel_hit, int32_t *miss_block,
                                           int32_t *miss_slot, int32_t *miss_count, const void *q, void *pool_k,
                                           void *pool_v, const void *src_k, const void *src_v, int32_t src_kind,
                                           float scale, int32_t num_splits, float *out, float *lse, void *workspace,
                                           size_t workspace_bytes, void *stream) {
    Dims d;
    int splits = 0;
    skv_status st = check_select_attend(shape, scores, seq_lens, k_blocks, sink_tokens, recent_tokens, capacity,
                                        sel_blocks, sel_count, slot_block, slot_stamp, clock, sel_slot, sel_hit,
                                        miss_block, miss_slot, miss_count, q, pool_k, pool_v, src_k, src_v, src_kind,
                                        num_splits, out, d, splits);
    if (st != SKV_OK)
        return st;
    const size_t need = skv::fused_ws_bytes(d, k_blocks, splits);
    if (!workspace || workspace_bytes < need || ((uintptr_t)workspace & 255u) != 0)
        return SKV_ERR_WORKSPACE;
    skv::FusedArgs f{scores,   seq_lens,  k_blocks,  sink_tokens, recent_tokens, capacity,   sel_blocks,
                     sel_count, slot_block, slot_stamp, clock,     sel_slot,      sel_hit,    miss_block,
                     miss_slot, miss_count, q,          pool_k,    pool_v,        src_k,      src_v,
                     scale,     splits,     out,        lse,       workspace};
    return hip_status(skv::launch_select_attend(d, f, (hipStream_t)stream));
}

SKV_API skv_status sparse_kv_select_attend_noalloc(const skv_shape *shape, const float *scores,
                                                   const int32_t *seq_lens, int32_t k_blocks, int32_t sink_tokens,
                                                   int32_t recent_tokens, int32_t capacity, int32_t *sel_blocks,
                                                   int32_t *sel_count, int32_t *slot_block, uint32_t *slot_stamp,
                                                   uint32_t *clock, int32_t *sel_slot, uint8_t *sel_hit,
                                                   int32_t *miss_block, int32_t *miss_slot, int32_t *miss_count,
                                                   const void *q, void *pool_k, void *pool_v, const void *src_k,
                                                   const void *src_v, int32_t src_kind, float scale,
                                                   int32_t num_splits, float *out, float *lse, void *stream) {
    Dims d;
    int splits = 0;
    skv_status st = check_select_attend(shape, scores, seq_lens, k_blocks, sink_tokens, recent_tokens, capacity,
                                        sel_blocks, sel_count, slot_block, slot_stamp, clock, sel_slot, sel_hit,
                                        miss_block, miss_slot, miss_count, q, pool_k, pool_v, src_k, src_v, src_kind,
                                        num_splits, out, d, splits);
    if (st != SKV_OK)
        return st;
    if (skv::fused_ws_bytes(d, k_blocks, splits) > (size_t)SKV_NOALLOC_SCRATCH_BYTES)
        return SKV_ERR_SCRATCH;
    void *ws = nullptr;
    hipError_t e = scratch_on_current_device(&ws);
    if (e != hipSuccess)
        return SKV_ERR_HIP;
    // every split workgroup writes its whole partial before the merge reads
    // it, so nothing in the scratch needs clearing between calls
    skv::FusedArgs f{scores,   seq_lens,  k_blocks,  sink_tokens, recent_tokens, capacity,   sel_blocks,
                     sel_count, slot_block, slot_stamp, clock,     sel_slot,      sel_hit,    miss_block,
                     miss_slot, miss_count, q,          pool_k,    pool_v,        src_k,      src_v,
                     scale,     splits,     out,        lse,       ws};
    return hip_status(skv::launch_select_attend(d, f, (hipStream_t)stream));
}

SKV_API skv_status sparse_kv_check_state(const skv_shape *shape, int32_t capacity, const int32_t *slot_block,
                                         const uint32_t *slot_stamp, const uint32_t *clock, int32_t *flags,
                                         void *stream) {
    Dims d;
    skv_status st = check_shape(shape, d);
    if (st != SKV_OK)
        return st;
    if (!slot_block || !slot_stamp || !clock || !flags)
        return SKV_ERR_NULL;
    if (capacity < 1)
        return SKV_ERR_SHAPE;
    if (capacity > skv::kMaxCapacity)
        return SKV_ERR_UNSUPPORTED;
    return hip_status(skv::launch_check_state(d, capacity, slot_block, slot_stamp, clock, flags, (hipStream_t)stream));
}

SKV_API skv_status sparse_kv_quest_meta(const skv_shape *shape, const void *keys, const int32_t *seq_lens, void *meta,
                                        void *stream) {
    Dims d;
    skv_status st = check_shape(shape, d);
    if (st != SKV_OK)
        return st;
    if (!keys || !seq_lens || !meta)
        return SKV_ERR_NULL;
    return hip_status(skv::launch_quest_meta(d, keys, seq_lens, meta, (hipStream_t)stream));
}

SKV_API skv_status sparse_kv_stream_read(const skv_shape *shape, const void *keys, uint32_t *sink, void *stream) {
    Dims d;
    skv_status st = check_shape(shape, d);
    if (st != SKV_OK)
        return st;
    if (!keys || !sink)
        return SKV_ERR_NULL;
    return hip_status(skv::launch_stream_read(d, keys, sink, (hipStream_t)stream));
}

SKV_API skv_status sparse_kv_host_alloc(size_t bytes, void **host_ptr, void **device_ptr) {
    if (!host_ptr || !device_ptr)
        return SKV_ERR_NULL;
    *host_ptr = nullptr;
    *device_ptr = nullptr;
    if (bytes == 0)
        return SKV_ERR_SHAPE;
    void *h = nullptr;
    if (hipHostMalloc(&h, bytes, hipHostMallocMapped | hipHostMallocPortable) != hipSuccess)
        return SKV_ERR_HIP;
    void *dptr = nullptr;
    if (hipHostGetDevicePointer(&dptr, h, 0) != hipSuccess) {
        (void)hipHostFree(h);
        return SKV_ERR_HIP;
    }
    *host_ptr = h;
    *device_ptr = dptr;
    return SKV_OK;
}

SKV_API skv_status sparse_kv_host_free(void *host_ptr) {
    if (!host_ptr)
        return SKV_ERR_NULL;
    return hip_status(hipHostFree(host_ptr));
}

SKV_API const char *sparse_kv_status_string(skv_status s) {
    switch (s) {
    case SKV_OK:
        return "ok";
    case SKV_ERR_NULL:
        return "a required pointer is NULL";
    case SKV_ERR_SHAPE:
        return "sizes are inconsistent or outside the supported range";
    case SKV_ERR_DTYPE:
        return "unsupported dtype";
    case SKV_ERR_CAPACITY:
        return "capacity smaller than k_blocks, or forced blocks exceed k_blocks";
    case SKV_ERR_WORKSPACE:
        return "workspace missing, misaligned or too small";
    case SKV_ERR_UNSUPPORTED:
        return "request not supported by this library";
    case SKV_ERR_HIP:
        return "HIP runtime error at launch";
    case SKV_ERR_SCRATCH:
        return "the call needs more scratch than the library's static buffer holds (SKV_NOALLOC_SCRATCH_BYTES)";
    }
    return "unknown status";
}
