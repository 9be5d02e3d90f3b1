// Internal launchers (host side) for the gfx950 kernels.  The C ABI in
// abi.hip validates arguments and then calls these; each returns the
// hipError_t of its launch(es).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace skv {

struct Dims {
    int B, Hq, Hkv, D, T, NB, dtype;  // dtype: 0 = f32, 1 = bf16
    int rows() const { return B * Hkv; }
    int G() const { return Hq / Hkv; }
    int elem_bytes() const { return dtype == 0 ? 4 : 2; }
};

hipError_t launch_score_blockmax(const Dims &d, const void *q, int n_queries, const void *keys,
                                 const int32_t *seq_lens, float scale, float *scores, hipStream_t st);
hipError_t launch_score_quest(const Dims &d, const void *q, int n_queries, const void *meta,
                              const int32_t *seq_lens, float scale, float *scores, hipStream_t st);
hipError_t launch_stream_read(const Dims &d, const void *keys, uint32_t *sink, hipStream_t st);
hipError_t launch_quest_meta(const Dims &d, const void *keys, const int32_t *seq_lens, void *meta,
                             hipStream_t st);
hipError_t launch_topk(const Dims &d, const float *scores, const int32_t *seq_lens, int k, int sink,
                       int recent, int32_t *sel_blocks, int32_t *sel_count, void *ws, hipStream_t st);
// Rows over 16384 blocks: the top-k's first (chunk) launch and its workspace
// size (0 for shorter rows), the keys per thread of the second launch.
hipError_t launch_topk_chunks(const Dims &d, const float *scores, const int32_t *seq_lens, int k, int sink,
                              int recent, float *ws, hipStream_t st);
size_t long_row_ws_bytes(const Dims &d, int k);
int long_row_kpt(const Dims &d, int k);
hipError_t launch_cache_update(const Dims &d, int k, int cap, const int32_t *sel_blocks,
                               const int32_t *sel_count, int32_t *slot_block, uint32_t *slot_stamp,
                               uint32_t *clock, int32_t *sel_slot, uint8_t *sel_hit, int32_t *miss_block,
                               int32_t *miss_slot, int32_t *miss_count, const float *scores, hipStream_t st);
hipError_t launch_append(const Dims &d, const void *new_k, const void *new_v, int32_t *seq_lens, void *keys,
                         void *values, void *meta, const int32_t *slot_block, int cap, void *pool_k, void *pool_v,
                         hipStream_t st);
hipError_t launch_select(const Dims &d, const float *scores, const int32_t *lens, int k, int sink, int recent,
                         int cap, int32_t *sel_blocks, int32_t *sel_count, int32_t *slot_block, uint32_t *slot_stamp,
                         uint32_t *clock, int32_t *sel_slot, uint8_t *sel_hit, int32_t *miss_block,
                         int32_t *miss_slot, int32_t *miss_count, void *ws, hipStream_t st);
hipError_t launch_check_state(const Dims &d, int cap, const int32_t *slot_block, const uint32_t *slot_stamp,
                              const uint32_t *clock, int32_t *flags, hipStream_t st);
hipError_t launch_gather(const Dims &d, int k, int cap, const int32_t *miss_block, const int32_t *miss_slot,
                         const int32_t *miss_count, const void *src_k, const void *src_v, void *pool_k,
                         void *pool_v, hipStream_t st);
struct AttnArgs {
    const void *q;
    void *pool_k, *pool_v;
    int cap;
    const int32_t *sel_blocks, *sel_slot;
    const uint8_t *sel_hit;  // needed only with a source
    const int32_t *sel_count, *seq_lens;
    int k;
    float scale;
    int splits;
    const void *src_k, *src_v;  // NULL: every selected block is already in the pool
    float *out, *lse;
    void *ws;
};
hipError_t launch_attention(const Dims &d, const AttnArgs &a, hipStream_t st);
struct FusedArgs {
    const float *scores;
    const int32_t *seq_lens;
    int k, sink, recent, cap;
    int32_t *sel_blocks, *sel_count, *slot_block;
    uint32_t *slot_stamp, *clock;
    int32_t *sel_slot;
    uint8_t *sel_hit;
    int32_t *miss_block, *miss_slot, *miss_count;
    const void *q;
    void *pool_k, *pool_v;
    const void *src_k, *src_v;
    float scale;
    int splits;
    float *out, *lse;
    void *ws;
};
hipError_t launch_select_attend(const Dims &d, const FusedArgs &f, hipStream_t st);

// limits shared by validation and launch code
constexpr int kMaxQueryRows = 32;  // G * n_queries for scoring
constexpr int kMaxTopkBlocks = 65536;
constexpr int kMaxK = 1024;
constexpr int kMaxCapacity = 1024;
constexpr int kMaxUpdateBlocks = 1 << 21;  // NB limit of the working-set update (block ids in 21 key bits)
constexpr int kMaxGroup = 16;  // G for attention
constexpr int kMaxSplits = 128;

int attention_auto_splits(int rows, int k);
int fused_auto_splits(const Dims &d, int k);
size_t attention_ws_bytes(int rows, int G, int D, int splits);
// Workspace of the fused call: the partials, then (rows over 16384 blocks)
// the top-k's chunk candidates.
size_t fused_ws_bytes(const Dims &d, int k, int splits);

}  // namespace skv
