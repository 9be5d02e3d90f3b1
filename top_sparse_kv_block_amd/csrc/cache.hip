// Stage 3: delta / working-set manager and miss fetch on gfx950.
//
// Each (sequence, kv-head) row owns a fixed set of slots holding whole
// 16-token blocks (a fixed-size GPU working set kept LRU: HiSparse promo,
// insight 1; the slot table is a block table: KV-Cache 压缩技术的工程原理
// §5.2).  A step diffs the selection S against the resident blocks, keeps
// hits in place, and sends only the misses S - R to victim slots ("KV Cache
// 塞不进 HBM 了" §2.1 and §3 step 1; OasisKV summary, key module 3).  Hit
// detection, replacement and the clock update are one kernel with no host
// synchronisation, the clock advanced by a device atomic (HiSparse promo,
// insight 2).  Evicted slots are overwritten in place (KV-Cache 压缩技术的工程
// 原理 §4.3).
//
// Importance-capped eviction (OasisKV summary, key module 3: when the capped
// cache has no room the least important blocks go) is the same kernel with
// the row's scores of this step: occupied unselected slots are then ranked
// by (score, block id) instead of (stamp, block id).
//
// LRU as stamps.  Every slot of S gets the row's new clock value, and the
// least recently used slot is the smallest (stamp, block id).  Because a
// step touches its blocks in ascending id order, ordering by (stamp, id) is
// exactly the order of a linked list that appends S in ascending order, so
// parallel code reproduces the list bit for bit.
//
// cache_update_kernel: one 1024-thread workgroup per row, state in LDS (with
// 1024 threads each candidate slot is ranked by 8 lanes: 9.5 us per call at
// 64 rows x 128 slots against 12.5 us with 256 threads).
//   hits:    every occupied slot binary-searches its block in S (S is
//            ascending); a hit claims S[i] with an LDS compare-and-swap, so
//            a selected block resident twice is detected, and the other
//            occupied slots pass an LDS set of block ids, which detects an
//            unselected one.
//   misses:  S indices without a slot, compacted in ascending order with a
//            workgroup prefix count.
//   victims: candidate slots (empty, or occupied and not hit) ranked by the
//            64-bit key (occupied, stamp, block-or-slot) precomputed in LDS;
//            rank r < #misses takes miss r.
//   The count, selection and slot table are read in one round of
//   independent loads and the clock atomic is issued as soon as the row is
//   known to be valid (after hit detection), so its latency overlaps the
//   rest.
// gather_kernel: one wave per miss copies the block's K and V rows (16*D
// elements each) from the source (HBM, or mapped pinned host memory read
// over PCIe) into its slot with 16-byte loads and stores.
#include "skv_rowops.h"

namespace skv {

constexpr int kCacheThreads = 1024;

__global__ __launch_bounds__(kCacheThreads) void cache_update_kernel(
    const int32_t *__restrict__ sel_blocks, const int32_t *__restrict__ sel_count, int k, int C, int NB,
    int32_t *__restrict__ slot_block, uint32_t *__restrict__ slot_stamp, uint32_t *__restrict__ clock,
    int32_t *__restrict__ sel_slot, uint8_t *__restrict__ sel_hit, int32_t *__restrict__ miss_block,
    int32_t *__restrict__ miss_slot, int32_t *__restrict__ miss_count, const float *__restrict__ scores) {
    __shared__ int32_t sS[kMaxK];
    __shared__ CacheScratch cs;
    __shared__ uint32_t sClock;
    const int row = blockIdx.x;
    const int tid = threadIdx.x;
    const int32_t *S = sel_blocks + (size_t)row * k;
    int32_t *sb = slot_block + (size_t)row * C;
    uint32_t *ss = slot_stamp + (size_t)row * C;

    const int n = sel_count[row];
    SlotRegs<kCacheThreads> regs;
    load_slots<kCacheThreads>(regs, C, sb, ss);
    for (int i = tid; i < k; i += kCacheThreads)
        sS[i] = S[i];
    cache_plan_clear<kCacheThreads>(cs, k, C);  // published by the barrier below
    int32_t *o_slot = sel_slot + (size_t)row * k, *o_mb = miss_block + (size_t)row * k;
    int32_t *o_ms = miss_slot + (size_t)row * k;
    uint8_t *o_hit = sel_hit + (size_t)row * k;
    const bool bad_count = n < 0 || n > k || n > C;  // uniform over the workgroup
    if (bad_count) {
        write_invalid_lists<kCacheThreads>(k, o_slot, o_hit, o_mb, o_ms, miss_count + row);
        return;
    }
    __syncthreads();
    int bad;
    const int nm = cache_plan_row<kCacheThreads>(sS, n, C, NB, regs, cs, bad,
                                                 scores ? scores + (size_t)row * NB : nullptr);
    if (bad) {
        write_invalid_lists<kCacheThreads>(k, o_slot, o_hit, o_mb, o_ms, miss_count + row);
        return;
    }
    if (tid == 0)
        sClock = atomicAdd(&clock[row], 1u) + 1u;
    __syncthreads();
    const uint32_t now = sClock;
    write_lists<kCacheThreads>(sS, n, nm, k, cs, o_slot, o_hit, o_mb, o_ms, miss_count + row);
    for (int i = tid; i < n; i += kCacheThreads) {
        const int s = cs.slot_of[i];
        if (s >= 0 && s < C) {
            sb[s] = sS[i];
            ss[s] = now;
        }
    }
}

// select_kernel: the top-k and the working-set update of one row in one
// workgroup (the same results as the two calls, bit for bit): the row's selection
// stays in LDS between the two, the slot table is read while the top-k runs,
// and the plan is committed by the same workgroup.  Rows up to 8192 blocks
// run with 512 threads, up to 16384 with 1024; the top-k's bits go straight
// into the plan (select_plan_row).  Longer rows run the top-k's phase A
// (topk_chunk_kernel) first; select_long_kernel then takes the selection from
// its candidates and plans it with cache_plan_row.

// Writes a row's selection and lists and commits its plan (the selected
// slots take the blocks and the row's new clock as stamp); a refused row
// gets padded lists and keeps its table, stamps and clock.
template <int THREADS>
__device__ void select_commit(int row, int k, int C, int n, int nm, int bad, const int32_t *sS, const CacheScratch &cs,
                              int32_t *__restrict__ sel_blocks, int32_t *__restrict__ sel_count,
                              int32_t *__restrict__ sb, uint32_t *__restrict__ ss, uint32_t *__restrict__ clock,
                              int32_t *__restrict__ sel_slot, uint8_t *__restrict__ sel_hit,
                              int32_t *__restrict__ miss_block, int32_t *__restrict__ miss_slot,
                              int32_t *__restrict__ miss_count, uint32_t &sClock) {
    const int tid = threadIdx.x;
    for (int i = tid; i < k; i += THREADS)
        sel_blocks[(size_t)row * k + i] = sS[i];
    if (tid == 0)
        sel_count[row] = n;
    if (bad) {
        write_invalid_lists<THREADS>(k, sel_slot + (size_t)row * k, sel_hit + (size_t)row * k,
                                     miss_block + (size_t)row * k, miss_slot + (size_t)row * k, miss_count + row);
        return;
    }
    if (tid == 0)
        sClock = atomicAdd(&clock[row], 1u) + 1u;
    __syncthreads();
    const uint32_t now = sClock;
    write_lists<THREADS>(sS, n, nm, k, cs, sel_slot + (size_t)row * k, sel_hit + (size_t)row * k,
                         miss_block + (size_t)row * k, miss_slot + (size_t)row * k, miss_count + row);
    for (int i = tid; i < n; i += THREADS) {
        const int s = cs.slot_of[i];
        if (s >= 0 && s < C) {
            sb[s] = sS[i];
            ss[s] = now;
        }
    }
}

template <int THREADS, int KPT>
__global__ __launch_bounds__(THREADS) void select_kernel(
    const float *__restrict__ scores, const int32_t *__restrict__ seq_lens, int Hkv, int T, int NB, int k, int sink,
    int recent, int C, int32_t *__restrict__ sel_blocks, int32_t *__restrict__ sel_count,
    int32_t *__restrict__ slot_block, uint32_t *__restrict__ slot_stamp, uint32_t *__restrict__ clock,
    int32_t *__restrict__ sel_slot, uint8_t *__restrict__ sel_hit, int32_t *__restrict__ miss_block,
    int32_t *__restrict__ miss_slot, int32_t *__restrict__ miss_count) {
    __shared__ TopkScratch sc;
    __shared__ PlanScratch<THREADS> ps;
    __shared__ int32_t sS[kMaxK];
    __shared__ CacheScratch cs;
    __shared__ uint32_t sClock;
    const int row = blockIdx.x;
    TopkScores<KPT> pre;  // issued first (no dependence on the length)
    topk_load<KPT>(scores + (size_t)row * NB, NB, pre);
    const int len = min(max(seq_lens[row / Hkv], 0), T);
    int32_t *sb = slot_block + (size_t)row * C;
    uint32_t *ss = slot_stamp + (size_t)row * C;
    SlotRegs<THREADS> regs;  // in flight while the top-k runs
    load_slots<THREADS>(regs, C, sb, ss);
    select_plan_clear<THREADS>(cs, ps, k, C);  // published by the top-k's barriers
    int n, bad;
    const uint64_t take = topk_take_loaded<THREADS, KPT>(pre, len, NB, k, sink, recent, sc);
    const int nm = select_plan_row<THREADS, KPT>(take, k, C, NB, regs, sS, cs, ps, n, bad, [](int) {});
    select_commit<THREADS>(row, k, C, n, nm, bad, sS, cs, sel_blocks, sel_count, sb, ss, clock, sel_slot, sel_hit,
                           miss_block, miss_slot, miss_count, sClock);
}

// Long rows, phase B with the working-set update (after topk_chunk_kernel).
template <int KPT>
__global__ __launch_bounds__(kLongRowThreads) void select_long_kernel(
    const int32_t *__restrict__ seq_lens, int Hkv, int T, int NB, int k, int sink, int recent, int C,
    int chunk_blocks, int nchunks, const float *__restrict__ ws, int32_t *__restrict__ sel_blocks,
    int32_t *__restrict__ sel_count, int32_t *__restrict__ slot_block, uint32_t *__restrict__ slot_stamp,
    uint32_t *__restrict__ clock, int32_t *__restrict__ sel_slot, uint8_t *__restrict__ sel_hit,
    int32_t *__restrict__ miss_block, int32_t *__restrict__ miss_slot, int32_t *__restrict__ miss_count) {
    constexpr int THREADS = kLongRowThreads;
    __shared__ TopkScratch sc;
    __shared__ int32_t sS[kMaxK];
    __shared__ CacheScratch cs;
    __shared__ uint32_t sClock;
    const int row = blockIdx.x;
    const int nc = nchunks * long_row_stride(k);
    const float *wrow = ws + (size_t)row * 2 * nc;
    LongCands<KPT> cands;  // issued before the length is known
    long_row_load<KPT>(wrow, reinterpret_cast<const int32_t *>(wrow + nc), nc, cands);
    const int len = min(max(seq_lens[row / Hkv], 0), T);
    int32_t *sb = slot_block + (size_t)row * C;
    uint32_t *ss = slot_stamp + (size_t)row * C;
    SlotRegs<THREADS> regs;  // in flight while the selection runs
    load_slots<THREADS>(regs, C, sb, ss);
    cache_plan_clear<THREADS>(cs, k, C);  // published by the selection's barriers
    const int ncand = (min(nb_of(len), NB) + chunk_blocks - 1) / chunk_blocks * long_row_stride(k);
    const int n = long_row_select<THREADS, KPT>(cands, ncand, len, NB, k, sink, recent, sS, sc);
    int bad;
    const int nm = cache_plan_row<THREADS>(sS, n, C, NB, regs, cs, bad);
    select_commit<THREADS>(row, k, C, n, nm, bad, sS, cs, sel_blocks, sel_count, sb, ss, clock, sel_slot, sel_hit,
                           miss_block, miss_slot, miss_count, sClock);
}

// check_state_kernel: one 256-thread workgroup per row checks the row's
// working-set state (failure detection: a block table maps each resident
// block to one slot, KV-Cache 压缩技术的工程原理 §5.2) and writes flags[row]:
// 1 = a slot id outside [-1, NB), 2 = a block held by two slots (an LDS set
// of block ids, as in the update's plan), 4 = an occupied slot stamped after
// the row's clock.  Reads only; the state is not modified.
constexpr int kCheckThreads = 256;

__global__ __launch_bounds__(kCheckThreads) void check_state_kernel(const int32_t *__restrict__ slot_block,
                                                                    const uint32_t *__restrict__ slot_stamp,
                                                                    const uint32_t *__restrict__ clock, int C, int NB,
                                                                    int32_t *__restrict__ flags) {
    __shared__ int32_t dup[kDupSet];
    __shared__ int sflag;
    const int row = blockIdx.x, tid = threadIdx.x;
    SlotRegs<kCheckThreads> regs;
    load_slots<kCheckThreads>(regs, C, slot_block + (size_t)row * C, slot_stamp + (size_t)row * C);
    const uint32_t now = clock[row];
    const int bits = dup_set_bits(C);
    for (int i = tid; i < (1 << bits); i += kCheckThreads)
        dup[i] = -1;
    if (tid == 0)
        sflag = 0;
    __syncthreads();
    int f = 0;
#pragma unroll
    for (int u = 0; u < SlotRegs<kCheckThreads>::SPT; ++u) {
        const int s = tid + u * kCheckThreads;
        if (s < C) {
            const int32_t blk = regs.blk[u];
            if (blk < -1 || blk >= NB)
                f |= 1;
            if (blk >= 0 && dup_set_add(dup, bits, blk))
                f |= 2;
            if (blk >= 0 && regs.stamp[u] > now)
                f |= 4;
        }
    }
    if (f)
        atomicOr(&sflag, f);
    __syncthreads();
    if (tid == 0)
        flags[row] = sflag;
}

hipError_t launch_check_state(const Dims &d, int cap, const int32_t *slot_block, const uint32_t *slot_stamp,
                              const uint32_t *clock, int32_t *flags, hipStream_t st) {
    hipLaunchKernelGGL(check_state_kernel, dim3(d.rows()), dim3(kCheckThreads), 0, st, slot_block, slot_stamp, clock,
                       cap, d.NB, flags);
    return hipGetLastError();
}

// One wave copies one missed block: K then V, 16*D elements each.
template <int BLOCK_BYTES>
__global__ __launch_bounds__(256) void gather_kernel(const int32_t *__restrict__ miss_block,
                                                     const int32_t *__restrict__ miss_slot,
                                                     const int32_t *__restrict__ miss_count, int k, int C, int T,
                                                     int NB, const uint8_t *__restrict__ src_k,
                                                     const uint8_t *__restrict__ src_v, uint8_t *__restrict__ pool_k,
                                                     uint8_t *__restrict__ pool_v) {
    constexpr int ITER = BLOCK_BYTES / 1024;
    const int row = blockIdx.y;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int m = blockIdx.x * 4 + wave;
    const int nm = miss_count[row];
    if (m >= nm)
        return;
    const int blk = miss_block[(size_t)row * k + m];
    const int s = miss_slot[(size_t)row * k + m];
    if (blk < 0 || blk >= NB || s < 0 || s >= C)
        return;
    const size_t so = ((size_t)row * T + (size_t)blk * 16) * (BLOCK_BYTES / 16);
    const size_t po = ((size_t)row * C + s) * (size_t)BLOCK_BYTES;
    u32x4 a[ITER], c[ITER];
#pragma unroll
    for (int i = 0; i < ITER; ++i) {
        a[i] = load_nt(src_k + so + i * 1024 + lane * 16);
        c[i] = load_nt(src_v + so + i * 1024 + lane * 16);
    }
#pragma unroll
    for (int i = 0; i < ITER; ++i) {
        store16(pool_k + po + i * 1024 + lane * 16, a[i]);
        store16(pool_v + po + i * 1024 + lane * 16, c[i]);
    }
}

hipError_t launch_cache_update(const Dims &d, int k, int cap, const int32_t *sel_blocks, const int32_t *sel_count,
                               int32_t *slot_block, uint32_t *slot_stamp, uint32_t *clock, int32_t *sel_slot,
                               uint8_t *sel_hit, int32_t *miss_block, int32_t *miss_slot, int32_t *miss_count,
                               const float *scores, hipStream_t st) {
    hipLaunchKernelGGL(cache_update_kernel, dim3(d.rows()), dim3(kCacheThreads), 0, st, sel_blocks, sel_count, k,
                       cap, d.NB, slot_block, slot_stamp, clock, sel_slot, sel_hit, miss_block, miss_slot,
                       miss_count, scores);
    return hipGetLastError();
}

template <int THREADS, int KPT>
static hipError_t select_t(const Dims &d, const float *scores, const int32_t *lens, int k, int sink, int recent,
                           int cap, int32_t *sel_blocks, int32_t *sel_count, int32_t *slot_block, uint32_t *slot_stamp,
                           uint32_t *clock, int32_t *sel_slot, uint8_t *sel_hit, int32_t *miss_block,
                           int32_t *miss_slot, int32_t *miss_count, hipStream_t st) {
    hipLaunchKernelGGL((select_kernel<THREADS, KPT>), dim3(d.rows()), dim3(THREADS), 0, st, scores, lens, d.Hkv, d.T,
                       d.NB, k, sink, recent, cap, sel_blocks, sel_count, slot_block, slot_stamp, clock, sel_slot,
                       sel_hit, miss_block, miss_slot, miss_count);
    return hipGetLastError();
}

hipError_t launch_select(const Dims &d, const float *scores, const int32_t *lens, int k, int sink, int recent,
                         int cap, int32_t *sel_blocks, int32_t *sel_count, int32_t *slot_block, uint32_t *slot_stamp,
                         uint32_t *clock, int32_t *sel_slot, uint8_t *sel_hit, int32_t *miss_block,
                         int32_t *miss_slot, int32_t *miss_count, void *ws, hipStream_t st) {
#define SKV_SELECT(TH, KP)                                                                                          \
    return select_t<TH, KP>(d, scores, lens, k, sink, recent, cap, sel_blocks, sel_count, slot_block, slot_stamp, \
                            clock, sel_slot, sel_hit, miss_block, miss_slot, miss_count, st)
    const int kpt = (d.NB + 511) / 512;
    if (kpt <= 1)
        SKV_SELECT(512, 1);
    if (kpt <= 2)
        SKV_SELECT(512, 2);
    if (kpt <= 4)
        SKV_SELECT(512, 4);
    if (kpt <= 8)
        SKV_SELECT(512, 8);
    if (kpt <= 16)
        SKV_SELECT(512, 16);
    if (kpt <= 32)
        SKV_SELECT(1024, 16);
#undef SKV_SELECT
    hipError_t e = launch_topk_chunks(d, scores, lens, k, sink, recent, static_cast<float *>(ws), st);
    if (e != hipSuccess)
        return e;
    const int ch = long_row_chunk(d.NB, k), nch = long_row_chunks(d.NB, k);
    const float *w = static_cast<const float *>(ws);
#define SKV_SELECT_LONG(KP)                                                                                       \
    hipLaunchKernelGGL(select_long_kernel<KP>, dim3(d.rows()), dim3(kLongRowThreads), 0, st, lens, d.Hkv, d.T,     \
                       d.NB, k, sink, recent, cap, ch, nch, w, sel_blocks, sel_count, slot_block, slot_stamp, clock, \
                       sel_slot, sel_hit, miss_block, miss_slot, miss_count)
    switch (long_row_kpt(d, k)) {
    case 4:
        SKV_SELECT_LONG(4);
        break;
    case 8:
        SKV_SELECT_LONG(8);
        break;
    default:
        SKV_SELECT_LONG(32);
    }
#undef SKV_SELECT_LONG
    return hipGetLastError();
}

template <int BB>
static hipError_t gather_t(const Dims &d, int k, int cap, const int32_t *mb, const int32_t *ms, const int32_t *mc,
                           const void *sk, const void *sv, void *pk, void *pv, hipStream_t st) {
    dim3 grid((k + 3) / 4, d.rows());
    hipLaunchKernelGGL((gather_kernel<BB>), grid, dim3(256), 0, st, mb, ms, mc, k, cap, d.T, d.NB,
                       (const uint8_t *)sk, (const uint8_t *)sv, (uint8_t *)pk, (uint8_t *)pv);
    return hipGetLastError();
}

hipError_t launch_gather(const Dims &d, int k, int cap, const int32_t *mb, const int32_t *ms, const int32_t *mc,
                         const void *sk, const void *sv, void *pk, void *pv, hipStream_t st) {
    const int bb = 16 * d.D * d.elem_bytes();
    switch (bb) {
    case 2048:
        return gather_t<2048>(d, k, cap, mb, ms, mc, sk, sv, pk, pv, st);
    case 4096:
        return gather_t<4096>(d, k, cap, mb, ms, mc, sk, sv, pk, pv, st);
    default:
        return gather_t<8192>(d, k, cap, mb, ms, mc, sk, sv, pk, pv, st);
    }
}

}  // namespace skv
