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
// LRU as stamps.  Every slot of S gets the row's new clock value, and the
// least recently used slot is the smallest (stamp, block id).  Because a
// step touches its blocks in ascending id order, ordering by (stamp, id) is
// exactly the order of a linked list that appends S in ascending order, so
// parallel code reproduces the list bit for bit.
//
// cache_update_kernel: one 256-thread workgroup per row, state in LDS.
//   hits:    every occupied slot binary-searches its block in S (S is
//            ascending); a hit claims S[i] with an LDS compare-and-swap, so
//            a block resident twice is detected.
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
#include "skv_device.h"
#include "skv_launch.h"

namespace skv {

constexpr int kCacheThreads = 256;
constexpr int kCacheWaves = kCacheThreads / 64;

// inclusive-scan helper over the workgroup: returns the exclusive prefix of
// v in thread order and the total
__device__ __forceinline__ int wg_exclusive_scan(int v, int *wsum, int &total) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    int x = v;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        int y = __shfl_up(x, off);
        if (lane >= off)
            x += y;
    }
    if (lane == 63)
        wsum[wave] = x;
    __syncthreads();
    int base = 0, tot = 0;
#pragma unroll
    for (int w = 0; w < kCacheWaves; ++w) {
        base += (w < wave) ? wsum[w] : 0;
        tot += wsum[w];
    }
    __syncthreads();
    total = tot;
    return base + x - v;
}

__device__ __forceinline__ int find_sorted(const int32_t *S, int n, int32_t x) {
    int lo = 0, hi = n - 1;
    while (lo <= hi) {
        const int mid = (lo + hi) >> 1;
        const int32_t v = S[mid];
        if (v == x)
            return mid;
        if (v < x)
            lo = mid + 1;
        else
            hi = mid - 1;
    }
    return -1;
}

__global__ __launch_bounds__(kCacheThreads) void cache_update_kernel(
    const int32_t *__restrict__ sel_blocks, const int32_t *__restrict__ sel_count, int k, int C, int NB,
    int32_t *__restrict__ slot_block, uint32_t *__restrict__ slot_stamp, uint32_t *__restrict__ clock,
    int32_t *__restrict__ sel_slot, uint8_t *__restrict__ sel_hit, int32_t *__restrict__ miss_block,
    int32_t *__restrict__ miss_slot, int32_t *__restrict__ miss_count) {
    __shared__ int32_t sS[kMaxK];       // selection
    __shared__ int32_t sSlotOf[kMaxK];  // slot of S[i]
    __shared__ uint8_t sHit[kMaxK];
    __shared__ int32_t sMissI[kMaxK];   // S index of miss m
    __shared__ int32_t sBlk[kMaxCapacity];
    __shared__ uint64_t sKey[kMaxCapacity];  // LRU key of a candidate slot, ~0 otherwise
    __shared__ int wsum[kCacheWaves];
    __shared__ uint32_t sClock;

    const int row = blockIdx.x;
    const int tid = threadIdx.x;
    const int32_t *S = sel_blocks + (size_t)row * k;
    int32_t *sb = slot_block + (size_t)row * C;
    uint32_t *ss = slot_stamp + (size_t)row * C;

    // one round of independent global loads: count, selection, slot table
    const int n = sel_count[row];
    for (int i = tid; i < k; i += kCacheThreads) {
        sS[i] = S[i];
        sSlotOf[i] = -1;
    }
    uint32_t stamp_reg[(kMaxCapacity + kCacheThreads - 1) / kCacheThreads];
#pragma unroll
    for (int u = 0; u < (kMaxCapacity + kCacheThreads - 1) / kCacheThreads; ++u) {
        const int s = tid + u * kCacheThreads;
        if (s < C) {
            sBlk[s] = sb[s];
            stamp_reg[u] = ss[s];
        }
    }
    __syncthreads();
    const bool bad_count = n < 0 || n > k || n > C;
    const int nn = bad_count ? 0 : n;
    int bad = bad_count ? 1 : 0;
    for (int i = tid; i < nn; i += kCacheThreads) {
        const int32_t v = sS[i];
        if (v < 0 || v >= NB || (i > 0 && v <= sS[i - 1]))
            bad = 1;
    }
    for (int s = tid; s < C; s += kCacheThreads)
        if (sBlk[s] < -1 || sBlk[s] >= NB)
            bad = 1;
    if (__syncthreads_or(bad)) {
        if (tid == 0)
            miss_count[row] = -1;
        return;
    }
    // hits: each occupied slot looks its block up in the ascending selection
    int dup = 0;
    for (int s = tid; s < C; s += kCacheThreads) {
        const int32_t blk = sBlk[s];
        const int i = blk >= 0 ? find_sorted(sS, nn, blk) : -1;
        if (i >= 0 && atomicCAS(&sSlotOf[i], -1, s) != -1)
            dup = 1;
    }
    if (__syncthreads_or(dup)) {  // a block resident twice: nothing written yet
        if (tid == 0)
            miss_count[row] = -1;
        return;
    }
    // the row is valid: advance its clock now; the value is needed only at
    // the end, so the atomic's latency overlaps the work below
    uint32_t now = 0;
    if (tid == 0)
        now = atomicAdd(&clock[row], 1u) + 1u;

    // misses, compacted in ascending S order: thread t owns S indices
    // [t*per, t*per+per)
    const int per = (k + kCacheThreads - 1) / kCacheThreads;
    int cnt = 0;
    for (int u = 0; u < per; ++u) {
        const int i = tid * per + u;
        if (i < nn) {
            const bool hit = sSlotOf[i] >= 0;
            sHit[i] = hit ? 1 : 0;
            cnt += hit ? 0 : 1;
        }
    }
    int nm;
    int pos = wg_exclusive_scan(cnt, wsum, nm);
    for (int u = 0; u < per; ++u) {
        const int i = tid * per + u;
        if (i < nn && !sHit[i])
            sMissI[pos++] = i;
    }
    // LRU keys of the candidate slots (empty, or occupied and not selected):
    // empty slots first by slot index, then (stamp, block) ascending
#pragma unroll
    for (int u = 0; u < (kMaxCapacity + kCacheThreads - 1) / kCacheThreads; ++u) {
        const int s = tid + u * kCacheThreads;
        if (s < C) {
            const int32_t blk = sBlk[s];
            const bool taken = blk >= 0 && find_sorted(sS, nn, blk) >= 0;
            sKey[s] = taken ? ~0ull
                            : (blk < 0 ? (uint64_t)s
                                       : ((1ull << 63) | ((uint64_t)stamp_reg[u] << 31) | (uint64_t)blk));
        }
    }
    __syncthreads();

    // victims: candidate rank r < #misses takes miss r.  Keys of a valid
    // table are distinct; the slot index breaks ties of a corrupt one.
    if (nm > 0) {
        for (int s = tid; s < C; s += kCacheThreads) {
            const uint64_t key = sKey[s];
            if (key == ~0ull)
                continue;
            int rank = 0;
#pragma unroll 8
            for (int o = 0; o < C; ++o) {
                const uint64_t ok = sKey[o];
                rank += (ok < key || (ok == key && o < s)) ? 1 : 0;
            }
            if (rank < nm)
                sSlotOf[sMissI[rank]] = s;
        }
    }
    if (tid == 0)
        sClock = now;
    __syncthreads();
    now = sClock;

    int32_t *o_slot = sel_slot + (size_t)row * k;
    uint8_t *o_hit = sel_hit + (size_t)row * k;
    int32_t *o_mb = miss_block + (size_t)row * k;
    int32_t *o_ms = miss_slot + (size_t)row * k;
    for (int i = tid; i < k; i += kCacheThreads) {
        const bool in = i < nn;
        const int s = in ? sSlotOf[i] : -1;
        o_slot[i] = s;
        o_hit[i] = in ? sHit[i] : 0;
        if (in && s >= 0 && s < C) {
            sb[s] = sS[i];
            ss[s] = now;
        }
        const bool mi = i < nm;
        const int si = mi ? sMissI[i] : 0;
        o_mb[i] = mi ? sS[si] : -1;
        o_ms[i] = mi ? sSlotOf[si] : -1;
    }
    if (tid == 0)
        miss_count[row] = nm;
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
                               hipStream_t st) {
    hipLaunchKernelGGL(cache_update_kernel, dim3(d.rows()), dim3(kCacheThreads), 0, st, sel_blocks, sel_count, k,
                       cap, d.NB, slot_block, slot_stamp, clock, sel_slot, sel_hit, miss_block, miss_slot,
                       miss_count);
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
