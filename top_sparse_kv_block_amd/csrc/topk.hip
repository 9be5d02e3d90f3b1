// Stage 2: per-(sequence, kv-head) top-k under the KV budget on gfx950.
//
// Each row keeps its forced blocks (the ones covering the first sink tokens
// and the last recent tokens: sink + recent + top-scored, "KV Cache 塞不进 HBM
// 了" §2.3) and fills the rest of its budget (a per-head, per-step cap, same
// page §3 step 2) with the best-scored remaining valid blocks, ties broken
// towards the lower block id.  Output is ascending by block id.
//
// One 1024-thread workgroup per row.  Scores become order-preserving 32-bit
// keys held in registers (KPT per thread, thread t owns the contiguous ids
// [t*KPT, t*KPT+KPT)).  Four 8-bit radix passes with an LDS histogram find
// the key of the last block the budget admits and how many blocks with
// exactly that key still fit; one pass of two workgroup prefix sums then
// emits the chosen ids in ascending order (ties at the threshold go to the
// lowest ids because the equal-key rank is a prefix count in id order).
#include "skv_device.h"
#include "skv_launch.h"

namespace skv {

constexpr int kTopkThreads = 1024;
constexpr int kTopkWaves = kTopkThreads / 64;

__device__ __forceinline__ uint32_t order_key(float f) {
    uint32_t u = __float_as_uint(f + 0.0f);  // -0 -> +0 so equal floats give equal keys
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Exclusive prefix sum over the 1024 threads in thread order; also returns
// the total.  `wsum` is LDS scratch of kTopkWaves entries.
__device__ __forceinline__ uint32_t block_exclusive_scan(uint32_t v, uint32_t *wsum, uint32_t &total) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    uint32_t x = v;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        uint32_t y = __shfl_up(x, off);
        if (lane >= off)
            x += y;
    }
    if (lane == 63)
        wsum[wave] = x;
    __syncthreads();
    uint32_t base = 0, tot = 0;
#pragma unroll
    for (int w = 0; w < kTopkWaves; ++w) {
        uint32_t s = wsum[w];
        base += (w < wave) ? s : 0u;
        tot += s;
    }
    __syncthreads();
    total = tot;
    return base + x - v;
}

template <int KPT>
__global__ __launch_bounds__(kTopkThreads) void topk_kernel(const float *__restrict__ scores,
                                                            const int32_t *__restrict__ seq_lens, int Hkv, int T,
                                                            int NB, int k, int sink, int recent,
                                                            int32_t *__restrict__ sel_blocks,
                                                            int32_t *__restrict__ sel_count) {
    __shared__ uint32_t hist[256];
    __shared__ uint32_t wsum[kTopkWaves];
    __shared__ uint32_t sh_digit, sh_remaining;

    const int row = blockIdx.x;
    const int b = row / Hkv;
    const int tid = threadIdx.x;
    const int len = min(max(seq_lens[b], 0), T);
    const int nvalid = min(nb_of(len), NB);
    int32_t *out = sel_blocks + (size_t)row * k;

    if (nvalid <= k) {
        for (int i = tid; i < k; i += kTopkThreads)
            out[i] = i < nvalid ? i : -1;
        if (tid == 0)
            sel_count[row] = nvalid;
        return;
    }
    // forced ranges [0, fs) and [fr, nvalid)
    const int fs = sink > 0 ? min(nb_of(min(sink, len)), nvalid) : 0;
    const int fr = recent > 0 ? max(0, len - recent) / 16 : nvalid;
    const int n_forced = fs + (nvalid - fr) - max(0, fs - fr);
    const int need = k - n_forced;

    const float *srow = scores + (size_t)row * NB;
    uint32_t key[KPT];
    uint64_t cand = 0, forced = 0;  // bit m: id tid*KPT+m is a candidate / forced
#pragma unroll
    for (int m = 0; m < KPT; ++m) {
        const int i = tid * KPT + m;
        key[m] = 0;
        if (i < nvalid) {
            if (i < fs || i >= fr) {
                forced |= 1ull << m;
            } else {
                cand |= 1ull << m;
                key[m] = order_key(srow[i]);
            }
        }
    }

    uint32_t prefix = 0, mask = 0;
    uint32_t remaining = (uint32_t)max(need, 0);
    if (need > 0) {
#pragma unroll 1
        for (int pass = 0; pass < 4; ++pass) {
            const int shift = 24 - 8 * pass;
            if (tid < 256)
                hist[tid] = 0;
            __syncthreads();
#pragma unroll
            for (int m = 0; m < KPT; ++m)
                if (((cand >> m) & 1u) && (key[m] & mask) == prefix)
                    atomicAdd(&hist[(key[m] >> shift) & 255u], 1u);
            __syncthreads();
            // find the digit holding the remaining-th largest key: an
            // inclusive scan over the bins from the top digit down (waves
            // 0-3 scan; every wave reaches both barriers)
            uint32_t c = 0, x = 0;
            if (tid < 256) {
                const int lane = tid & 63;
                c = hist[255 - tid];
                x = c;
#pragma unroll
                for (int off = 1; off < 64; off <<= 1) {
                    uint32_t y = __shfl_up(x, off);
                    if (lane >= off)
                        x += y;
                }
                if (lane == 63)
                    wsum[tid >> 6] = x;
            }
            __syncthreads();
            if (tid < 256) {
                uint32_t base = 0;
                for (int w = 0; w < (tid >> 6); ++w)
                    base += wsum[w];
                const uint32_t incl = base + x, excl = incl - c;
                if (excl < remaining && remaining <= incl) {
                    sh_digit = 255u - (uint32_t)tid;
                    sh_remaining = remaining - excl;
                }
            }
            __syncthreads();
            prefix |= sh_digit << shift;
            mask |= 255u << shift;
            remaining = sh_remaining;
            __syncthreads();
        }
    }
    const uint32_t tau = prefix;  // key of the last admitted block; `remaining` of that key are taken

    uint32_t n_eq = 0;
#pragma unroll
    for (int m = 0; m < KPT; ++m)
        n_eq += (need > 0 && ((cand >> m) & 1u) && key[m] == tau) ? 1u : 0u;
    uint32_t tot;
    uint32_t eq_rank = block_exclusive_scan(n_eq, wsum, tot);
    uint64_t take = 0;  // bit m: selected
#pragma unroll
    for (int m = 0; m < KPT; ++m) {
        const bool c = (cand >> m) & 1u;
        bool s = ((forced >> m) & 1u) || (need > 0 && c && key[m] > tau);
        if (need > 0 && c && key[m] == tau) {
            s = eq_rank < remaining;
            ++eq_rank;
        }
        take |= (uint64_t)s << m;
    }
    uint32_t pos = block_exclusive_scan((uint32_t)__builtin_popcountll(take), wsum, tot);
#pragma unroll
    for (int m = 0; m < KPT; ++m)
        if (((take >> m) & 1u) && pos < (uint32_t)k)
            out[pos++] = tid * KPT + m;
    tot = min(tot, (uint32_t)k);
    for (int i = (int)tot + tid; i < k; i += kTopkThreads)
        out[i] = -1;
    if (tid == 0)
        sel_count[row] = (int)tot;
}

template <int KPT>
static hipError_t topk_t(const Dims &d, const float *scores, const int32_t *lens, int k, int sink, int recent,
                         int32_t *sel, int32_t *cnt, hipStream_t st) {
    hipLaunchKernelGGL((topk_kernel<KPT>), dim3(d.rows()), dim3(kTopkThreads), 0, st, scores, lens, d.Hkv, d.T, d.NB,
                       k, sink, recent, sel, cnt);
    return hipGetLastError();
}

hipError_t launch_topk(const Dims &d, const float *scores, const int32_t *lens, int k, int sink, int recent,
                       int32_t *sel, int32_t *cnt, hipStream_t st) {
    const int kpt = (d.NB + kTopkThreads - 1) / kTopkThreads;
    if (kpt <= 1)
        return topk_t<1>(d, scores, lens, k, sink, recent, sel, cnt, st);
    if (kpt <= 2)
        return topk_t<2>(d, scores, lens, k, sink, recent, sel, cnt, st);
    if (kpt <= 4)
        return topk_t<4>(d, scores, lens, k, sink, recent, sel, cnt, st);
    if (kpt <= 8)
        return topk_t<8>(d, scores, lens, k, sink, recent, sel, cnt, st);
    if (kpt <= 16)
        return topk_t<16>(d, scores, lens, k, sink, recent, sel, cnt, st);
    if (kpt <= 32)
        return topk_t<32>(d, scores, lens, k, sink, recent, sel, cnt, st);
    return topk_t<64>(d, scores, lens, k, sink, recent, sel, cnt, st);
}

}  // namespace skv
