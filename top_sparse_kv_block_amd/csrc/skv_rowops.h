// Row-level device routines shared by the standalone stage kernels and the
// fused select -> update -> attend kernel, so that both give bit-identical
// results.  A "row" is one (sequence, kv-head) pair; each routine is called
// by every thread of one workgroup (they contain barriers).
#pragma once

#include "skv_device.h"
#include "skv_launch.h"

namespace skv {

// ------------------------------------------------------------ scans
// Exclusive prefix sum of v over the workgroup in thread order, and the total.
template <int THREADS, typename T>
__device__ __forceinline__ T wg_exclusive_scan(T v, T *wsum, T &total) {
    constexpr int WAVES = THREADS / 64;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    (void)lane;
    const T x = (T)wave_incl_scan((uint32_t)v);
    if (lane == 63)
        wsum[wave] = x;
    __syncthreads();
    T base = 0, tot = 0;
#pragma unroll
    for (int w = 0; w < WAVES; ++w) {
        const T s = wsum[w];
        base += (w < wave) ? s : T(0);
        tot += s;
    }
    __syncthreads();
    total = tot;
    return base + x - v;
}

// ------------------------------------------------------------ top-k
__device__ __forceinline__ uint32_t order_key(float f) {
    uint32_t u = __float_as_uint(f + 0.0f);  // -0 -> +0 so equal floats give equal keys
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

struct TopkScratch {
    uint32_t hist[2][256];  // passes alternate buffers, so clearing needs no barrier of its own
    uint32_t wsum[16];
    uint32_t digit, remaining, n_tau;
};

// Wave 0 finds the digit bin holding the `remaining`-th largest key of the
// pass: lane l scans bins 255-4l .. 252-4l, a DPP scan adds the lanes.
// Writes the digit, the rank left inside its bin and the bin's count.
__device__ __forceinline__ void pick_digit(const uint32_t *hist, uint32_t remaining, TopkScratch &sc) {
    const int lane = threadIdx.x & 63;
    uint32_t c[4], t = 0;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
        c[u] = hist[255 - 4 * lane - u];
        t += c[u];
    }
    uint32_t run = wave_incl_scan(t) - t;  // keys in higher bins
#pragma unroll
    for (int u = 0; u < 4; ++u) {
        if (run < remaining && remaining <= run + c[u]) {
            sc.digit = 255u - (uint32_t)(4 * lane + u);
            sc.remaining = remaining - run;
            sc.n_tau = c[u];
        }
        run += c[u];
    }
}

// Per-row selection under the budget (sink + recent blocks forced, the rest
// by (score desc, id asc)); writes the ascending ids to out[0, count) and -1
// to out[count, k) and returns count.  Thread t owns ids [t*KPT, t*KPT+KPT);
// four 8-bit radix passes over order-preserving keys find the key of the
// last admitted block, and one pass of two prefix sums emits the ids in
// ascending order (ties at the threshold go to the lowest ids).
template <int THREADS, int KPT>
__device__ int topk_row(const float *__restrict__ srow, int len, int NB, int k, int sink, int recent, int32_t *out,
                        TopkScratch &sc) {
    const int tid = threadIdx.x;
    const int nvalid = min(nb_of(len), NB);
    if (nvalid <= k) {
        for (int i = tid; i < k; i += THREADS)
            out[i] = i < nvalid ? i : -1;
        __syncthreads();
        return nvalid;
    }
    const int fs = sink > 0 ? min(nb_of(min(sink, len)), nvalid) : 0;
    const int fr = recent > 0 ? max(0, len - recent) / 16 : nvalid;
    const int n_forced = fs + (nvalid - fr) - max(0, fs - fr);
    const int need = k - n_forced;

    uint32_t key[KPT];
    uint64_t cand = 0, forced = 0;
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
    uint32_t remaining = (uint32_t)max(need, 0), n_tau = 0;
    if (need > 0) {
        if (tid < 256)
            sc.hist[0][tid] = 0;
        __syncthreads();
#pragma unroll 1
        for (int pass = 0; pass < 4; ++pass) {
            const int shift = 24 - 8 * pass;
            uint32_t *hist = sc.hist[pass & 1];
            if (pass == 0) {
                // the leading byte (sign and high exponent bits) is shared by
                // nearly every score of a row: count each distinct digit of
                // the wave once (ballot) instead of one contended atomic per key
                const int lane = tid & 63;
#pragma unroll
                for (int m = 0; m < KPT; ++m) {
                    const uint32_t dg = key[m] >> 24;
                    bool pending = (cand >> m) & 1u;
                    uint64_t act = __builtin_amdgcn_ballot_w64(pending);
                    while (act) {
                        const int leader = __builtin_ctzll(act);
                        const uint32_t dl = (uint32_t)__builtin_amdgcn_readlane((int)dg, leader);
                        const bool same = pending && dg == dl;
                        const uint64_t grp = __builtin_amdgcn_ballot_w64(same);
                        if (lane == leader)
                            atomicAdd(&hist[dl], (uint32_t)__builtin_popcountll(grp));
                        pending = pending && !same;
                        act &= ~grp;
                    }
                }
            } else {
#pragma unroll
                for (int m = 0; m < KPT; ++m)
                    if (((cand >> m) & 1u) && (key[m] & mask) == prefix)
                        atomicAdd(&hist[(key[m] >> shift) & 255u], 1u);
            }
            if (tid < 256)
                sc.hist[(pass + 1) & 1][tid] = 0;  // last read by the previous pass's pick
            __syncthreads();
            if (tid < 64)
                pick_digit(hist, remaining, sc);
            __syncthreads();
            prefix |= sc.digit << shift;
            mask |= 255u << shift;
            remaining = sc.remaining;
            n_tau = sc.n_tau;  // after the last pass: the keys equal to tau
        }
    }
    const uint32_t tau = prefix;
    uint64_t take = 0;
    if (need > 0 && n_tau > remaining) {
        // exact ties at the threshold: the lowest ids among them are taken
        uint32_t n_eq = 0;
#pragma unroll
        for (int m = 0; m < KPT; ++m)
            n_eq += (((cand >> m) & 1u) && key[m] == tau) ? 1u : 0u;
        uint32_t tot;
        uint32_t eq_rank = wg_exclusive_scan<THREADS, uint32_t>(n_eq, sc.wsum, tot);
#pragma unroll
        for (int m = 0; m < KPT; ++m) {
            const bool c = (cand >> m) & 1u;
            bool s = ((forced >> m) & 1u) || (c && key[m] > tau);
            if (c && key[m] == tau) {
                s = eq_rank < remaining;
                ++eq_rank;
            }
            take |= (uint64_t)s << m;
        }
    } else {
#pragma unroll
        for (int m = 0; m < KPT; ++m) {
            const bool c = (cand >> m) & 1u;
            const bool s = ((forced >> m) & 1u) || (need > 0 && c && key[m] >= tau);
            take |= (uint64_t)s << m;
        }
    }
    uint32_t tot;
    uint32_t pos = wg_exclusive_scan<THREADS, uint32_t>((uint32_t)__builtin_popcountll(take), sc.wsum, tot);
#pragma unroll
    for (int m = 0; m < KPT; ++m)
        if (((take >> m) & 1u) && pos < (uint32_t)k)
            out[pos++] = tid * KPT + m;
    tot = min(tot, (uint32_t)k);
    for (int i = (int)tot + tid; i < k; i += THREADS)
        out[i] = -1;
    __syncthreads();
    return (int)tot;
}

// ------------------------------------------------------------ working set
struct CacheScratch {
    int32_t slot_of[kMaxK];  // slot of S[i]
    uint8_t hit[kMaxK];
    int32_t miss_i[kMaxK];   // S index of miss m
    uint64_t key[kMaxCapacity];  // LRU key of a candidate slot, ~0 otherwise
    int wsum[16];
};

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

// The row's slot table and stamps, read into registers by thread t for the
// slots t, t + THREADS, ...  (issued early so the loads overlap other work).
template <int THREADS> struct SlotRegs {
    static constexpr int SPT = (kMaxCapacity + THREADS - 1) / THREADS;
    int32_t blk[SPT];
    uint32_t stamp[SPT];
};

template <int THREADS>
__device__ __forceinline__ void load_slots(SlotRegs<THREADS> &r, int C, const int32_t *__restrict__ sb,
                                           const uint32_t *__restrict__ ss) {
#pragma unroll
    for (int u = 0; u < SlotRegs<THREADS>::SPT; ++u) {
        const int s = threadIdx.x + u * THREADS;
        r.blk[u] = s < C ? sb[s] : -1;
        r.stamp[u] = s < C ? ss[s] : 0u;
    }
}

// Plans one step of the row's working set for the selection S[0, nn) (in
// LDS, ascending): hit detection, compacted misses (ascending), victims
// (empty slots by index, then (stamp, block) ascending among the slots not
// selected) and the miss -> victim assignment, all in cs.  The slot table
// comes in registers from load_slots.  Returns the number of misses, or -1
// (nothing planned) if the selection or the table is invalid.  Writes no
// global memory.  THREADS >= 256.
template <int THREADS>
__device__ int cache_plan_row(const int32_t *S, int nn, int C, int NB, const SlotRegs<THREADS> &r, CacheScratch &cs,
                              int &bad_out) {
    const int tid = threadIdx.x;
    constexpr int SPT = SlotRegs<THREADS>::SPT;
    for (int i = tid; i < nn; i += THREADS)
        cs.slot_of[i] = -1;
    __syncthreads();
    // validation and hits in one round: the selection must be ascending and
    // in range and the table's ids in [-1, NB); each occupied slot looks its
    // block up in the selection (a binary search that ends whatever S holds)
    // and claims the entry, so a block held by two slots is caught too.  If
    // anything is wrong the claims are discarded with the whole plan.
    int bad = 0;
    for (int i = tid; i < nn; i += THREADS) {
        const int32_t v = S[i];
        if (v < 0 || v >= NB || (i > 0 && v <= S[i - 1]))
            bad = 1;
    }
    // the same pass also stores each slot's LRU key: ~0 for a selected
    // (taken) slot, else empty slots first by index, then (stamp, block)
#pragma unroll
    for (int u = 0; u < SPT; ++u) {
        const int s = tid + u * THREADS;
        if (s < C) {
            const int32_t blk = r.blk[u];
            if (blk < -1 || blk >= NB)
                bad = 1;
            const int i = blk >= 0 ? find_sorted(S, nn, blk) : -1;
            if (i >= 0 && atomicCAS(&cs.slot_of[i], -1, s) != -1)
                bad = 1;
            cs.key[s] = i >= 0 ? ~0ull
                               : (blk < 0 ? (uint64_t)s
                                          : ((1ull << 63) | ((uint64_t)r.stamp[u] << 31) | (uint64_t)blk));
        }
    }
    if (__syncthreads_or(bad)) {
        bad_out = 1;
        return -1;
    }
    // misses in ascending S order: thread t owns S indices [t*per, t*per+per)
    const int per = (nn + THREADS - 1) / THREADS;
    int cnt = 0;
    for (int u = 0; u < per; ++u) {
        const int i = tid * per + u;
        if (i < nn) {
            const bool h = cs.slot_of[i] >= 0;
            cs.hit[i] = h ? 1 : 0;
            cnt += h ? 0 : 1;
        }
    }
    int nm;
    int pos = wg_exclusive_scan<THREADS, int>(cnt, cs.wsum, nm);
    for (int u = 0; u < per; ++u) {
        const int i = tid * per + u;
        if (i < nn && !cs.hit[i])
            cs.miss_i[pos++] = i;
    }
    // victims: candidate rank r < #misses takes miss r (keys of a valid table
    // are distinct; the slot index breaks ties of a corrupt one).  Q lanes
    // share a candidate, each counting over every Q-th slot (the Q lanes
    // then read Q neighbouring keys: different LDS banks), so the loads of
    // one thread stay few and independent.  (The keys were written before
    // the barrier of the miss scan.)
    if (nm > 0) {
        constexpr int Q = THREADS >= 1024 ? 8 : (THREADS >= 512 ? 4 : 1);
        for (int base = 0; base < C * Q; base += THREADS) {
            const int t = base + tid;
            const int s = t / Q, part = t % Q;
            const bool on = s < C;
            const uint64_t key = on ? cs.key[s] : ~0ull;
            int rank = 0;
            if (on && key != ~0ull) {
#pragma unroll 8
                for (int o = part; o < C; o += Q) {
                    const uint64_t ok = cs.key[o];
                    rank += (ok < key || (ok == key && o < s)) ? 1 : 0;
                }
            }
            if constexpr (Q >= 2)
                rank += __builtin_amdgcn_update_dpp(0, rank, DPP_QUAD_XOR1, 0xf, 0xf, false);
            if constexpr (Q >= 4)
                rank += __builtin_amdgcn_update_dpp(0, rank, DPP_QUAD_XOR2, 0xf, 0xf, false);
            if constexpr (Q >= 8)
                rank += __builtin_amdgcn_update_dpp(0, rank, DPP_ROW_HALF_MIRROR, 0xf, 0xf, false);
            if (on && part == 0 && key != ~0ull && rank < nm)
                cs.slot_of[cs.miss_i[rank]] = s;
        }
    }
    __syncthreads();
    bad_out = 0;
    return nm;
}

// Writes the step's lists (sel_slot, sel_hit, miss_block, miss_slot for all
// k entries, -1 / 0 padded) and miss_count for one row.
template <int THREADS>
__device__ __forceinline__ void write_lists(const int32_t *S, int nn, int nm, int k, const CacheScratch &cs,
                                            int32_t *o_slot, uint8_t *o_hit, int32_t *o_mb, int32_t *o_ms,
                                            int32_t *o_count) {
    for (int i = threadIdx.x; i < k; i += THREADS) {
        const bool in = i < nn;
        o_slot[i] = in ? cs.slot_of[i] : -1;
        o_hit[i] = in ? cs.hit[i] : 0;
        const bool mi = i < nm;
        const int si = mi ? cs.miss_i[i] : 0;
        o_mb[i] = mi ? S[si] : -1;
        o_ms[i] = mi ? cs.slot_of[si] : -1;
    }
    if (threadIdx.x == 0)
        *o_count = nm;
}

}  // namespace skv
