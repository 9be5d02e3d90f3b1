// Row-level device routines shared by the standalone stage kernels and the
// fused select -> update -> attend kernel, so that both give bit-identical
// results.  A "row" is one (sequence, kv-head) pair; each routine is called
// by every thread of one workgroup (they contain barriers).
#pragma once

#include "skv_device.h"
#include "skv_launch.h"

namespace skv {

// ------------------------------------------------------------ scans
// Exclusive prefix sum of v over the workgroup in thread order, and the
// total.  publish(pos, total) runs between the scan's two barriers, so what
// it writes to LDS is visible to every thread once the scan returns.  The
// barriers order LDS only (global writes made in publish are not ordered).
template <int THREADS, typename T, typename F>
__device__ __forceinline__ T wg_exclusive_scan_publish(T v, T *wsum, T &total, F &&publish) {
    constexpr int WAVES = THREADS / 64;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    (void)lane;
    const T x = (T)wave_incl_scan((uint32_t)v);
    if (lane == 63)
        wsum[wave] = x;
    lds_barrier();
    T base = 0, tot = 0;
#pragma unroll
    for (int w = 0; w < WAVES; ++w) {
        const T s = wsum[w];
        base += (w < wave) ? s : T(0);
        tot += s;
    }
    const T pos = base + x - v;
    publish(pos, tot);
    lds_barrier();
    total = tot;
    return pos;
}

template <int THREADS, typename T>
__device__ __forceinline__ T wg_exclusive_scan(T v, T *wsum, T &total) {
    return wg_exclusive_scan_publish<THREADS, T>(v, wsum, total, [](T, T) {});
}

// Sum of v over the workgroup (every thread gets it).
template <int THREADS> __device__ __forceinline__ uint32_t wg_reduce_sum(uint32_t v, uint32_t *wsum) {
    uint32_t tot;
    (void)wg_exclusive_scan<THREADS, uint32_t>(v, wsum, tot);
    return tot;
}

// ------------------------------------------------------------ top-k
__device__ __forceinline__ uint32_t order_key(float f) {
    uint32_t u = __float_as_uint(f + 0.0f);  // -0 -> +0 so equal floats give equal keys
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

struct TopkScratch {
    uint32_t hist[2][256];  // passes alternate buffers, so clearing needs no barrier of its own
    uint32_t wsum[16];
    uint32_t wlo[16], whi[16];  // per-wave key range
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

// Radix select: the key of the `need`-th largest of the keys flagged in
// `cand` (KPT per thread; need >= 1 and at most the number of flagged keys).
// Up to four 8-bit passes over an LDS histogram, on the keys minus the
// smallest flagged key; each pass needs two barriers (the histogram buffers
// alternate, so clearing the next one needs none).  Returns the key;
// `remaining` = how many keys equal to it are admitted, `n_tau` = how many
// flagged keys equal it.  The passes stop early once the bin holding the
// need-th key is admitted whole (its count equals the rank still needed):
// the returned key is then the smallest one with the decided leading bits,
// every flagged key at or above it is admitted, and remaining == n_tau
// (no tie to break), so the admitted set is the one the full passes give.
template <int THREADS, int KPT>
__device__ __forceinline__ uint32_t radix_select(const uint32_t (&key)[KPT], uint64_t cand, uint32_t need,
                                                 TopkScratch &sc, uint32_t &remaining_out, uint32_t &n_tau_out) {
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    // the flagged keys' range [lo, hi]: the passes take the bits of key - lo
    // from the highest one in which the keys differ, so even the first pass
    // spreads them over the bins (the leading bits of raw keys are shared by
    // most scores of a row, and colliding LDS atomics serialise)
    uint32_t lo = 0xffffffffu, hi = 0;
#pragma unroll
    for (int m = 0; m < KPT; ++m)
        if ((cand >> m) & 1u) {
            lo = min(lo, key[m]);
            hi = max(hi, key[m]);
        }
    lo = wave_min_u32(lo);
    hi = wave_max_u32(hi);
    if (lane == 0) {
        sc.wlo[wave] = lo;
        sc.whi[wave] = hi;
    }
    if (tid < 256)
        sc.hist[0][tid] = 0;
    lds_barrier();
#pragma unroll
    for (int w = 0; w < THREADS / 64; ++w) {
        lo = min(lo, sc.wlo[w]);
        hi = max(hi, sc.whi[w]);
    }
    const int top = hi > lo ? 32 - __builtin_clz(hi - lo) : 1;  // significant bits of the range
    const int passes = (top + 7) / 8;
    uint32_t prefix = 0, mask = 0;
    uint32_t remaining = need, n_tau = 0;
#pragma unroll 1
    for (int pass = 0; pass < passes; ++pass) {
        const int shift = max(top - 8 * (pass + 1), 0);
        const uint32_t dmask = (1u << (top - 8 * pass - shift)) - 1u;
        uint32_t *hist = sc.hist[pass & 1];
#pragma unroll
        for (int m = 0; m < KPT; ++m) {
            const uint32_t kr = key[m] - lo;
            if (((cand >> m) & 1u) && (kr & mask) == prefix)
                atomicAdd(&hist[(kr >> shift) & dmask], 1u);
        }
        if (tid < 256)
            sc.hist[(pass + 1) & 1][tid] = 0;  // last read by the previous pass's pick
        lds_barrier();
        if (tid < 64)
            pick_digit(hist, remaining, sc);
        lds_barrier();
        prefix |= sc.digit << shift;
        mask |= dmask << shift;
        remaining = sc.remaining;
        n_tau = sc.n_tau;  // after the last pass: the keys equal to tau
        if (n_tau == remaining)  // uniform (read from LDS after the barrier)
            break;
    }
    remaining_out = remaining;
    n_tau_out = n_tau;
    return prefix + lo;
}

// Per-row selection under the budget (sink + recent blocks forced, the rest
// by (score desc, id asc)) as bits: thread t owns ids [t*KPT, t*KPT+KPT) and
// bit m of the result admits id t*KPT + m.  Up to four 8-bit radix passes
// over order-preserving keys find the key of the last admitted block (ties
// at the threshold go to the lowest ids).  A row with at most k valid blocks
// takes all of them without reading its scores.  Contains barriers.
template <int THREADS, int KPT>
__device__ __forceinline__ uint64_t topk_take(const float *__restrict__ srow, int len, int NB, int k, int sink, int recent,
                              TopkScratch &sc) {
    const int tid = threadIdx.x;
    const int nvalid = min(nb_of(len), NB);
    if (nvalid <= k) {
        uint64_t all = 0;
#pragma unroll
        for (int m = 0; m < KPT; ++m)
            all |= (uint64_t)(tid * KPT + m < nvalid) << m;
        return all;
    }
    const int fs = sink > 0 ? min(nb_of(min(sink, len)), nvalid) : 0;
    const int fr = recent > 0 ? max(0, len - recent) / 16 : nvalid;
    const int n_forced = fs + (nvalid - fr) - max(0, fs - fr);
    const int need = k - n_forced;

    uint32_t key[KPT];
    uint64_t cand = 0, forced = 0;
    const int base = tid * KPT;
    auto classify = [&](int m, float v) {
        const int i = base + m;
        key[m] = 0;
        if (i < nvalid) {
            if (i < fs || i >= fr) {
                forced |= 1ull << m;
            } else {
                cand |= 1ull << m;
                key[m] = order_key(v);
            }
        }
    };
    if constexpr ((KPT == 4 || KPT >= 16) && KPT % 4 == 0) {
        // 16-byte loads: a quarter of the load instructions and cache lines
        // touched (measured: 1.4% on the whole 32K step at 4 keys per
        // thread; at 8 the vector form spills in the fused kernel).  With a
        // 16-byte aligned row of NB % 4 == 0 blocks (uniform) the loads are
        // unconditional, the index clamped into the row and ids past the
        // valid length masked afterwards, so all of a thread's loads are in
        // flight at once (a branch around each one makes the compiler wait
        // for it before the next).
        const bool vec = ((reinterpret_cast<uintptr_t>(srow) & 15u) == 0) && (NB & 3) == 0;
        if (vec) {
            float4 f[KPT / 4];
#pragma unroll
            for (int u = 0; u < KPT / 4; ++u)
                f[u] = *reinterpret_cast<const float4 *>(srow + min(base + 4 * u, NB - 4));
#pragma unroll
            for (int u = 0; u < KPT / 4; ++u) {
                classify(4 * u, f[u].x);
                classify(4 * u + 1, f[u].y);
                classify(4 * u + 2, f[u].z);
                classify(4 * u + 3, f[u].w);
            }
        } else {
#pragma unroll
            for (int u = 0; u < KPT / 4; ++u) {
                const int i = base + 4 * u;
                classify(4 * u, i < nvalid ? srow[i] : 0.0f);
                classify(4 * u + 1, i + 1 < nvalid ? srow[i + 1] : 0.0f);
                classify(4 * u + 2, i + 2 < nvalid ? srow[i + 2] : 0.0f);
                classify(4 * u + 3, i + 3 < nvalid ? srow[i + 3] : 0.0f);
            }
        }
    } else {
#pragma unroll
        for (int m = 0; m < KPT; ++m)
            classify(m, base + m < nvalid ? srow[base + m] : 0.0f);
    }
    uint32_t remaining = 0, n_tau = 0;
    const uint32_t tau = need > 0 ? radix_select<THREADS, KPT>(key, cand, (uint32_t)need, sc, remaining, n_tau) : 0u;
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
    return take;
}

// Writes the ascending ids of the admitted bits to out[0, count) and -1 to
// out[count, k), count = min(admitted, k); one prefix sum over the threads.
// publish(pos, bits) also runs between the sum's barriers (pos = the
// thread's first output index), so all of it is visible on return.
template <int THREADS, int KPT, typename F>
__device__ __forceinline__ int topk_emit(uint64_t take, int k, int32_t *out, uint32_t *wsum, F &&publish) {
    const int tid = threadIdx.x;
    uint32_t tot;
    (void)wg_exclusive_scan_publish<THREADS, uint32_t>(
        (uint32_t)__builtin_popcountll(take), wsum, tot, [&](uint32_t pos, uint32_t total) {
            publish(pos, take);
#pragma unroll
            for (int m = 0; m < KPT; ++m)
                if (((take >> m) & 1u) && pos < (uint32_t)k)
                    out[pos++] = tid * KPT + m;
            for (int i = (int)min(total, (uint32_t)k) + tid; i < k; i += THREADS)
                out[i] = -1;
        });
    return (int)min(tot, (uint32_t)k);
}

// topk_take + topk_emit: the row's selection, ascending, in out[0, k).
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
    const uint64_t take = topk_take<THREADS, KPT>(srow, len, NB, k, sink, recent, sc);
    return topk_emit<THREADS, KPT>(take, k, out, sc.wsum, [](uint32_t, uint64_t) {});
}

// ------------------------------------------------------------ long rows
// Top-k for long rows (up to 65536 blocks with 1024 threads); same result as
// topk_row, without holding the row in registers:
//  1. a lower bound of the threshold: the need-th largest of the per-thread
//     maxima, since at least `need` keys reach it.  One more pass over the
//     row puts the keys that reach it (typically not many more than need)
//     with their ids into LDS, and a
//     radix select over those gives the threshold key, how many keys equal
//     it and how many of those are admitted.  If more than kLongRowCand keys
//     reach the bound (many equal scores) the radix passes stream the row.
//  2. the choice goes into a bitmap of the row: forced ids and keys above the
//     threshold; keys equal to it go to a second bitmap whose prefix
//     popcounts rank them by id (the lowest ids are admitted);
//  3. one prefix sum over the bitmap words emits the ids in ascending order.
constexpr int kLongRowCand = 4096;

struct TopkLongScratch {
    TopkScratch sc;
    uint32_t n_cand;
    uint32_t cand_key[kLongRowCand];
    int32_t cand_id[kLongRowCand];
    uint32_t bits[kMaxTopkBlocks / 32];
    uint32_t eq[kMaxTopkBlocks / 32];
};

// Adds `digit` to hist for every lane with `on` set, one atomic per distinct
// digit of the wave (lanes must be converged).
__device__ __forceinline__ void wave_hist_add(uint32_t *hist, uint32_t digit, bool on) {
    const int lane = threadIdx.x & 63;
    uint64_t act = __builtin_amdgcn_ballot_w64(on);
    while (act) {
        const int leader = __builtin_ctzll(act);
        const uint32_t dl = (uint32_t)__builtin_amdgcn_readlane((int)digit, leader);
        const bool same = on && digit == dl;
        const uint64_t grp = __builtin_amdgcn_ballot_w64(same);
        if (lane == leader)
            atomicAdd(&hist[dl], (uint32_t)__builtin_popcountll(grp));
        on = on && !same;
        act &= ~grp;
    }
}

template <int THREADS>
__device__ int topk_long_row(const float *__restrict__ srow, int len, int NB, int k, int sink, int recent,
                             int32_t *out, TopkLongScratch &ls) {
    static_assert(THREADS * 4 >= kLongRowCand && THREADS * 2 * 32 >= kMaxTopkBlocks, "coverage");
    constexpr int BATCH = 8;
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
    const int nwords = (nvalid + 31) >> 5;
    for (int w = tid; w < nwords; w += THREADS) {
        ls.bits[w] = 0;
        ls.eq[w] = 0;
    }
    // f(id, key, is_candidate) for this thread's ids, every lane of a wave
    // calling f together (keys of non-candidates are 0).  Thread t reads the
    // 4-id groups t, t + THREADS, ... with BATCH groups in flight: 16-byte
    // loads when the row is 16-byte aligned and NB a multiple of 4, else
    // single floats.  The 16-byte loads are unconditional (group index
    // clamped into the row, ids past the valid length masked afterwards):
    // with each load in a branch of its own the compiler waits for every
    // one before issuing the next.
    const bool vec = (reinterpret_cast<uintptr_t>(srow) & 15) == 0 && (NB & 3) == 0;  // uniform
    const int gmax = (NB >> 2) - 1;
    auto stream = [&](auto &&f) {
        const int ngroups = (nvalid + 3) >> 2;
        for (int g0 = tid; g0 < ngroups; g0 += BATCH * THREADS) {
            float v[BATCH][4];
            if (vec) {
                u32x4 w[BATCH];
#pragma unroll
                for (int u = 0; u < BATCH; ++u)
                    w[u] = load16(srow + 4 * min(g0 + u * THREADS, gmax));
#pragma unroll
                for (int u = 0; u < BATCH; ++u)
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        v[u][e] = 4 * (g0 + u * THREADS) + e < nvalid ? __uint_as_float(w[u][e]) : 0.0f;
            } else {
#pragma unroll
                for (int u = 0; u < BATCH; ++u) {
                    const int g = g0 + u * THREADS;
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        v[u][e] = 4 * g + e < nvalid ? srow[4 * g + e] : 0.0f;
                }
            }
#pragma unroll
            for (int u = 0; u < BATCH; ++u) {
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int i = 4 * (g0 + u * THREADS) + e;
                    const bool c = i < nvalid && i >= fs && i < fr;
                    f(i, c ? order_key(v[u][e]) : 0u, c);
                }
            }
        }
    };
    __syncthreads();  // bitmaps cleared
    uint32_t remaining = 0, n_tau = 0, tau = 0;
    if (need > 0) {
        // 1a. a lower bound of the threshold: the need-th largest of the
        //     per-thread maxima (at least `need` keys reach it).  (A sampled
        //     subset of the row reads less but its radix select, over a few
        //     thousand keys, measured slower than this one over 1024.)
        uint32_t bound = 1u;
        {
            uint32_t tmax[1] = {0u}, r1, n1;
            stream([&](int, uint32_t kk, bool) { tmax[0] = max(tmax[0], kk); });
            if (__syncthreads_count(tmax[0] != 0u) >= need)
                bound = radix_select<THREADS, 1>(tmax, tmax[0] != 0u ? 1ull : 0ull, (uint32_t)need, ls.sc, r1, n1);
        }
        // 1b. the keys that reach the bound, with their ids, into LDS (in
        //     any order: neither the select nor the marking needs one)
        if (tid == 0)
            ls.n_cand = 0;
        __syncthreads();
        stream([&](int i, uint32_t kk, bool c) {
            if (c && kk >= bound) {
                const uint32_t p = atomicAdd(&ls.n_cand, 1u);
                if (p < (uint32_t)kLongRowCand) {
                    ls.cand_key[p] = kk;
                    ls.cand_id[p] = i;
                }
            }
        });
        __syncthreads();
        const uint32_t total = ls.n_cand;
        if (total <= (uint32_t)kLongRowCand) {  // uniform
            uint32_t ck[4];
            uint64_t cm = 0;
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const uint32_t p = (uint32_t)(tid + THREADS * u);
                ck[u] = p < total ? ls.cand_key[p] : 0u;
                cm |= (uint64_t)(p < total) << u;
            }
            tau = radix_select<THREADS, 4>(ck, cm, (uint32_t)need, ls.sc, remaining, n_tau);
            // 2. mark from the candidate list (every key >= tau is in it)
            const bool all_eq = n_tau == remaining;
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const uint32_t p = (uint32_t)(tid + THREADS * u);
                if (p < total && ck[u] >= tau) {
                    const int i = ls.cand_id[p];
                    if (ck[u] > tau || all_eq)
                        atomicOr(&ls.bits[i >> 5], 1u << (i & 31));
                    else
                        atomicOr(&ls.eq[i >> 5], 1u << (i & 31));
                }
            }
        } else {
            // many keys reach the bound (many equal scores): radix passes that
            // stream the row (wave-aggregated histogram adds), then marking
            uint32_t prefix = 0, mask = 0;
            remaining = (uint32_t)need;
            if (tid < 256)
                ls.sc.hist[0][tid] = 0;
            __syncthreads();
            for (int pass = 0; pass < 4; ++pass) {
                const int shift = 24 - 8 * pass;
                uint32_t *hist = ls.sc.hist[pass & 1];
                stream([&](int, uint32_t kk, bool c) {
                    wave_hist_add(hist, (kk >> shift) & 255u, c && (kk & mask) == prefix);
                });
                if (tid < 256)
                    ls.sc.hist[(pass + 1) & 1][tid] = 0;
                __syncthreads();
                if (tid < 64)
                    pick_digit(hist, remaining, ls.sc);
                __syncthreads();
                prefix |= ls.sc.digit << shift;
                mask |= 255u << shift;
                remaining = ls.sc.remaining;
                n_tau = ls.sc.n_tau;
            }
            tau = prefix;
            const bool all_eq = n_tau == remaining;
            stream([&](int i, uint32_t kk, bool c) {
                if (c && kk >= tau) {
                    if (kk > tau || all_eq)
                        atomicOr(&ls.bits[i >> 5], 1u << (i & 31));
                    else
                        atomicOr(&ls.eq[i >> 5], 1u << (i & 31));
                }
            });
        }
    }
    // forced blocks: the id ranges [0, fs) and [fr, nvalid)
    for (int i = tid; i < fs; i += THREADS)
        atomicOr(&ls.bits[i >> 5], 1u << (i & 31));
    for (int i = fr + tid; i < nvalid; i += THREADS)
        atomicOr(&ls.bits[i >> 5], 1u << (i & 31));
    __syncthreads();
    // thread t owns words 2t, 2t + 1
    const int w0i = 2 * tid, w1i = 2 * tid + 1;
    uint32_t w0 = w0i < nwords ? ls.bits[w0i] : 0u, w1 = w1i < nwords ? ls.bits[w1i] : 0u;
    if (need > 0 && n_tau > remaining) {  // uniform: exact ties, the lowest ids among them
        const uint32_t e0 = w0i < nwords ? ls.eq[w0i] : 0u, e1 = w1i < nwords ? ls.eq[w1i] : 0u;
        uint32_t n_eq;
        const uint32_t r0 = wg_exclusive_scan<THREADS, uint32_t>(
            (uint32_t)(__builtin_popcount(e0) + __builtin_popcount(e1)), ls.sc.wsum, n_eq);
        const uint32_t r1 = r0 + (uint32_t)__builtin_popcount(e0);
        auto keep = [&](uint32_t e, uint32_t r) -> uint32_t {  // the first remaining - r set bits
            uint32_t kept = 0;
            while (e && r < remaining) {
                kept |= e & (0u - e);
                e &= e - 1;
                ++r;
            }
            return kept;
        };
        w0 |= keep(e0, r0);
        w1 |= keep(e1, r1);
    }
    uint32_t n_out;
    uint32_t o = wg_exclusive_scan<THREADS, uint32_t>((uint32_t)(__builtin_popcount(w0) + __builtin_popcount(w1)),
                                                      ls.sc.wsum, n_out);
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        uint32_t w = h ? w1 : w0;
        while (w) {
            const int bit = __builtin_ctz(w);
            w &= w - 1;
            if (o < (uint32_t)k)
                out[o] = (2 * tid + h) * 32 + bit;
            ++o;
        }
    }
    n_out = min(n_out, (uint32_t)k);
    for (int i = (int)n_out + tid; i < k; i += THREADS)
        out[i] = -1;
    __syncthreads();
    return (int)n_out;
}

// ------------------------------------------------------------ working set
// The slot table maps each resident block to one slot, so a table that holds
// one block in two slots is corrupt whether or not the step selects that
// block.  A selected block held twice is caught by the claims on its
// selection entry; the others go through a set of block ids in LDS (open
// addressing, linear probing) sized to a power of two of at least 2C
// entries: at most half full, so every probe sequence meets an empty entry.
constexpr int kDupSet = 2 * kMaxCapacity;

__device__ __forceinline__ int dup_set_bits(int C) {  // C >= 1
    return max(6, 32 - __builtin_clz((unsigned)(2 * C - 1)));
}

// Adds blk (>= 0) to the set; true if it was there already.
__device__ __forceinline__ bool dup_set_add(int32_t *set, int bits, int32_t blk) {
    const uint32_t mask = (1u << bits) - 1u;
    uint32_t p = ((uint32_t)blk * 0x9E3779B1u) >> (32 - bits);
    for (uint32_t n = 0; n <= mask; ++n) {
        const int32_t old = atomicCAS(&set[p], -1, blk);
        if (old == -1)
            return false;
        if (old == blk)
            return true;
        p = (p + 1u) & mask;
    }
    return true;  // not reached (the set is at most half full)
}

struct CacheScratch {
    int32_t slot_of[kMaxK];  // slot of S[i]
    uint8_t hit[kMaxK];
    int32_t miss_i[kMaxK];   // S index of miss m
    uint64_t key[kMaxCapacity];  // LRU key of a candidate slot, ~0 otherwise
    int32_t dup[kDupSet];    // block ids of the unselected occupied slots
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

// The loads are unconditional (slot index clamped to C - 1, C >= 1) and the
// out-of-range lanes are masked afterwards: with the loads inside a branch
// the compiler moves the key arithmetic next to them and waits for the data
// right there, before the top-k's own loads are even issued.
template <int THREADS>
__device__ __forceinline__ void load_slots(SlotRegs<THREADS> &r, int C, const int32_t *__restrict__ sb,
                                           const uint32_t *__restrict__ ss) {
#pragma unroll
    for (int u = 0; u < SlotRegs<THREADS>::SPT; ++u) {
        const int s = threadIdx.x + u * THREADS;
        const int sc = min(s, C - 1);
        const int32_t b = sb[sc];
        const uint32_t t = ss[sc];
        r.blk[u] = s < C ? b : -1;
        r.stamp[u] = s < C ? t : 0u;
    }
}

// Clears the plan's slot column for a selection of up to k entries and the
// duplicate set of a C-slot table.  Call it before a barrier that precedes
// cache_plan_row (a top-k, or the barrier after the selection is staged):
// the plan relies on the cleared entries being visible to every thread and
// has no barrier of its own for it.
template <int THREADS> __device__ __forceinline__ void cache_plan_clear(CacheScratch &cs, int k, int C) {
    for (int i = threadIdx.x; i < k; i += THREADS)
        cs.slot_of[i] = -1;
    const int nd = 1 << dup_set_bits(C);
    for (int i = threadIdx.x; i < nd; i += THREADS)
        cs.dup[i] = -1;
}

// Plans one step of the row's working set for the selection S[0, nn) (in
// LDS, ascending): hit detection, compacted misses (ascending), victims
// (empty slots by index, then (stamp, block) ascending among the slots not
// selected) and the miss -> victim assignment, all in cs.  The slot table
// comes in registers from load_slots; cs.slot_of[0, nn) must have been
// cleared by cache_plan_clear before an earlier barrier.  Returns the number
// of misses, or -1 (nothing planned) if the selection or the table is
// invalid.  Writes no global memory.  THREADS >= 256.
template <int THREADS>
__device__ int cache_plan_row(const int32_t *S, int nn, int C, int NB, const SlotRegs<THREADS> &r, CacheScratch &cs,
                              int &bad_out, const float *__restrict__ importance = nullptr) {
    const int tid = threadIdx.x;
    constexpr int SPT = SlotRegs<THREADS>::SPT;
    // validation and hits in one round: the selection must be ascending and
    // in range and the table's ids in [-1, NB); each occupied slot looks its
    // block up in the selection (a binary search that ends whatever S holds)
    // and claims the entry, so a selected block held by two slots is caught,
    // and an unselected one goes into the duplicate set, which catches the
    // rest.  If anything is wrong the claims are discarded with the plan.
    const int dbits = dup_set_bits(C);
    int bad = 0;
    for (int i = tid; i < nn; i += THREADS) {
        const int32_t v = S[i];
        if (v < 0 || v >= NB || (i > 0 && v <= S[i - 1]))
            bad = 1;
    }
    // the same pass also stores each slot's eviction key: ~0 for a selected
    // (taken) slot, else empty slots first by index, then occupied slots by
    // (stamp, block) for LRU or, with `importance` (the row's scores of this
    // step), by (score, block): the least important block goes first
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
            if (i < 0 && blk >= 0 && dup_set_add(cs.dup, dbits, blk))
                bad = 1;
            const uint32_t order = importance && blk >= 0 && blk < NB ? order_key(importance[blk]) : r.stamp[u];
            cs.key[s] = i >= 0 ? ~0ull
                               : (blk < 0 ? (uint64_t)s
                                          : ((1ull << 63) | ((uint64_t)order << 31) | (uint64_t)blk));
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
    // the compacted miss list is written between the scan's two barriers,
    // so the victim pass below (other threads) reads it complete
    int nm;
    (void)wg_exclusive_scan_publish<THREADS, int>(cnt, cs.wsum, nm, [&](int pos, int) {
        for (int u = 0; u < per; ++u) {
            const int i = tid * per + u;
            if (i < nn && !cs.hit[i])
                cs.miss_i[pos++] = i;
        }
    });
    // victims: candidate rank r < #misses takes miss r (keys of a valid table
    // are distinct; the slot index breaks ties of a corrupt one).  Q lanes
    // share a candidate, each counting over every Q-th slot (the Q lanes
    // then read Q neighbouring keys: different LDS banks), so the loads of
    // one thread stay few and independent.  (The keys were written before
    // the barrier of the validation round.)
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

// The selection and the working-set plan of a row in one pass, for kernels
// that run the top-k themselves (same results as topk_row followed by
// cache_plan_row).  The selection's index of a block is found from the
// bits and output position of the thread that owns it (published by the
// emit), not by a search; the eviction candidates (slots whose block is not
// selected) are gathered into a short list while the slots claim their
// blocks, each is ranked against that list only, in the same round as the
// hit / miss flags, and each miss takes the victim of its rank between the
// barriers of the miss prefix sum.  Five barriers from the admitted bits to
// a complete plan.
template <int THREADS> struct PlanScratch {
    uint32_t pos[THREADS];   // a thread's first index in the selection
    uint32_t take[THREADS];  // its admitted bits
    int32_t victim[kMaxCapacity];  // the slot of eviction rank r
    int32_t cand_slot[kMaxCapacity];  // candidate list (keys in CacheScratch::key), any order
    uint32_t wsum[16];
    int iwsum[16];
    int bad, n_cand;
};

// Clears what select_plan_row expects cleared (call before a barrier that
// precedes it, e.g. before the top-k).
template <int THREADS>
__device__ __forceinline__ void select_plan_clear(CacheScratch &cs, PlanScratch<THREADS> &ps, int k, int C) {
    cache_plan_clear<THREADS>(cs, k, C);
    if (threadIdx.x == 0) {
        ps.bad = 0;
        ps.n_cand = 0;
    }
}

// take: topk_take's bits (KPT <= 32, NB <= THREADS * KPT).  Writes the
// selection to S[0, k) (ascending, -1 padded) and returns its size in nn;
// returns the number of misses, or -1 with bad_out set if the slot table is
// invalid (a block id out of range, or a block in two slots).
// after_claims(nn) runs once the selection is in S and the hits have their
// slots in cs.slot_of (misses still -1); the barriers after it order LDS
// only, so global loads it issues stay in flight through the rest.
template <int THREADS, int KPT, typename F>
__device__ int select_plan_row(uint64_t take, int k, int C, int NB, const SlotRegs<THREADS> &r, int32_t *S,
                               CacheScratch &cs, PlanScratch<THREADS> &ps, int &nn_out, int &bad_out,
                               F &&after_claims) {
    static_assert(KPT <= 32, "take bits are kept as 32-bit words");
    const int tid = threadIdx.x;
    constexpr int SPT = SlotRegs<THREADS>::SPT;
    const int nn = topk_emit<THREADS, KPT>(take, k, S, ps.wsum, [&](uint32_t pos, uint64_t t) {
        ps.pos[tid] = pos;
        ps.take[tid] = (uint32_t)t;
    });
    // claims: an occupied slot whose block is selected takes the block's
    // selection index (a selected block held by two slots is caught by the
    // second claim); every other slot joins the candidate list with its
    // eviction key (as in cache_plan_row: empty slots by index, then
    // (stamp, block)), an occupied one after passing the duplicate set
    const int dbits = dup_set_bits(C);
    int bad = 0;
#pragma unroll
    for (int u = 0; u < SPT; ++u) {
        const int s = tid + u * THREADS;
        if (s < C) {
            const int32_t blk = r.blk[u];
            if (blk < -1 || blk >= NB)
                bad = 1;
            int i = -1;
            if (blk >= 0 && blk < NB && blk / KPT < THREADS) {
                const int c = blk / KPT, m = blk - c * KPT;
                const uint32_t t = ps.take[c];
                const uint32_t p = ps.pos[c] + (uint32_t)__builtin_popcount(t & ((1u << m) - 1u));
                if (((t >> m) & 1u) && p < (uint32_t)nn)
                    i = (int)p;
            }
            if (i >= 0) {
                if (atomicCAS(&cs.slot_of[i], -1, s) != -1)
                    bad = 1;
            } else {
                if (blk >= 0 && dup_set_add(cs.dup, dbits, blk))
                    bad = 1;
                const int c = atomicAdd(&ps.n_cand, 1);
                cs.key[c] = blk < 0 ? (uint64_t)s : ((1ull << 63) | ((uint64_t)r.stamp[u] << 31) | (uint64_t)blk);
                ps.cand_slot[c] = s;
            }
        }
    }
    if (bad)
        ps.bad = 1;
    lds_barrier();
    nn_out = nn;
    if (ps.bad) {  // uniform
        bad_out = 1;
        return -1;
    }
    after_claims(nn);  // the selection and its hits are known here
    // hit flags and miss counts of the selection indices a thread owns ...
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
    // ... and, in the same round, every candidate's eviction rank among the
    // candidates (Q lanes per candidate, each counting over every Q-th list
    // entry; equal keys of a corrupt table rank by slot index); candidates
    // outnumber the misses since C >= k
    {
        constexpr int Q = THREADS >= 1024 ? 8 : (THREADS >= 512 ? 4 : 1);
        const int nc = ps.n_cand;
        for (int base = 0; base < nc * Q; base += THREADS) {
            const int t = base + tid;
            const int c = t / Q, part = t % Q;
            const bool on = c < nc;
            const uint64_t key = on ? cs.key[c] : ~0ull;
            const int s = on ? ps.cand_slot[c] : 0;
            int rank = 0;
            if (on) {
#pragma unroll 4
                for (int o = part; o < nc; o += Q) {
                    const uint64_t ok = cs.key[o];
                    rank += ok < key ? 1 : 0;
                    if (ok == key && o != c)
                        rank += ps.cand_slot[o] < s ? 1 : 0;
                }
            }
            if constexpr (Q >= 2)
                rank += __builtin_amdgcn_update_dpp(0, rank, DPP_QUAD_XOR1, 0xf, 0xf, false);
            if constexpr (Q >= 4)
                rank += __builtin_amdgcn_update_dpp(0, rank, DPP_QUAD_XOR2, 0xf, 0xf, false);
            if constexpr (Q >= 8)
                rank += __builtin_amdgcn_update_dpp(0, rank, DPP_ROW_HALF_MIRROR, 0xf, 0xf, false);
            if (on && part == 0)
                ps.victim[rank] = s;
        }
    }
    // misses in ascending selection order: miss j takes the victim of rank j
    int nm;
    (void)wg_exclusive_scan_publish<THREADS, int>(cnt, ps.iwsum, nm, [&](int pos, int) {
        for (int u = 0; u < per; ++u) {
            const int i = tid * per + u;
            if (i < nn && !cs.hit[i]) {
                cs.miss_i[pos] = i;
                cs.slot_of[i] = ps.victim[pos];
                ++pos;
            }
        }
    });
    bad_out = 0;
    return nm;
}

// The lists of a row refused as invalid: every entry padded (sel_slot -1,
// sel_hit 0, miss_block / miss_slot -1) and miss_count -1, so a later
// attention over them reads nothing.
template <int THREADS>
__device__ __forceinline__ void write_invalid_lists(int k, int32_t *o_slot, uint8_t *o_hit, int32_t *o_mb,
                                                    int32_t *o_ms, int32_t *o_count) {
    for (int i = threadIdx.x; i < k; i += THREADS) {
        o_slot[i] = -1;
        o_hit[i] = 0;
        o_mb[i] = -1;
        o_ms[i] = -1;
    }
    if (threadIdx.x == 0)
        *o_count = -1;
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
