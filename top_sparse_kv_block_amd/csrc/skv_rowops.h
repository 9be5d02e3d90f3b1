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
    uint32_t wbeta[16];         // per-wave lower bound (small budgets)
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
// smallest flagged key (for a small need: minus a lower bound on the
// need-th key, counting only the keys above it); each pass needs two
// barriers (the histogram buffers
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
    constexpr int WAVES = THREADS / 64;
    uint32_t lo = 0xffffffffu, hi = 0;
#pragma unroll
    for (int m = 0; m < KPT; ++m)
        if ((cand >> m) & 1u) {
            lo = min(lo, key[m]);
            hi = max(hi, key[m]);
        }
    // A small budget (at most four keys per wave) also gets a lower bound
    // beta on the need-th largest key, so that the passes count only the
    // few keys at or above it instead of every key of the row (at 8192 keys
    // and one LDS atomic per key the first pass cost more than the rest of
    // the selection).  Each wave takes the m-th largest of its lanes'
    // largest keys, m = ceil(need / waves): its m lanes at or above that
    // value hold at least m keys, so all waves together hold at least need
    // keys at or above the smallest of the waves' values.  A wave with fewer
    // than m lanes holding keys gives 0, which bounds nothing.
    const bool bound = need <= 4u * WAVES;  // uniform
    uint32_t beta = 0;
    if (bound) {
        const int mm = ((int)need + WAVES - 1) / WAVES;
        uint32_t v = hi;
        for (int it = 0; it < mm; ++it) {
            beta = wave_max_u32(v);
            if (lane == __builtin_ctzll(__builtin_amdgcn_ballot_w64(v == beta)))
                v = 0;  // one lane holding the maximum drops out
        }
    }
    lo = wave_min_u32(lo);
    hi = wave_max_u32(hi);
    if (lane == 0) {
        sc.wlo[wave] = lo;
        sc.whi[wave] = hi;
        sc.wbeta[wave] = beta;
    }
    for (int i = tid; i < 256; i += THREADS)
        sc.hist[0][i] = 0;
    lds_barrier();
    beta = 0xffffffffu;
#pragma unroll
    for (int w = 0; w < WAVES; ++w) {
        lo = min(lo, sc.wlo[w]);
        hi = max(hi, sc.whi[w]);
        beta = min(beta, sc.wbeta[w]);
    }
    if (bound && beta > lo) {  // uniform: no key below beta can be admitted
#pragma unroll
        for (int m = 0; m < KPT; ++m)
            if (key[m] < beta)
                cand &= ~(1ull << m);
        lo = beta;
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
        for (int i = tid; i < 256; i += THREADS)
            sc.hist[(pass + 1) & 1][i] = 0;  // last read by the previous pass's pick
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
__device__ __forceinline__ uint64_t select_take(const uint32_t (&key)[KPT], uint64_t cand, uint64_t forced, int need,
                                                TopkScratch &sc);

// A thread's KPT scores of a row (ids [t*KPT, t*KPT+KPT)), loaded without
// reading the row's length: the loads depend only on the row pointer and
// NB, so a kernel can issue them first and let their latency run under its
// other set-up (the length and everything before the top-k).  Ids past the
// valid length are masked when the keys are formed.  (A load under a branch
// on the length waited for the length first, and each scalar load for the
// one before it.)
template <int KPT> struct TopkScores {
    float v[KPT];
};

template <int KPT>
__device__ __forceinline__ void topk_load(const float *__restrict__ srow, int NB, TopkScores<KPT> &L) {
    const int base = threadIdx.x * KPT;
    if constexpr (KPT % 4 == 0) {
        if ((NB & 3) == 0) {  // uniform
            // 16-byte loads (a quarter of the instructions and cache lines
            // touched), the index clamped into the row: a group past the end
            // reads the row's last four scores, which its masked ids ignore.
            // (The empty asm keeps the compiler from merging this form with
            // the scalar one below into scalar loads.)
            asm volatile("" ::: "memory");
            u32x4 w[KPT / 4];
#pragma unroll
            for (int u = 0; u < KPT / 4; ++u)
                __builtin_memcpy(&w[u], srow + min(base + 4 * u, NB - 4), 16);
#pragma unroll
            for (int u = 0; u < KPT / 4; ++u)
#pragma unroll
                for (int x = 0; x < 4; ++x)
                    L.v[4 * u + x] = __uint_as_float(w[u][x]);
            return;
        }
    }
#pragma unroll
    for (int m = 0; m < KPT; ++m)
        L.v[m] = srow[min(base + m, NB - 1)];
}

// Per-row selection under the budget (sink + recent blocks forced, the rest
// by (score desc, id asc)) as bits: thread t owns ids [t*KPT, t*KPT+KPT) and
// bit m of the result admits id t*KPT + m.  Up to four 8-bit radix passes
// over order-preserving keys find the key of the last admitted block (ties
// at the threshold go to the lowest ids).  A row with at most k valid blocks
// takes all of them without looking at its scores.  L: the thread's scores
// from topk_load.  Contains barriers.
template <int THREADS, int KPT>
__device__ __forceinline__ uint64_t topk_take_loaded(const TopkScores<KPT> &L, int len, int NB, int k, int sink,
                                                     int recent, TopkScratch &sc) {
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
#pragma unroll
    for (int m = 0; m < KPT; ++m) {
        const int i = base + m;
        key[m] = 0;
        if (i < nvalid) {
            if (i < fs || i >= fr) {
                forced |= 1ull << m;
            } else {
                cand |= 1ull << m;
                key[m] = order_key(L.v[m]);
            }
        }
    }
    return select_take<THREADS, KPT>(key, cand, forced, need, sc);
}

template <int THREADS, int KPT>
__device__ __forceinline__ uint64_t topk_take(const float *__restrict__ srow, int len, int NB, int k, int sink,
                                              int recent, TopkScratch &sc) {
    TopkScores<KPT> L;
    topk_load<KPT>(srow, NB, L);
    return topk_take_loaded<THREADS, KPT>(L, len, NB, k, sink, recent, sc);
}

// The admitted bits of a thread's KPT keys: every forced key, and the `need`
// largest flagged (`cand`) keys, ties at the threshold going to the lowest
// positions (thread order, then m).  need <= number of flagged keys.
// Contains barriers (every thread of the workgroup calls it).
template <int THREADS, int KPT>
__device__ __forceinline__ uint64_t select_take(const uint32_t (&key)[KPT], uint64_t cand, uint64_t forced, int need,
                                                TopkScratch &sc) {
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

// topk_take_loaded + topk_emit: the row's selection, ascending, in out[0, k).
template <int THREADS, int KPT>
__device__ int topk_row(const TopkScores<KPT> &L, int len, int NB, int k, int sink, int recent, int32_t *out,
                        TopkScratch &sc) {
    const int tid = threadIdx.x;
    const int nvalid = min(nb_of(len), NB);
    if (nvalid <= k) {
        for (int i = tid; i < k; i += THREADS)
            out[i] = i < nvalid ? i : -1;
        __syncthreads();
        return nvalid;
    }
    const uint64_t take = topk_take_loaded<THREADS, KPT>(L, len, NB, k, sink, recent, sc);
    return topk_emit<THREADS, KPT>(take, k, out, sc.wsum, [](uint32_t, uint64_t) {});
}

// ------------------------------------------------------------ long rows
// Rows over kLongRowBlocks blocks are selected in two launches that spread
// a row over many workgroups (one workgroup holding a 65536-block row streams
// it at one CU's rate).  The row's blocks are cut into chunks of
// long_row_chunk() blocks:
//  A. one workgroup per (row, chunk) keeps the chunk's `need` best
//     non-forced blocks (need = k - forced blocks; order (score desc,
//     id asc); all of them if fewer) as (score, id) pairs, ascending by id,
//     in the chunk's kp = long_row_stride(k) entries of the workspace,
//     padded with id -1;
//  B. one workgroup per row takes the `need` best of those candidates
//     (ties to the lower position, which is the lower id) and adds the
//     forced blocks in front (sink) and behind (recent).
// Exact: a block among the row's `need` best is among its chunk's `need`
// best under the same total order; padding never competes.
constexpr int kLongRowBlocks = 16384;
constexpr int kChunkThreads = 256;     // phase A
constexpr int kLongRowThreads = 512;   // phase B
constexpr int kLongRowMaxCand = 32 * kLongRowThreads;  // candidates per row phase B holds in registers

// Entries per chunk in the workspace: k rounded up to a multiple of 4, so
// that every chunk and row starts 16-byte aligned.
__host__ __device__ inline int long_row_stride(int k) { return (k + 3) & ~3; }
// Blocks per phase-A chunk (1024, 2048 or 4096) for a row of NB blocks and
// budget k: the smallest whose candidates (chunks * stride) number at most
// 4096, else the smallest whose candidates fit phase B (4096 always does:
// NB <= 65536, k <= 1024).  Measured on rows of 65536 blocks with k = 128:
// 2048-block chunks (4096 candidates) take 19.4 us for both launches,
// 1024-block chunks (8192 candidates) 20.6 us; one workgroup per row
// selecting from the candidates costs about twice what a chunk does, and
// more so the more candidates it reads.
__host__ __device__ inline int long_row_chunk(int NB, int k) {
    const int kp = long_row_stride(k);
    for (int lim : {4096, kLongRowMaxCand})
        for (int ch = 1024; ch <= 4096; ch *= 2)
            if ((NB + ch - 1) / ch * kp <= lim)
                return ch;
    return 4096;
}
__host__ __device__ inline int long_row_chunks(int NB, int k) {
    const int ch = long_row_chunk(NB, k);
    return (NB + ch - 1) / ch;
}

// The row's forced ranges [0, fs) (sink) and [fr, nvalid) (recent) and the
// number of blocks the budget leaves to the scores.
__device__ __forceinline__ int forced_ranges(int len, int nvalid, int k, int sink, int recent, int &fs, int &fr) {
    fs = sink > 0 ? min(nb_of(min(sink, len)), nvalid) : 0;
    fr = recent > 0 ? max(0, len - recent) / 16 : nvalid;
    const int n_forced = fs + (nvalid - fr) - max(0, fs - fr);
    return k - n_forced;
}

// Phase A's scores for chunk `chunk` of a row: thread t's KPT blocks from
// chunk * THREADS * KPT + t * KPT, read before the row's length is known
// (indexes clamped into the NB allocated scores; what lies past the valid
// part is masked by chunk_candidates).
template <int THREADS, int KPT>
__device__ __forceinline__ void chunk_load(const float *__restrict__ srow, int NB, int chunk, float (&v)[KPT]) {
    static_assert(KPT % 4 == 0, "16-byte loads");
    const int base = chunk * THREADS * KPT + threadIdx.x * KPT;
    if ((reinterpret_cast<uintptr_t>(srow) & 15u) == 0 && (NB & 3) == 0) {  // uniform
        // 16-byte loads; a clamped group lies past NB, so all of its ids are
        // masked
#pragma unroll
        for (int u = 0; u < KPT / 4; ++u) {
            const float4 f = *reinterpret_cast<const float4 *>(srow + min(base + 4 * u, NB - 4));
            v[4 * u] = f.x;
            v[4 * u + 1] = f.y;
            v[4 * u + 2] = f.z;
            v[4 * u + 3] = f.w;
        }
    } else {
#pragma unroll
        for (int m = 0; m < KPT; ++m)
            v[m] = srow[min(base + m, NB - 1)];
    }
}

// Phase A for chunk `chunk` of a row (THREADS threads, KPT keys each, chunk
// = THREADS * KPT blocks; the caller has checked chunk * THREADS * KPT <
// nvalid), over the scores chunk_load read.  ws_score / ws_id: this chunk's
// long_row_stride(k) entries.  Contains barriers.
template <int THREADS, int KPT>
__device__ void chunk_candidates(const float (&v)[KPT], int len, int NB, int k, int sink, int recent, int chunk,
                                 float *__restrict__ ws_score, int32_t *__restrict__ ws_id, TopkScratch &sc) {
    const int tid = threadIdx.x;
    const int nvalid = min(nb_of(len), NB);
    int fs, fr;
    const int need = forced_ranges(len, nvalid, k, sink, recent, fs, fr);
    const int c0 = chunk * THREADS * KPT, c1 = c0 + THREADS * KPT;
    const int base = c0 + tid * KPT;
    uint32_t key[KPT];
    uint64_t cand = 0;
#pragma unroll
    for (int m = 0; m < KPT; ++m) {
        const int i = base + m;
        const bool c = i < nvalid && i >= fs && i < fr;
        key[m] = c ? order_key(v[m]) : 0u;
        cand |= (uint64_t)c << m;
    }
    // candidates in the chunk: all of it when it lies inside [fs, min(fr, nvalid))
    uint32_t ncand = THREADS * KPT;
    if (c0 < fs || c1 > min(fr, nvalid))  // uniform
        (void)wg_exclusive_scan<THREADS, uint32_t>((uint32_t)__builtin_popcountll(cand), sc.wsum, ncand);
    const int q = min(need, (int)ncand);
    const uint64_t take = q == (int)ncand ? cand : select_take<THREADS, KPT>(key, cand, 0ull, q, sc);
    uint32_t tot;
    uint32_t pos = wg_exclusive_scan<THREADS, uint32_t>((uint32_t)__builtin_popcountll(take), sc.wsum, tot);
#pragma unroll
    for (int m = 0; m < KPT; ++m)
        if ((take >> m) & 1u) {
            ws_score[pos] = v[m];
            ws_id[pos] = base + m;
            ++pos;
        }
    const int kp = long_row_stride(k);
    for (int i = (int)tot + tid; i < kp; i += THREADS)
        ws_id[i] = -1;
}

// Phase B's candidates for a row: thread t's KPT entries from t * KPT of the
// row's nc = chunks * stride entries (THREADS * KPT >= nc; nc a multiple of
// 4; both arrays 16-byte aligned), read before the row's length is known
// (indexes clamped into the nc entries; long_row_select masks the entries
// past the chunks the length covers).
template <int KPT>
struct LongCands {
    float v[KPT];
    int32_t id[KPT];
};

template <int KPT>
__device__ __forceinline__ void long_row_load(const float *__restrict__ ws_score, const int32_t *__restrict__ ws_id,
                                              int nc, LongCands<KPT> &c) {
    static_assert(KPT % 4 == 0, "16-byte loads");
#pragma unroll
    for (int u = 0; u < KPT / 4; ++u) {
        const int p = min((int)threadIdx.x * KPT + 4 * u, nc - 4);
        const float4 f = *reinterpret_cast<const float4 *>(ws_score + p);
        const int4 d = *reinterpret_cast<const int4 *>(ws_id + p);
        c.v[4 * u] = f.x;
        c.v[4 * u + 1] = f.y;
        c.v[4 * u + 2] = f.z;
        c.v[4 * u + 3] = f.w;
        c.id[4 * u] = d.x;
        c.id[4 * u + 1] = d.y;
        c.id[4 * u + 2] = d.z;
        c.id[4 * u + 3] = d.w;
    }
}

// Phase B: the row's selection, ascending, into S[0, k) (LDS; -1 padded);
// returns its size.  c: what long_row_load read; ncand: the entries of the
// chunks that hold valid blocks (the rest is not current).  Contains
// barriers; S is complete on return.
template <int THREADS, int KPT>
__device__ int long_row_select(const LongCands<KPT> &c, int ncand, int len, int NB, int k, int sink, int recent,
                               int32_t *S, TopkScratch &sc) {
    const int tid = threadIdx.x;
    const int nvalid = min(nb_of(len), NB);
    if (nvalid <= k) {
        for (int i = tid; i < k; i += THREADS)
            S[i] = i < nvalid ? i : -1;
        __syncthreads();
        return nvalid;
    }
    int fs, fr;
    const int need = forced_ranges(len, nvalid, k, sink, recent, fs, fr);
    // candidates: current entries with an id (padding never competes, even
    // against a -inf score); position order is id order
    const float *v = c.v;
    const int32_t *ids = c.id;
    uint32_t key[KPT];
    uint64_t cand = 0;
#pragma unroll
    for (int m = 0; m < KPT; ++m) {
        const bool c = tid * KPT + m < ncand && ids[m] >= 0;
        key[m] = c ? order_key(v[m]) : 0u;
        cand |= (uint64_t)c << m;
    }
    const uint64_t take = select_take<THREADS, KPT>(key, cand, 0ull, need, sc);
    uint32_t tot;
    uint32_t pos = wg_exclusive_scan<THREADS, uint32_t>((uint32_t)__builtin_popcountll(take), sc.wsum, tot);
#pragma unroll
    for (int m = 0; m < KPT; ++m)
        if ((take >> m) & 1u)
            S[fs + pos++] = ids[m];
    for (int i = tid; i < fs; i += THREADS)
        S[i] = i;
    for (int i = tid; i < nvalid - fr; i += THREADS)
        S[fs + need + i] = fr + i;
    const int n = fs + need + (nvalid - fr);
    for (int i = n + tid; i < k; i += THREADS)
        S[i] = -1;
    __syncthreads();
    return n;
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
    uint64_t key[kMaxCapacity];  // eviction keys: cache_plan_row's candidate list (slot in the low bits);
                                 // select_plan_row's candidate list
    int32_t dup[kDupSet];    // block ids of the unselected occupied slots; then the slot of eviction rank r
    int wsum[16];
    int n_cand;              // cache_plan_row's candidates
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
    if (threadIdx.x == 0)
        cs.n_cand = 0;
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
    const int tid = threadIdx.x, lane = tid & 63;
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
    // the same pass lists the eviction candidates (slots whose block is not
    // selected) with their keys: empty slots first by index, then occupied
    // ones by (stamp, block) for LRU or, with `importance` (the row's scores
    // of this step), by (score, block): the least important block goes
    // first.  Key bits: 1 | order (32) | block (21) | slot (10): the slot
    // leaves the order of a valid table's keys unchanged (they differ in
    // (order, block) already; the host refuses NB > 2^21); one list append
    // per wave
#pragma unroll
    for (int u = 0; u < SPT; ++u) {
        const int s = tid + u * THREADS;
        bool cand = false;
        uint64_t key = 0;
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
            cand = i < 0;
            key = blk < 0 ? (uint64_t)s
                          : ((1ull << 63) | ((uint64_t)order << 31) | ((uint64_t)blk << 10) | (uint64_t)s);
        }
        const uint64_t bal = __builtin_amdgcn_ballot_w64(cand);
        if (bal) {  // uniform over the wave
            const int first = (int)__builtin_ctzll(bal);
            int c0 = 0;
            if (lane == first)
                c0 = atomicAdd(&cs.n_cand, (int)__builtin_popcountll(bal));
            c0 = __builtin_amdgcn_readlane(c0, first);
            if (cand)
                cs.key[c0 + (int)__builtin_popcountll(bal & ((1ull << lane) - 1ull))] = key;
        }
    }
    if (__syncthreads_or(bad)) {
        bad_out = 1;
        return -1;
    }
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
    // entry; the keys are distinct), the slot of rank r going to cs.dup[r]
    // (the duplicate set is done with); candidates outnumber the misses since
    // C >= k
    int32_t *victim = cs.dup;
    {
        constexpr int Q = THREADS >= 1024 ? 8 : (THREADS >= 512 ? 4 : 1);
        const int nc = cs.n_cand;
        for (int base = 0; base < nc * Q; base += THREADS) {
            const int t = base + tid;
            const int c = t / Q, part = t % Q;
            const bool on = c < nc;
            const uint64_t key = on ? cs.key[c] : ~0ull;
            int rank = 0;
            if (on) {
#pragma unroll 4
                for (int o = part; o < nc; o += Q)
                    rank += cs.key[o] < key ? 1 : 0;
            }
            if constexpr (Q >= 2)
                rank += __builtin_amdgcn_update_dpp(0, rank, DPP_QUAD_XOR1, 0xf, 0xf, false);
            if constexpr (Q >= 4)
                rank += __builtin_amdgcn_update_dpp(0, rank, DPP_QUAD_XOR2, 0xf, 0xf, false);
            if constexpr (Q >= 8)
                rank += __builtin_amdgcn_update_dpp(0, rank, DPP_ROW_HALF_MIRROR, 0xf, 0xf, false);
            if (on && part == 0)
                victim[rank] = (int32_t)(key & 1023u);
        }
    }
    // misses in ascending selection order: miss j takes the victim of rank
    // j, between the scan's barriers (so the plan is complete on return)
    int nm;
    (void)wg_exclusive_scan_publish<THREADS, int>(cnt, cs.wsum, nm, [&](int pos, int) {
        for (int u = 0; u < per; ++u) {
            const int i = tid * per + u;
            if (i < nn && !cs.hit[i]) {
                cs.miss_i[pos] = i;
                cs.slot_of[i] = victim[pos];
                ++pos;
            }
        }
    });
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
