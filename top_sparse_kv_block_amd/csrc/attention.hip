// Stage 4: GQA decode attention over the selected blocks, split-K with an
// online-softmax merge, on gfx950; and the fused select -> update -> attend
// kernel that runs stages 2-4 of a row in one launch.
//
// Exact attention over the KV the step kept (OasisKV summary, key module 1)
// read from the working set through the slot table (a block-table
// indirection: KV-Cache 压缩技术的工程原理 §5.2), so the result does not
// depend on which tier the blocks came from (HiSparse promo, insight 1).
//
// attn_body: one workgroup of 8 waves owns a contiguous share of a row's
// selection and each wave takes one block of it at a time, so all of the
// workgroup's K and V loads are in flight at once.  A wave loads the block's
// K and V (16 tokens) with the coalesced 16-byte lane layout of the scoring
// kernel and uses them for all G query heads of the kv group (each byte is
// read once per group).  Logits are kept in base-2 units (scale*log2(e)*q.k);
// the running max is per head and wave-uniform; each lane accumulates its
// own tokens' share of l and of the output, so per block the only
// cross-lane work is the dot-product sums and one max per head.  Waves are
// combined in LDS; with one split the workgroup writes the output directly,
// otherwise (max, sum, unnormalised output) per head go to the workspace.
//
// Fetch on attend (optional): when a source cache is given, a selected block
// that was not resident (hit == 0) is read from the source by block id and
// also written into its pool slot, so a miss costs one read and one write
// and no separate copy pass.
//
// select_attend_kernel: grid (splits, rows).  Every workgroup of a row first
// recomputes the row's top-k and working-set plan in LDS (a few KB of scores
// and slot state: the standalone kernels' radix select, then a plan built
// straight from the top-k's per-thread bits that gives the standalone
// working-set update's result bit for bit), then attends its share, the
// first block of each wave loaded as soon as the plan knows its hits.  Split 0 also writes the selection and
// the step's lists.  The slot table is only read here; merge_commit_kernel
// applies the plan after every workgroup has read the old table (with one
// split per row the kernel applies it itself).  This replaces three
// launches and their global round trips with one: the alternative, handing
// results between workgroups inside one launch, needs a device-scope release
// per workgroup, which on this chip writes back the whole L2 each time.
// Rows over 16384 blocks first run the top-k's chunk launch
// (topk_chunk_kernel); every workgroup of such a row then selects from the
// chunk candidates and plans with the standalone update's routine.
//
// merge_commit_kernel: one workgroup per (row, head) merges the head's
// split partials (weights exp2(m_s - m*) formed once by one wave) and, when
// asked, the row's first one commits the working-set plan (new blocks and
// stamps for the selected slots, the clock advanced by a device atomic).
#include "skv_rowops.h"

namespace skv {

template <int LPT> __device__ __forceinline__ float token_groups_max(float v);
template <> __device__ __forceinline__ float token_groups_max<8>(float v) {
    v = fmaxf(v, dpp<DPP_ROW_ROR8>(v));
    return rows_max(v);
}
template <> __device__ __forceinline__ float token_groups_max<16>(float v) { return rows_max(v); }
template <> __device__ __forceinline__ float token_groups_max<32>(float v) { return xor32_max(v); }

template <int LPT> __device__ __forceinline__ float token_groups_sum(float v);
template <> __device__ __forceinline__ float token_groups_sum<8>(float v) {
    v += dpp<DPP_ROW_ROR8>(v);  // lanes i and i+8 of a row: the other 8-lane group
    return rows_sum(v);
}
template <> __device__ __forceinline__ float token_groups_sum<16>(float v) { return rows_sum(v); }
template <> __device__ __forceinline__ float token_groups_sum<32>(float v) { return xor32_sum(v); }

template <typename E> __device__ __forceinline__ float elem(u32x4 v, int e) {
    if constexpr (E::bytes == 2)
        return (e & 1) ? bf16_hi(v[e >> 1]) : bf16_lo(v[e >> 1]);
    else
        return __uint_as_float(v[e]);
}

constexpr int kAttnWaves = 8;
constexpr int kAttnThreads = 64 * kAttnWaves;
constexpr float kLn2 = 0.69314718055994531f;

template <int D, int GMAX> struct AttnSmem {
    float sm[kAttnWaves][GMAX][D + 2];
    float shM[GMAX], shL[GMAX];
};

struct AttnRow {
    const uint8_t *q;              // q of the group's first head, [G, D]
    uint8_t *pool_k, *pool_v;      // the row's slots, [C, 16, D]
    const uint8_t *src_k, *src_v;  // the row's source [T, D], or NULL
    const int32_t *blk, *slot;
    const uint8_t *hit;
    int C, NB, G, len, i0, i1, splits;
    float scale_log2;
    float *part;  // this workgroup's partials [G, D + 2] (splits > 1)
    float *out;   // the group's outputs [G, D] (splits == 1)
    float *lse;   // [G] or NULL (splits == 1)
};

template <int D, int GMAX> __device__ void combine_waves(const AttnRow &a, AttnSmem<D, GMAX> &S);

// float32 storage: dot products and the value accumulation on the vector
// ALU; every lane owns a 16-byte slice of the block's tokens.
template <typename E, int D, int GMAX, int DEPTH>
__device__ __forceinline__ void attn_body_valu(const AttnRow &a, AttnSmem<D, GMAX> &S) {
    constexpr int LPT = D * E::bytes / 16;
    constexpr int TPL = 64 / LPT;
    constexpr int LPB = 16 / TPL;
    constexpr int EPL = E::EPL;
    constexpr size_t kBlockBytes = (size_t)16 * D * E::bytes;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int sub = lane % LPT, tg = lane / LPT;
    const int G = a.G;

    u32x4 qf[GMAX];
#pragma unroll
    for (int g = 0; g < GMAX; ++g)
        qf[g] = g < G ? load16(a.q + ((size_t)g * D + sub * EPL) * E::bytes) : u32x4{0, 0, 0, 0};

    float m[GMAX], l[GMAX], acc[GMAX][EPL];
#pragma unroll
    for (int g = 0; g < GMAX; ++g) {
        m[g] = -__builtin_inff();
        l[g] = 0.0f;
#pragma unroll
        for (int e = 0; e < EPL; ++e)
            acc[g][e] = 0.0f;
    }

    // one block of the selection: where to read it, whether to fetch it
    auto describe = [&](int i, int &blk, int &s, int &nv, bool &fetch) -> bool {
        if (i >= a.i1)
            return false;
        blk = a.blk[i];
        s = a.slot[i];
        if (blk < 0 || s < 0 || s >= a.C)
            return false;
        fetch = a.src_k != nullptr && blk < a.NB && a.hit[i] == 0;
        nv = min(max(a.len - blk * 16, 0), 16);
        return nv > 0 || fetch;
    };
    const size_t lo = ((size_t)tg * D + sub * EPL) * E::bytes;
    constexpr size_t step = (size_t)TPL * D * E::bytes;
    auto load_block = [&](int blk, int s, bool fetch, u32x4 *kv, u32x4 *vv) {
        const uint8_t *rk = fetch ? a.src_k + (size_t)blk * kBlockBytes : a.pool_k + (size_t)s * kBlockBytes;
        const uint8_t *rv = fetch ? a.src_v + (size_t)blk * kBlockBytes : a.pool_v + (size_t)s * kBlockBytes;
#pragma unroll
        for (int li = 0; li < LPB; ++li)
            kv[li] = fetch ? load_nt(rk + lo + li * step) : load16(rk + lo + li * step);
#pragma unroll
        for (int li = 0; li < LPB; ++li)
            vv[li] = fetch ? load_nt(rv + lo + li * step) : load16(rv + lo + li * step);
    };
    auto attend_block = [&](int s, int nv, bool fetch, const u32x4 *kv, const u32x4 *vv) {
        if (fetch) {
            uint8_t *pk = a.pool_k + (size_t)s * kBlockBytes;
            uint8_t *pv = a.pool_v + (size_t)s * kBlockBytes;
#pragma unroll
            for (int li = 0; li < LPB; ++li) {
                store16(pk + lo + li * step, kv[li]);
                store16(pv + lo + li * step, vv[li]);
            }
        }
        if (nv == 0)
            return;
        float z[LPB][GMAX];
#pragma unroll
        for (int li = 0; li < LPB; ++li) {
#pragma unroll
            for (int g = 0; g < GMAX; ++g)
                z[li][g] = g < G ? group_sum<LPT>(dot_chunk<E>(kv[li], qf[g], 0.0f)) * a.scale_log2
                                 : -__builtin_inff();
        }
        if (nv < 16) {  // partial last block: drop the tokens past the end
#pragma unroll
            for (int li = 0; li < LPB; ++li)
                if (li * TPL + tg >= nv) {
#pragma unroll
                    for (int g = 0; g < GMAX; ++g)
                        z[li][g] = -__builtin_inff();
                }
        }
#pragma unroll
        for (int g = 0; g < GMAX; ++g) {
            if (g >= G)
                continue;
            float bm = z[0][g];
#pragma unroll
            for (int li = 1; li < LPB; ++li)
                bm = fmaxf(bm, z[li][g]);
            bm = token_groups_max<LPT>(bm);
            const float mn = fmaxf(m[g], bm);
            const float alpha = exp2_fast(m[g] - mn);  // m = -inf -> 0
            m[g] = mn;
            l[g] *= alpha;
#pragma unroll
            for (int e = 0; e < EPL; ++e)
                acc[g][e] *= alpha;
#pragma unroll
            for (int li = 0; li < LPB; ++li) {
                const float p = exp2_fast(z[li][g] - mn);
                l[g] += p;
#pragma unroll
                for (int e = 0; e < EPL; ++e)
                    acc[g][e] = __builtin_fmaf(p, elem<E>(vv[li], e), acc[g][e]);
            }
        }
    };

    // The wave's blocks are i0 + wave + 8*j.  DEPTH 1: one at a time.
    // DEPTH 2: rolling, the next block's K and V loads are in flight while
    // the current block is attended.  DEPTH > 2: taken DEPTH at a time, all
    // their loads issued before any is used.
    if constexpr (DEPTH == 2) {
        int blk0, s0, nv0, blk1, s1, nv1;
        bool f0, f1;
        u32x4 k0[LPB], v0[LPB], k1[LPB], v1[LPB];
        int i = a.i0 + wave;
        bool h0 = describe(i, blk0, s0, nv0, f0);
        if (h0)
            load_block(blk0, s0, f0, k0, v0);
        for (; i < a.i1; i += 2 * kAttnWaves) {
            const bool h1 = describe(i + kAttnWaves, blk1, s1, nv1, f1);
            if (h1)
                load_block(blk1, s1, f1, k1, v1);
            if (h0)
                attend_block(s0, nv0, f0, k0, v0);
            h0 = describe(i + 2 * kAttnWaves, blk0, s0, nv0, f0);
            if (h0)
                load_block(blk0, s0, f0, k0, v0);
            if (h1)
                attend_block(s1, nv1, f1, k1, v1);
        }
    } else {
        for (int base = a.i0 + wave; base < a.i1; base += DEPTH * kAttnWaves) {
            int blk[DEPTH], s[DEPTH], nv[DEPTH];
            bool fetch[DEPTH], have[DEPTH];
            u32x4 kv[DEPTH][LPB], vv[DEPTH][LPB];
#pragma unroll
            for (int d = 0; d < DEPTH; ++d) {
                have[d] = describe(base + d * kAttnWaves, blk[d], s[d], nv[d], fetch[d]);
                if (have[d])
                    load_block(blk[d], s[d], fetch[d], kv[d], vv[d]);
            }
#pragma unroll
            for (int d = 0; d < DEPTH; ++d)
                if (have[d])
                    attend_block(s[d], nv[d], fetch[d], kv[d], vv[d]);
        }
    }

    // combine the token groups of each wave, then the waves through LDS
#pragma unroll
    for (int g = 0; g < GMAX; ++g) {
        if (g >= G)
            continue;
        l[g] = token_groups_sum<LPT>(l[g]);
#pragma unroll
        for (int e = 0; e < EPL; ++e)
            acc[g][e] = token_groups_sum<LPT>(acc[g][e]);
        if (tg == 0) {
#pragma unroll
            for (int e = 0; e < EPL; ++e)
                S.sm[wave][g][sub * EPL + e] = acc[g][e];
            if (sub == 0) {
                S.sm[wave][g][D] = m[g];
                S.sm[wave][g][D + 1] = l[g];
            }
        }
    }
    combine_waves<D, GMAX>(a, S);
}

// Waves' partials (S.sm[w][g] = unnormalised output, max, sum) -> the
// workgroup's output (one split) or its partial for the merge.
template <int D, int GMAX> __device__ void combine_waves(const AttnRow &a, AttnSmem<D, GMAX> &S) {
    const int tid = threadIdx.x;
    const int G = a.G;
    __syncthreads();
    // per head: max over waves, then sum and output rescaled to it
    const int W = G * (D + 2);
    for (int idx = tid; idx < W; idx += kAttnThreads) {
        const int g = idx / (D + 2), c = idx - g * (D + 2);
        float M = -__builtin_inff();
#pragma unroll
        for (int w = 0; w < kAttnWaves; ++w)
            M = fmaxf(M, S.sm[w][g][D]);
        float r = M;
        if (c != D) {
            r = 0.0f;
            if (M != -__builtin_inff()) {
#pragma unroll
                for (int w = 0; w < kAttnWaves; ++w)
                    r = __builtin_fmaf(exp2f(S.sm[w][g][D] - M), S.sm[w][g][c], r);
            }
        }
        if (a.splits == 1) {
            if (c == D + 1)
                S.shL[g] = r;
            else if (c == D)
                S.shM[g] = r;
            else
                S.sm[0][g][c] = r;  // only this thread reads sm[.][g][c] for this c < D
        } else {
            a.part[idx] = r;
        }
    }
    if (a.splits == 1) {
        __syncthreads();
        for (int idx = tid; idx < G * D; idx += kAttnThreads) {
            const int g = idx / D, d = idx - g * D;
            const float L = S.shL[g];
            a.out[idx] = L > 0.0f ? S.sm[0][g][d] / L : 0.0f;
        }
        if (a.lse && tid < G)
            a.lse[tid] = S.shL[tid] > 0.0f ? S.shM[tid] * kLn2 + logf(S.shL[tid]) : -__builtin_inff();
    }
}

// bf16 storage: q.k of a whole block on the matrix cores, the value
// accumulation on the vector ALU.
//
// One v_mfma_f32_16x16x32_bf16 per 32 dims gives the block's 16 x 16 tile
// S[token][head] (heads beyond G are zero columns): the block's keys are the
// A operand (lane l holds token l%16, dims 32c + 8(l/16) .. +8, i.e. 16
// contiguous bytes) and the group's q the B operand (head l%16, same dims).
// Lane l then holds S for tokens 4(l/16) .. +4 of head l%16, so per block
// the max over tokens is 3 max + one cross-row max and each lane does 4
// exponentials for all heads at once.  V is read as rows: lane l holds
// dims (l%16)*D/16 .. of tokens 4(l/16) .. +4, and p[token][head g] reaches
// it by a row broadcast of lane g.  The lane's output is summed over its
// row's tokens; the 4 rows are added at the end.
// One block's K and V in the matrix-core body's lane layout (below).
template <int D> struct MfmaBlock {
    using VT = typename std::conditional<D / 8 == 16, u32x4, u32x2>::type;
    u32x4 kf[D / 32];
    VT vf[4];
    bool have;  // wave-uniform: loaded ahead for the wave's first block
};

// Loads block blk from the source (fetch) or pool slot s into b.
template <int D>
__device__ __forceinline__ void mfma_load_block(const AttnRow &a, int blk, int s, bool fetch, MfmaBlock<D> &b) {
    constexpr int KCH = D / 32, TB = D * 2, VB = D / 8;
    constexpr size_t kBlockBytes = (size_t)16 * TB;
    using VT = typename MfmaBlock<D>::VT;
    const int lane = threadIdx.x & 63, col = lane & 15, rsub = lane >> 4;
    const size_t k_off = (size_t)col * TB + rsub * 16;       // + 64 c
    const size_t v_off = (size_t)(4 * rsub) * TB + col * VB;  // + TB i
    const uint8_t *rk = fetch ? a.src_k + (size_t)blk * kBlockBytes : a.pool_k + (size_t)s * kBlockBytes;
    const uint8_t *rv = fetch ? a.src_v + (size_t)blk * kBlockBytes : a.pool_v + (size_t)s * kBlockBytes;
#pragma unroll
    for (int c = 0; c < KCH; ++c)
        b.kf[c] = fetch ? load_nt(rk + k_off + c * 64) : load16(rk + k_off + c * 64);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const VT *pv = reinterpret_cast<const VT *>(rv + v_off + i * TB);
        b.vf[i] = fetch ? __builtin_nontemporal_load(pv) : *pv;
    }
}

// first: the wave's first block (a.i0 + wave), when already loaded
// (first.have); its K and V registers are used in place of a load.
template <int D, int GMAX, int DEPTH>
__device__ __forceinline__ void attn_body_mfma(const AttnRow &a, AttnSmem<D, GMAX> &S, const MfmaBlock<D> &first) {
    constexpr int KCH = D / 32;   // 32-dim chunks of the contraction
    constexpr int VB = D / 8;     // bytes of a token's V per lane
    constexpr int EPLV = D / 16;  // V elements per lane per token
    constexpr int TB = D * 2;     // bytes of one token
    constexpr size_t kBlockBytes = (size_t)16 * TB;
    using VT = typename std::conditional<VB == 16, u32x4, u32x2>::type;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int col = lane & 15, rsub = lane >> 4;
    const int G = a.G;

    u32x4 qf[KCH];
#pragma unroll
    for (int c = 0; c < KCH; ++c)
        qf[c] = col < G ? load16(a.q + ((size_t)col * D + c * 32 + rsub * 8) * 2) : u32x4{0, 0, 0, 0};
    const size_t k_off = (size_t)col * TB + rsub * 16;       // + 64 c
    const size_t v_off = (size_t)(4 * rsub) * TB + col * VB;  // + TB i

    float m = -__builtin_inff(), lsum = 0.0f, acc[GMAX][EPLV];
#pragma unroll
    for (int g = 0; g < GMAX; ++g)
#pragma unroll
        for (int e = 0; e < EPLV; ++e)
            acc[g][e] = 0.0f;

    auto describe = [&](int i, int &blk, int &s, int &nv, bool &fetch) -> bool {
        if (i >= a.i1)
            return false;
        blk = a.blk[i];
        s = a.slot[i];
        if (blk < 0 || s < 0 || s >= a.C)
            return false;
        fetch = a.src_k != nullptr && blk < a.NB && a.hit[i] == 0;
        nv = min(max(a.len - blk * 16, 0), 16);
        return nv > 0 || fetch;
    };
    auto load_block = [&](int blk, int s, bool fetch, u32x4 *kf, VT *vf) {
        MfmaBlock<D> t;
        mfma_load_block<D>(a, blk, s, fetch, t);
#pragma unroll
        for (int c = 0; c < KCH; ++c)
            kf[c] = t.kf[c];
#pragma unroll
        for (int i = 0; i < 4; ++i)
            vf[i] = t.vf[i];
    };
    auto attend_block = [&](int s, int nv, bool fetch, const u32x4 *kf, const VT *vf) {
        if (fetch) {
            uint8_t *pk = a.pool_k + (size_t)s * kBlockBytes;
            uint8_t *pv = a.pool_v + (size_t)s * kBlockBytes;
#pragma unroll
            for (int c = 0; c < KCH; ++c)
                store16(pk + k_off + c * 64, kf[c]);
#pragma unroll
            for (int i = 0; i < 4; ++i)
                *reinterpret_cast<VT *>(pv + v_off + i * TB) = vf[i];
        }
        if (nv == 0)
            return;
        f32x4 st = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int c = 0; c < KCH; ++c)
            st = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, kf[c]),
                                                          __builtin_bit_cast(bf16x8, qf[c]), st, 0, 0, 0);
        float z[4];
#pragma unroll
        for (int i = 0; i < 4; ++i)
            z[i] = st[i] * a.scale_log2;
        if (nv < 16) {  // partial last block: drop the tokens past the end
#pragma unroll
            for (int i = 0; i < 4; ++i)
                if (4 * rsub + i >= nv)
                    z[i] = -__builtin_inff();
        }
        const float bm = rows_max(fmaxf(fmaxf(z[0], z[1]), fmaxf(z[2], z[3])));
        const float mn = fmaxf(m, bm);  // finite: token 0 of the block is valid
        const float alpha = exp2_fast(m - mn);
        m = mn;
        float p[4];
#pragma unroll
        for (int i = 0; i < 4; ++i)
            p[i] = exp2_fast(z[i] - mn);
        lsum = __builtin_fmaf(lsum, alpha, (p[0] + p[1]) + (p[2] + p[3]));
        float v[4][EPLV];
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int e = 0; e < EPLV; ++e)
                v[i][e] = (e & 1) ? bf16_hi(vf[i][e >> 1]) : bf16_lo(vf[i][e >> 1]);
        StaticFor<0, GMAX>::run([&](auto gc) {
            constexpr int g = decltype(gc)::value;
            const float ag = row_bcast<g>(alpha);
#pragma unroll
            for (int e = 0; e < EPLV; ++e)
                acc[g][e] *= ag;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float pg = row_bcast<g>(p[i]);
#pragma unroll
                for (int e = 0; e < EPLV; ++e)
                    acc[g][e] = __builtin_fmaf(pg, v[i][e], acc[g][e]);
            }
        });
    };

    if constexpr (DEPTH == 2) {
        int blk0, s0, nv0, blk1, s1, nv1;
        bool f0, f1;
        u32x4 k0[KCH], k1[KCH];
        VT v0[4], v1[4];
        int i = a.i0 + wave;
        bool h0 = describe(i, blk0, s0, nv0, f0);
        if (h0)
            load_block(blk0, s0, f0, k0, v0);
        for (; i < a.i1; i += 2 * kAttnWaves) {
            const bool h1 = describe(i + kAttnWaves, blk1, s1, nv1, f1);
            if (h1)
                load_block(blk1, s1, f1, k1, v1);
            if (h0)
                attend_block(s0, nv0, f0, k0, v0);
            h0 = describe(i + 2 * kAttnWaves, blk0, s0, nv0, f0);
            if (h0)
                load_block(blk0, s0, f0, k0, v0);
            if (h1)
                attend_block(s1, nv1, f1, k1, v1);
        }
    } else {
        static_assert(DEPTH == 1, "one or two blocks in flight");
        int i = a.i0 + wave;
        if (first.have) {  // wave-uniform; i < a.i1 when set
            int blk, s, nv;
            bool f;
            if (describe(i, blk, s, nv, f))
                attend_block(s, nv, f, first.kf, first.vf);
            i += kAttnWaves;
        }
        for (; i < a.i1; i += kAttnWaves) {
            int blk, s, nv;
            bool f;
            u32x4 kf[KCH];
            VT vf[4];
            if (describe(i, blk, s, nv, f)) {
                load_block(blk, s, f, kf, vf);
                attend_block(s, nv, f, kf, vf);
            }
        }
    }

    // the wave's totals: add the 4 rows (token groups); m is per column
    lsum = rows_sum(lsum);
#pragma unroll
    for (int g = 0; g < GMAX; ++g)
#pragma unroll
        for (int e = 0; e < EPLV; ++e)
            acc[g][e] = rows_sum(acc[g][e]);
    if (rsub == 0) {
#pragma unroll
        for (int g = 0; g < GMAX; ++g) {
            if (g >= G)
                continue;
#pragma unroll
            for (int e = 0; e < EPLV; ++e)
                S.sm[wave][g][col * EPLV + e] = acc[g][e];
        }
        if (col < G) {
            S.sm[wave][col][D] = m;
            S.sm[wave][col][D + 1] = lsum;
        }
    }
    combine_waves<D, GMAX>(a, S);
}

// bf16 takes the matrix-core body; the A/B build (SKV_AB_VALU_BF16, see
// build.py --ab-valu) runs the vector-ALU body for bf16 too, for the
// kernel-trace comparison only.
template <typename E> constexpr bool attn_matrix_cores() {
#ifdef SKV_AB_VALU_BF16
    return false;
#else
    return E::bytes == 2;
#endif
}

template <typename E, int D, int GMAX, int DEPTH>
__device__ __forceinline__ void attn_body(const AttnRow &a, AttnSmem<D, GMAX> &S, const MfmaBlock<D> &first) {
    if constexpr (attn_matrix_cores<E>())
        attn_body_mfma<D, GMAX, DEPTH>(a, S, first);
    else
        attn_body_valu<E, D, GMAX, DEPTH>(a, S);
}

template <typename E, int D, int GMAX, int DEPTH>
__device__ __forceinline__ void attn_body(const AttnRow &a, AttnSmem<D, GMAX> &S) {
    MfmaBlock<D> none;
    none.have = false;
    attn_body<E, D, GMAX, DEPTH>(a, S, none);
}

template <typename E, int D>
__device__ __forceinline__ void init_row(AttnRow &a, const uint8_t *q, uint8_t *pool_k, uint8_t *pool_v,
                                         const uint8_t *src_k, const uint8_t *src_v, int row, int b, int j, int Hq,
                                         int G, int C, int T, int split, int splits, float scale_log2, float *part,
                                         float *out, float *lse) {
    const size_t kv_row = (size_t)16 * D * E::bytes;
    a.q = q + ((size_t)b * Hq + (size_t)j * G) * D * E::bytes;
    a.pool_k = pool_k + (size_t)row * C * kv_row;
    a.pool_v = pool_v + (size_t)row * C * kv_row;
    a.src_k = src_k ? src_k + (size_t)row * T * D * E::bytes : nullptr;
    a.src_v = src_v ? src_v + (size_t)row * T * D * E::bytes : nullptr;
    a.C = C;
    a.NB = T / 16;
    a.G = G;
    a.splits = splits;
    a.scale_log2 = scale_log2;
    a.part = part + ((size_t)row * splits + split) * G * (D + 2);
    a.out = out + ((size_t)b * Hq + (size_t)j * G) * D;
    a.lse = lse ? lse + (size_t)b * Hq + (size_t)j * G : nullptr;
}

// Up to 4 heads per group: at least 4 waves per SIMD (<= 128 VGPRs), i.e.
// two 8-wave workgroups per CU; larger groups need the registers, and so
// does the vector-ALU body of the A/B build for bf16.
template <typename E> constexpr int attn_min_waves(int gmax) {
    return gmax <= 4 && (attn_matrix_cores<E>() || E::bytes == 4) ? 4 : 2;
}

template <typename E, int D, int GMAX>
__global__ __launch_bounds__(kAttnThreads, attn_min_waves<E>(GMAX)) void attn_kernel(
    const uint8_t *__restrict__ q, uint8_t *__restrict__ pool_k, uint8_t *__restrict__ pool_v, int C,
    const int32_t *__restrict__ sel_blocks, const int32_t *__restrict__ sel_slot, const uint8_t *__restrict__ sel_hit,
    const int32_t *__restrict__ sel_count, const int32_t *__restrict__ seq_lens, int Hq, int Hkv, int T, int k,
    int splits, int per_split, float scale_log2, const uint8_t *__restrict__ src_k, const uint8_t *__restrict__ src_v,
    float *__restrict__ part, float *__restrict__ out, float *__restrict__ lse) {
    __shared__ AttnSmem<D, GMAX> S;
    int row, split;
    xcd_row_part(row, split);
    const int b = row / Hkv, j = row - b * Hkv;
    const int n = min(max(sel_count[row], 0), k);
    AttnRow a;
    init_row<E, D>(a, q, pool_k, pool_v, src_k, src_v, row, b, j, Hq, Hq / Hkv, C, T, split, splits, scale_log2,
                   part, out, lse);
    a.blk = sel_blocks + (size_t)row * k;
    a.slot = sel_slot + (size_t)row * k;
    a.hit = sel_hit ? sel_hit + (size_t)row * k : nullptr;
    a.len = max(seq_lens[b], 0);
    a.i0 = split * per_split;
    a.i1 = min(a.i0 + per_split, n);
    attn_body<E, D, GMAX, 1>(a, S);
}

// Waves per SIMD of the fused kernel: 4 (two workgroups per CU, <= 128
// registers) where the top-k keys and the head state are small enough,
// else 2.  The host side (fused_waves_per_simd) applies the same rule.
template <typename E, int D, int GMAX, int KPT> constexpr int fused_min_waves() {
    return (attn_matrix_cores<E>() && GMAX <= 4 && KPT <= 8) ? 4 : 2;
}

// Blocks of K and V a wave of the fused kernel holds at once (see
// attn_body): at 4 waves per SIMD one; else two if they fit next to the
// per-head state in about 216 of its 256 registers.
template <typename E, int D, int GMAX> constexpr int fused_depth() {
    if constexpr (attn_matrix_cores<E>()) {  // matrix-core body: q, accumulators, K + V of a block
        constexpr int fixed = D / 8 + GMAX * D / 16 + 24;
        return fixed + 2 * (D / 4) <= 216 ? 2 : 1;
    } else {
        constexpr int lpb = D * E::bytes / 64;  // 16-byte loads per lane per block, K or V
        constexpr int fixed = GMAX * (4 + E::EPL + 2 + lpb);
        return fixed + 2 * 8 * lpb <= 216 ? 2 : 1;
    }
}

// LONG: rows over 16384 blocks, whose top-k's first launch
// (topk_chunk_kernel) has left each chunk's candidates in `cand`; every
// workgroup of the row selects from those (KPT candidates per thread) and
// plans with cache_plan_row.
template <typename E, int D, int GMAX, int KPT, bool LONG>
__global__ __launch_bounds__(kAttnThreads, (fused_min_waves<E, D, GMAX, LONG ? 32 : KPT>())) void select_attend_kernel(
    const float *__restrict__ scores, const float *__restrict__ cand, int chunk_blocks, int nchunks,
    const int32_t *__restrict__ seq_lens, int k, int sink, int recent, int C,
    int32_t *__restrict__ sel_blocks, int32_t *__restrict__ sel_count, int32_t *__restrict__ slot_block,
    uint32_t *__restrict__ slot_stamp, uint32_t *__restrict__ clock, int32_t *__restrict__ sel_slot,
    uint8_t *__restrict__ sel_hit,
    int32_t *__restrict__ miss_block, int32_t *__restrict__ miss_slot, int32_t *__restrict__ miss_count,
    const uint8_t *__restrict__ q, uint8_t *__restrict__ pool_k, uint8_t *__restrict__ pool_v,
    const uint8_t *__restrict__ src_k, const uint8_t *__restrict__ src_v, int Hq, int Hkv, int T, int splits,
    int per_split, float scale_log2, float *__restrict__ part, float *__restrict__ out, float *__restrict__ lse) {
    __shared__ TopkScratch tsc;
    __shared__ int32_t sS[kMaxK];
    __shared__ CacheScratch cs;
    __shared__ PlanScratch<kAttnThreads> ps;
    __shared__ AttnSmem<D, GMAX> S;
    __shared__ uint32_t sNow;
    int row, split;
    xcd_row_part(row, split);
    const int b = row / Hkv, j = row - b * Hkv;
    const int NB = T / 16;
    // the row's scores (a long row: its chunk candidates) first: their loads
    // need neither the length nor the slot table, and run while the rest is
    // set up
    TopkScores<LONG ? 1 : KPT> pre;
    LongCands<LONG ? KPT : 4> cands;
    const int nc = nchunks * long_row_stride(k);
    const float *wrow = cand + (size_t)row * 2 * nc;
    if constexpr (LONG)
        long_row_load<KPT>(wrow, reinterpret_cast<const int32_t *>(wrow + nc), nc, cands);
    else
        topk_load<KPT>(scores + (size_t)row * NB, NB, pre);
    const int len = min(max(seq_lens[b], 0), T);
    SlotRegs<kAttnThreads> regs;  // in flight while the top-k runs
    load_slots<kAttnThreads>(regs, C, slot_block + (size_t)row * C, slot_stamp + (size_t)row * C);
    select_plan_clear<kAttnThreads>(cs, ps, k, C);  // published by the emit's barriers
    AttnRow a;
    init_row<E, D>(a, q, pool_k, pool_v, src_k, src_v, row, b, j, Hq, Hq / Hkv, C, T, split, splits, scale_log2,
                   part, out, lse);
    constexpr int depth = fused_min_waves<E, D, GMAX, KPT>() == 4 ? 1 : fused_depth<E, D, GMAX>();

    uint64_t take = 0;
    if constexpr (!LONG)
        take = topk_take_loaded<kAttnThreads, KPT>(pre, len, NB, k, sink, recent, tsc);
    // once the hits are known, each wave loads its first block (a hit from
    // its pool slot, a miss from the source) so that the load is in flight
    // while the rest of the plan is worked out
    MfmaBlock<D> first;
    first.have = false;
    auto load_first = [&](int nn) {
        if constexpr (attn_matrix_cores<E>() && depth == 1) {
            // Every load issued before (scores, slot table, query) has long
            // landed.  Waiting for them here costs nothing and tells the
            // compiler that none is pending: otherwise, where this branch
            // rejoins, it assumes an older load may still be in flight and
            // makes the rest of the plan wait for this block's loads before
            // reusing that load's registers.
            __builtin_amdgcn_s_waitcnt(0x0f70);  // vmcnt(0)
            const int i0 = split * per_split;
            const int i = i0 + (threadIdx.x >> 6);
            if (i < min(i0 + per_split, nn)) {
                const int s = cs.slot_of[i];
                if (s >= 0 || src_k) {
                    mfma_load_block<D>(a, sS[i], s, s < 0, first);
                    first.have = true;
                }
            }
        }
    };
    int nn, bad, nm;
    if constexpr (LONG) {
        const int ncand = (min(nb_of(len), NB) + chunk_blocks - 1) / chunk_blocks * long_row_stride(k);
        nn = long_row_select<kAttnThreads, KPT>(cands, ncand, len, NB, k, sink, recent, sS, tsc);
        nm = cache_plan_row<kAttnThreads>(sS, nn, C, NB, regs, cs, bad);
    } else {
        nm = select_plan_row<kAttnThreads, KPT>(take, k, C, NB, regs, sS, cs, ps, nn, bad, load_first);
    }
    // one workgroup per row commits its own plan after attending (no other
    // workgroup reads the row's table); the clock's atomic goes out now
    const bool commit_here = splits == 1 && !bad;  // uniform
    if (commit_here && threadIdx.x == 0)
        sNow = atomicAdd(&clock[row], 1u) + 1u;
    if (split == 0) {
        for (int i = threadIdx.x; i < k; i += kAttnThreads)
            sel_blocks[(size_t)row * k + i] = sS[i];
        if (threadIdx.x == 0)
            sel_count[row] = nn;
        if (bad) {
            write_invalid_lists<kAttnThreads>(k, sel_slot + (size_t)row * k, sel_hit + (size_t)row * k,
                                              miss_block + (size_t)row * k, miss_slot + (size_t)row * k,
                                              miss_count + row);
        } else {
            write_lists<kAttnThreads>(sS, nn, nm, k, cs, sel_slot + (size_t)row * k, sel_hit + (size_t)row * k,
                                      miss_block + (size_t)row * k, miss_slot + (size_t)row * k, miss_count + row);
        }
    }
    a.blk = sS;
    a.slot = cs.slot_of;
    a.hit = cs.hit;
    a.len = len;
    a.i0 = split * per_split;
    a.i1 = bad ? a.i0 : min(a.i0 + per_split, nn);  // an invalid row attends nothing
    attn_body<E, D, GMAX, depth>(a, S, first);
    if (commit_here) {
        __syncthreads();
        const uint32_t now = sNow;
        for (int i = threadIdx.x; i < nn; i += kAttnThreads) {
            const int s = cs.slot_of[i];
            if (s >= 0 && s < C) {
                slot_block[(size_t)row * C + s] = sS[i];
                slot_stamp[(size_t)row * C + s] = now;
            }
        }
    }
}

// One workgroup per (row, head), rows placed on XCDs as the fused kernel
// places them (so a row's partials are read where they were written):
// merge the head's partials over the splits (when splits > 1); the row's
// head-0 workgroup also commits the row's working-set plan (when commit is
// set): every selected slot gets its block and the new stamp, the clock
// advances.  The kernel is a chain of dependent steps, so every global read
// it needs (commit operands, the clock advance, and the head's partials,
// staged in LDS when they fit) is issued before the first barrier; wave 0
// then forms the splits' weights exp2(m_s - M) and the denominator in
// registers.  (One workgroup per row merging all G heads read 33 KB per
// row at 32 splits x 8 heads, past the LDS stage, from global memory
// behind four barriers: 7 us on the 1M-context rows.)
constexpr int kMergeStage = 12288;  // floats of one head's partials staged in LDS (48 KiB)
constexpr int kCommitPerThread = kMaxK / kAttnThreads;
static_assert(kMaxSplits <= 128, "wave 0 holds two splits per lane");

__global__ __launch_bounds__(kAttnThreads) void merge_commit_kernel(
    const float *__restrict__ part, int Hq, int Hkv, int D, int splits, float *__restrict__ out,
    float *__restrict__ lse, int commit, int k, int C, const int32_t *__restrict__ sel_blocks,
    const int32_t *__restrict__ sel_count, const int32_t *__restrict__ sel_slot,
    const int32_t *__restrict__ miss_count, int32_t *__restrict__ slot_block, uint32_t *__restrict__ slot_stamp,
    uint32_t *__restrict__ clock) {
    __shared__ float stage[kMergeStage];
    __shared__ float sw[kMaxSplits];  // the weight exp2(m_s - M) of each split
    __shared__ float shM, shL;
    __shared__ uint32_t sNow;
    int row, g;
    xcd_row_part(row, g);  // grid (G, rows)
    const int tid = threadIdx.x;
    const int b = row / Hkv, j = row - b * Hkv;
    const int G = Hq / Hkv;
    const int HW = D + 2;      // floats of one head's partial: acc[D], m, l
    const int W = G * HW;      // floats of one split of the row
    const float *p = part + (size_t)row * splits * W + (size_t)g * HW;  // split s at p + s * W
    const bool staged = splits > 1 && splits * HW <= kMergeStage;
    const bool committer = commit && g == 0;  // uniform over the workgroup

    int mc = -1, n = 0, c_slot[kCommitPerThread], c_blk[kCommitPerThread];
    if (committer) {  // reads first, decisions after: none of these addresses depends on another read
        mc = miss_count[row];
        n = sel_count[row];
#pragma unroll
        for (int u = 0; u < kCommitPerThread; ++u) {
            const int i = tid + u * kAttnThreads;
            c_slot[u] = i < k ? sel_slot[(size_t)row * k + i] : -1;
            c_blk[u] = i < k ? sel_blocks[(size_t)row * k + i] : -1;
        }
    }
    if (staged) {
#pragma unroll 4
        for (int t = tid; t < splits * HW; t += kAttnThreads) {
            const int s = t / HW;
            stage[t] = p[(size_t)s * W + (t - s * HW)];
        }
    }
    const bool do_commit = committer && mc >= 0;  // uniform over the workgroup
    if (do_commit && tid == 0)
        sNow = atomicAdd(&clock[row], 1u) + 1u;
    n = min(max(n, 0), k);
    // split s's partial at src + s * stride, staged or in place
    const float *src = staged ? stage : p;
    const int stride = staged ? HW : W;
    if (splits > 1) {
        __syncthreads();
        if (tid < 64) {
            const int s0 = tid, s1 = tid + 64;
            const float m0 = s0 < splits ? src[s0 * stride + D] : -__builtin_inff();
            const float m1 = s1 < splits ? src[s1 * stride + D] : -__builtin_inff();
            const float M = wave_max(fmaxf(m0, m1));
            float w0 = 0.0f, w1 = 0.0f, l = 0.0f;
            if (M != -__builtin_inff()) {
                w0 = s0 < splits ? exp2f(m0 - M) : 0.0f;
                w1 = s1 < splits ? exp2f(m1 - M) : 0.0f;
                l = (s0 < splits ? w0 * src[s0 * stride + D + 1] : 0.0f) +
                    (s1 < splits ? w1 * src[s1 * stride + D + 1] : 0.0f);
            }
            const float L = rows_sum(group_sum<16>(l));
            if (s0 < splits)
                sw[s0] = L > 0.0f ? w0 : 0.0f;
            if (s1 < splits)
                sw[s1] = L > 0.0f ? w1 : 0.0f;
            if (tid == 0) {
                shM = M;
                shL = L;
            }
        }
        __syncthreads();
        const float L = shL;
        float *o = out + ((size_t)b * Hq + (size_t)j * G + g) * D;
        for (int d = tid; d < D; d += kAttnThreads) {
            float a = 0.0f;
#pragma unroll 8
            for (int s = 0; s < splits; ++s)
                a = __builtin_fmaf(sw[s], src[s * stride + d], a);
            o[d] = L > 0.0f ? a / L : 0.0f;
        }
        if (lse && tid == 0)
            lse[(size_t)b * Hq + (size_t)j * G + g] = L > 0.0f ? shM * kLn2 + logf(L) : -__builtin_inff();
    }
    if (do_commit) {
        __syncthreads();
        const uint32_t now = sNow;
#pragma unroll
        for (int u = 0; u < kCommitPerThread; ++u) {
            const int s = c_slot[u];
            if (tid + u * kAttnThreads < n && s >= 0 && s < C) {
                slot_block[(size_t)row * C + s] = c_blk[u];
                slot_stamp[(size_t)row * C + s] = now;
            }
        }
    }
}

// Enough workgroups for two per CU across the chip, but no more than one
// block per wave.  Measured on the 32K workload (64 rows, 128 blocks): 8
// splits 27 us, 16 splits (one block per wave) 31 us, 32 splits 41 us.
int attention_auto_splits(int rows, int k) {
    constexpr int kResident = 512;  // two 8-wave workgroups on each of 256 CUs
    int s = (kResident + rows - 1) / rows;
    const int one_per_wave = (k + kAttnWaves - 1) / kAttnWaves;
    if (s > one_per_wave)
        s = one_per_wave;
    return s < 1 ? 1 : (s > kMaxSplits ? kMaxSplits : s);
}

// The fused call redoes the row's top-k and plan in every workgroup, so it
// prefers as many workgroups as are resident at once (one or two per CU,
// see fused_min_waves), each wave streaming several blocks.
static_assert(kAttnThreads == kLongRowThreads, "the fused kernel runs the long-row selection's second step");

int fused_waves_per_simd(const Dims &d) {
    return (d.dtype == 1 && attn_matrix_cores<BF16>() && d.G() <= 4 && d.NB <= kAttnThreads * 8) ? 4 : 2;
}

int fused_auto_splits(const Dims &d, int k) {
    const int rows = d.rows();
    const int resident = 256 * fused_waves_per_simd(d) / 2;  // workgroups resident on 256 CUs
    int s = (resident + rows - 1) / rows;
    // at least one block for every other wave (128K Quest rows, 32 blocks: 8
    // splits 24.2 us, 4 splits 25.0, 16 splits 37.5)
    const int half_waves = (k + kAttnWaves / 2 - 1) / (kAttnWaves / 2);
    if (s > half_waves)
        s = half_waves;
    return s < 1 ? 1 : (s > kMaxSplits ? kMaxSplits : s);
}

size_t attention_ws_bytes(int rows, int G, int D, int splits) {
    if (splits <= 1)
        return 256;
    size_t b = (size_t)rows * splits * G * (D + 2) * sizeof(float);
    return (b + 255) & ~(size_t)255;
}

template <typename E, int D, int GMAX>
static hipError_t attn_t(const Dims &d, const AttnArgs &a, hipStream_t st) {
    const int per = (a.k + a.splits - 1) / a.splits;
    const float scale_log2 = a.scale * 1.4426950408889634f;
    float *part = (float *)a.ws;
    hipLaunchKernelGGL((attn_kernel<E, D, GMAX>), dim3(a.splits, d.rows()), dim3(kAttnThreads), 0, st,
                       (const uint8_t *)a.q, (uint8_t *)a.pool_k, (uint8_t *)a.pool_v, a.cap, a.sel_blocks, a.sel_slot,
                       a.sel_hit, a.sel_count, a.seq_lens, d.Hq, d.Hkv, d.T, a.k, a.splits, per, scale_log2,
                       (const uint8_t *)a.src_k, (const uint8_t *)a.src_v, part, a.out, a.lse);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || a.splits == 1)
        return e;
    hipLaunchKernelGGL(merge_commit_kernel, dim3(d.G(), d.rows()), dim3(kAttnThreads), 0, st, (const float *)part,
                       d.Hq, d.Hkv, d.D, a.splits, a.out, a.lse, 0, a.k, a.cap, nullptr, nullptr, nullptr, nullptr, nullptr,
                       nullptr, nullptr);
    return hipGetLastError();
}

template <typename E, int D>
static hipError_t attn_g(const Dims &d, const AttnArgs &a, hipStream_t st) {
    const int G = d.G();
    if (G <= 4)
        return attn_t<E, D, 4>(d, a, st);
    if (G <= 8)
        return attn_t<E, D, 8>(d, a, st);
    return attn_t<E, D, 16>(d, a, st);
}

hipError_t launch_attention(const Dims &d, const AttnArgs &a, hipStream_t st) {
    if (d.dtype == 1)
        return d.D == 128 ? attn_g<BF16, 128>(d, a, st) : attn_g<BF16, 64>(d, a, st);
    return d.D == 128 ? attn_g<F32, 128>(d, a, st) : attn_g<F32, 64>(d, a, st);
}

// ---------------------------------------------------------------- fused
size_t fused_ws_bytes(const Dims &d, int k, int splits) {
    return attention_ws_bytes(d.rows(), d.G(), d.D, splits) + long_row_ws_bytes(d, k);
}

template <typename E, int D, int GMAX, int KPT, bool LONG>
static hipError_t fused_t(const Dims &d, const FusedArgs &f, hipStream_t st) {
    const int per = (f.k + f.splits - 1) / f.splits;
    const float scale_log2 = f.scale * 1.4426950408889634f;
    float *part = (float *)f.ws;
    // rows over 16384 blocks: the chunk candidates follow the partials
    float *cand = (float *)((char *)f.ws + attention_ws_bytes(d.rows(), d.G(), d.D, f.splits));
    const int ch = LONG ? long_row_chunk(d.NB, f.k) : 0, nch = LONG ? long_row_chunks(d.NB, f.k) : 0;
    if (LONG) {
        hipError_t e = launch_topk_chunks(d, f.scores, f.seq_lens, f.k, f.sink, f.recent, cand, st);
        if (e != hipSuccess)
            return e;
    }
    hipLaunchKernelGGL((select_attend_kernel<E, D, GMAX, KPT, LONG>), dim3(f.splits, d.rows()), dim3(kAttnThreads), 0,
                       st, f.scores, cand, ch, nch, f.seq_lens, f.k, f.sink, f.recent, f.cap, f.sel_blocks,
                       f.sel_count, f.slot_block, f.slot_stamp, f.clock, f.sel_slot, f.sel_hit, f.miss_block,
                       f.miss_slot, f.miss_count, (const uint8_t *)f.q, (uint8_t *)f.pool_k, (uint8_t *)f.pool_v,
                       (const uint8_t *)f.src_k, (const uint8_t *)f.src_v, d.Hq, d.Hkv, d.T, f.splits, per,
                       scale_log2, part, f.out, f.lse);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || f.splits == 1)  // one split per row: the kernel wrote out / lse and committed
        return e;
    hipLaunchKernelGGL(merge_commit_kernel, dim3(d.G(), d.rows()), dim3(kAttnThreads), 0, st, (const float *)part,
                       d.Hq, d.Hkv, d.D, f.splits, f.out, f.lse, 1, f.k, f.cap, f.sel_blocks, f.sel_count, f.sel_slot,
                       f.miss_count, f.slot_block, f.slot_stamp, f.clock);
    return hipGetLastError();
}

template <typename E, int D, int GMAX>
static hipError_t fused_k(const Dims &d, const FusedArgs &f, hipStream_t st) {
    if (d.NB <= kAttnThreads * 4)
        return fused_t<E, D, GMAX, 4, false>(d, f, st);
    if (d.NB <= kAttnThreads * 8)
        return fused_t<E, D, GMAX, 8, false>(d, f, st);
    if (d.NB <= kAttnThreads * 16)
        return fused_t<E, D, GMAX, 16, false>(d, f, st);
    if (d.NB <= kAttnThreads * 32)
        return fused_t<E, D, GMAX, 32, false>(d, f, st);
    switch (long_row_kpt(d, f.k)) {  // phase B keys per thread (kAttnThreads == kLongRowThreads)
    case 4:
        return fused_t<E, D, GMAX, 4, true>(d, f, st);
    case 8:
        return fused_t<E, D, GMAX, 8, true>(d, f, st);
    default:
        return fused_t<E, D, GMAX, 32, true>(d, f, st);
    }
}

template <typename E, int D>
static hipError_t fused_g(const Dims &d, const FusedArgs &f, hipStream_t st) {
    const int G = d.G();
    if (G <= 4)
        return fused_k<E, D, 4>(d, f, st);
    if (G <= 8)
        return fused_k<E, D, 8>(d, f, st);
    return fused_k<E, D, 16>(d, f, st);
}

hipError_t launch_select_attend(const Dims &d, const FusedArgs &f, hipStream_t st) {
    if (d.dtype == 1)
        return d.D == 128 ? fused_g<BF16, 128>(d, f, st) : fused_g<BF16, 64>(d, f, st);
    return d.D == 128 ? fused_g<F32, 128>(d, f, st) : fused_g<F32, 64>(d, f, st);
}

}  // namespace skv
