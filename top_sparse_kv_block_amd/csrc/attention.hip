// Stage 4: GQA decode attention over the selected blocks, split-K with an
// online-softmax merge, on gfx950.
//
// Exact attention over the KV the step kept (OasisKV summary, key module 1)
// read from the working set through the slot table (a block-table
// indirection: KV-Cache 压缩技术的工程原理 §5.2), so the result does not
// depend on which tier the blocks came from (HiSparse promo, insight 1).
//
// attn_kernel: grid (splits, rows), 8 waves.  The workgroup of split s owns
// a contiguous share of the row's selection and each wave takes one block
// of it at a time, so a workgroup has all of its blocks' K and V loads in
// flight at once.  A wave loads the block's K and V (16 tokens) with the
// coalesced 16-byte lane layout of the scoring kernel and uses them for all
// G query heads of the kv group (each byte is read once per group).
// Logits are kept in base-2 units (scale*log2(e)*q.k); the running max is
// per head and wave-uniform; each lane accumulates its own tokens' share of
// l and of the output, so per block the only cross-lane work is the
// dot-product sums and one max per head.  Waves are combined in LDS; with
// one split the workgroup writes the output directly, otherwise it writes
// (max, sum, unnormalised output) per head to the workspace.
// attn_merge_kernel: one workgroup per (b, h) loads every split's (max, sum)
// in one round of independent loads, forms the weights exp2(m_s - m*) in
// LDS, and each thread sums its output element over the splits.  (A merge
// by the last workgroup of each row would need a device-scope release per
// workgroup, which on this chip writes back the whole L2 each time.)
//
// Fetch on attend (optional): when a source cache is given, a selected
// block that was not resident (sel_hit == 0) is read from the source by
// block id and also written into its pool slot, so the miss costs one read
// and one write and no separate copy pass.
#include "skv_device.h"
#include "skv_launch.h"

namespace skv {

template <int LPT> __device__ __forceinline__ float token_groups_max(float v);
template <> __device__ __forceinline__ float token_groups_max<8>(float v) {
    v = fmaxf(v, dpp<DPP_ROW_ROR8>(v));
    return rows_max(v);
}
template <> __device__ __forceinline__ float token_groups_max<16>(float v) { return rows_max(v); }
template <> __device__ __forceinline__ float token_groups_max<32>(float v) { return fmaxf(v, __shfl_xor(v, 32)); }

template <int LPT> __device__ __forceinline__ float token_groups_sum(float v);
template <> __device__ __forceinline__ float token_groups_sum<8>(float v) {
    v += __shfl_xor(v, 8);
    return rows_sum(v);
}
template <> __device__ __forceinline__ float token_groups_sum<16>(float v) { return rows_sum(v); }
template <> __device__ __forceinline__ float token_groups_sum<32>(float v) { return v + __shfl_xor(v, 32); }

template <typename E> __device__ __forceinline__ float elem(u32x4 v, int e) {
    if constexpr (E::bytes == 2)
        return (e & 1) ? bf16_hi(v[e >> 1]) : bf16_lo(v[e >> 1]);
    else
        return __uint_as_float(v[e]);
}

constexpr int kAttnWaves = 8;
constexpr int kAttnThreads = 64 * kAttnWaves;
constexpr float kLn2 = 0.69314718055994531f;

template <typename E, int D, int GMAX>
__global__ __launch_bounds__(kAttnThreads) void attn_kernel(
    const uint8_t *__restrict__ q, uint8_t *__restrict__ pool_k, uint8_t *__restrict__ pool_v, int C,
    const int32_t *__restrict__ sel_blocks, const int32_t *__restrict__ sel_slot, const uint8_t *__restrict__ sel_hit,
    const int32_t *__restrict__ sel_count, const int32_t *__restrict__ seq_lens, int Hq, int Hkv, int T, int k,
    int splits, int per_split, float scale_log2, const uint8_t *__restrict__ src_k, const uint8_t *__restrict__ src_v,
    float *__restrict__ part, float *__restrict__ out, float *__restrict__ lse) {
    constexpr int LPT = D * E::bytes / 16;
    constexpr int TPL = 64 / LPT;
    constexpr int LPB = 16 / TPL;
    constexpr int EPL = E::EPL;
    constexpr size_t kBlockBytes = (size_t)16 * D * E::bytes;
    __shared__ float sm[kAttnWaves][GMAX][D + 2];
    __shared__ float shM[GMAX], shL[GMAX];

    const int row = blockIdx.y, split = blockIdx.x;
    const int b = row / Hkv, j = row - b * Hkv;
    const int G = Hq / Hkv;
    const int NB = T / 16;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int sub = lane % LPT, tg = lane / LPT;

    u32x4 qf[GMAX];
#pragma unroll
    for (int g = 0; g < GMAX; ++g)
        qf[g] = g < G ? load16(q + (((size_t)b * Hq + (size_t)j * G + g) * D + sub * EPL) * E::bytes)
                      : u32x4{0, 0, 0, 0};

    const int len = max(seq_lens[b], 0);
    const int n = min(max(sel_count[row], 0), k);
    const int i0 = split * per_split;
    const int i1 = min(i0 + per_split, n);
    const int32_t *sblk = sel_blocks + (size_t)row * k;
    const int32_t *sslot = sel_slot + (size_t)row * k;

    float m[GMAX], l[GMAX], acc[GMAX][EPL];
#pragma unroll
    for (int g = 0; g < GMAX; ++g) {
        m[g] = -__builtin_inff();
        l[g] = 0.0f;
#pragma unroll
        for (int e = 0; e < EPL; ++e)
            acc[g][e] = 0.0f;
    }

    for (int i = i0 + wave; i < i1; i += kAttnWaves) {
        const int blk = sblk[i], s = sslot[i];
        if (blk < 0 || s < 0 || s >= C)
            continue;
        const bool fetch = src_k != nullptr && blk < NB && sel_hit[(size_t)row * k + i] == 0;
        const int nv = min(max(len - blk * 16, 0), 16);
        if (nv == 0 && !fetch)
            continue;
        uint8_t *pk = pool_k + ((size_t)row * C + s) * kBlockBytes;
        uint8_t *pv = pool_v + ((size_t)row * C + s) * kBlockBytes;
        const uint8_t *rk = fetch ? src_k + ((size_t)row * T + (size_t)blk * 16) * D * E::bytes : pk;
        const uint8_t *rv = fetch ? src_v + ((size_t)row * T + (size_t)blk * 16) * D * E::bytes : pv;
        const size_t lo = ((size_t)tg * D + sub * EPL) * E::bytes;
        constexpr size_t step = (size_t)TPL * D * E::bytes;
        u32x4 kv[LPB], vv[LPB];
#pragma unroll
        for (int li = 0; li < LPB; ++li)
            kv[li] = fetch ? load_nt(rk + lo + li * step) : load16(rk + lo + li * step);
#pragma unroll
        for (int li = 0; li < LPB; ++li)
            vv[li] = fetch ? load_nt(rv + lo + li * step) : load16(rv + lo + li * step);
        if (fetch) {
#pragma unroll
            for (int li = 0; li < LPB; ++li) {
                store16(pk + lo + li * step, kv[li]);
                store16(pv + lo + li * step, vv[li]);
            }
        }
        if (nv == 0)
            continue;

        float z[LPB][GMAX];
#pragma unroll
        for (int li = 0; li < LPB; ++li) {
            const bool valid = li * TPL + tg < nv;
#pragma unroll
            for (int g = 0; g < GMAX; ++g) {
                float t = -__builtin_inff();
                if (g < G) {
                    t = group_sum<LPT>(dot_chunk<E>(kv[li], qf[g], 0.0f)) * scale_log2;
                    if (!valid)
                        t = -__builtin_inff();
                }
                z[li][g] = t;
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
            const float alpha = exp2f(m[g] - mn);  // m = -inf -> 0
            m[g] = mn;
            l[g] *= alpha;
#pragma unroll
            for (int e = 0; e < EPL; ++e)
                acc[g][e] *= alpha;
#pragma unroll
            for (int li = 0; li < LPB; ++li) {
                const float p = exp2f(z[li][g] - mn);
                l[g] += p;
#pragma unroll
                for (int e = 0; e < EPL; ++e)
                    acc[g][e] = __builtin_fmaf(p, elem<E>(vv[li], e), acc[g][e]);
            }
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
                sm[wave][g][sub * EPL + e] = acc[g][e];
            if (sub == 0) {
                sm[wave][g][D] = m[g];
                sm[wave][g][D + 1] = l[g];
            }
        }
    }
    __syncthreads();
    // per head: max over waves, then sum and output rescaled to it
    const int W = G * (D + 2);
    float *wpart = part + ((size_t)row * splits + split) * W;
    for (int idx = tid; idx < W; idx += kAttnThreads) {
        const int g = idx / (D + 2), c = idx - g * (D + 2);
        float M = -__builtin_inff();
#pragma unroll
        for (int w = 0; w < kAttnWaves; ++w)
            M = fmaxf(M, sm[w][g][D]);
        float r = M;
        if (c != D) {
            r = 0.0f;
            if (M != -__builtin_inff()) {
#pragma unroll
                for (int w = 0; w < kAttnWaves; ++w)
                    r = __builtin_fmaf(exp2f(sm[w][g][D] - M), sm[w][g][c], r);
            }
        }
        if (splits == 1) {
            if (c == D + 1)
                shL[g] = r;
            else if (c == D)
                shM[g] = r;
            else
                sm[0][g][c] = r;  // only this thread reads sm[.][g][c] for this c < D
        } else {
            wpart[idx] = r;
        }
    }
    const size_t obase = ((size_t)b * Hq + (size_t)j * G) * D;
    if (splits == 1) {
        __syncthreads();
        for (int idx = tid; idx < G * D; idx += kAttnThreads) {
            const int g = idx / D, d = idx - g * D;
            const float L = shL[g];
            out[obase + idx] = L > 0.0f ? sm[0][g][d] / L : 0.0f;
        }
        if (lse && tid < G)
            lse[(size_t)b * Hq + (size_t)j * G + tid] = shL[tid] > 0.0f ? shM[tid] * kLn2 + logf(shL[tid])
                                                                          : -__builtin_inff();
        return;
    }
}

// one workgroup per (b, h); thread d owns output element d
__global__ __launch_bounds__(128) void attn_merge_kernel(const float *__restrict__ part, int Hq, int Hkv, int D,
                                                         int splits, float *__restrict__ out,
                                                         float *__restrict__ lse) {
    __shared__ float sw[kMaxSplits];  // weight of split s: exp2(m_s - M)
    __shared__ float sl[kMaxSplits];
    __shared__ float shM, shL;
    const int bh = blockIdx.x;
    const int b = bh / Hq, h = bh - b * Hq;
    const int G = Hq / Hkv;
    const int j = h / G, g = h - j * G;
    const size_t W = (size_t)G * (D + 2);
    const float *p = part + (size_t)(b * Hkv + j) * splits * W + (size_t)g * (D + 2);
    for (int s = threadIdx.x; s < splits; s += blockDim.x) {
        sw[s] = p[s * W + D];
        sl[s] = p[s * W + D + 1];
    }
    __syncthreads();
    if (threadIdx.x == 0) {
        float M = -__builtin_inff();
        for (int s = 0; s < splits; ++s)
            M = fmaxf(M, sw[s]);
        float L = 0.0f;
        if (M != -__builtin_inff())
            for (int s = 0; s < splits; ++s)
                L = __builtin_fmaf(exp2f(sw[s] - M), sl[s], L);
        shM = M;
        shL = L;
    }
    __syncthreads();
    const float M = shM, L = shL;
    for (int s = threadIdx.x; s < splits; s += blockDim.x)
        sw[s] = L > 0.0f ? exp2f(sw[s] - M) : 0.0f;
    __syncthreads();
    for (int d = threadIdx.x; d < D; d += blockDim.x) {
        float a = 0.0f;
#pragma unroll 8
        for (int s = 0; s < splits; ++s)
            a = __builtin_fmaf(sw[s], p[s * W + d], a);
        out[(size_t)bh * D + d] = L > 0.0f ? a / L : 0.0f;
    }
    if (lse && threadIdx.x == 0)
        lse[bh] = L > 0.0f ? M * kLn2 + logf(L) : -__builtin_inff();
}

int attention_auto_splits(int rows, int k) {
    (void)rows;
    int s = (k + kAttnWaves - 1) / kAttnWaves;  // one block per wave
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
    hipLaunchKernelGGL(attn_merge_kernel, dim3(d.B * d.Hq), dim3(128), 0, st, (const float *)part, d.Hq, d.Hkv, D,
                       a.splits, a.out, a.lse);
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

}  // namespace skv
