// Stage 4: GQA decode attention over the selected blocks, split-K with an
// online-softmax merge, on gfx950.
//
// Exact attention over the KV the step kept (OasisKV summary, key module 1)
// read from the working set through the slot table (a block-table
// indirection: KV-Cache 压缩技术的工程原理 §5.2), so the result does not
// depend on which tier the blocks came from (HiSparse promo, insight 1).
//
// attn_splitk_kernel: grid (splits, rows), 256 threads.  The workgroup of
// split s walks its contiguous share of the row's selection; its 4 waves
// take interleaved blocks.  A wave loads a block's K and V (16 tokens) with
// the same coalesced 16-byte lane layout as the scoring kernel and uses
// them for all G query heads of the kv group at once (each K/V byte is
// read once per group).  Logits are kept in base-2 units
// (scale*log2(e)*q.k), the running max is per head and wave-uniform, and
// each lane accumulates its own tokens' share of l and of the output, so
// the only per-block cross-lane traffic is the dot-product sums and one max
// per head.  The waves are merged through LDS and the workgroup writes
// (max, sum, unnormalised output) for each head to the workspace.
// attn_merge_kernel: one workgroup per (b, h) rescales the splits'
// partials by exp2(m_s - m*) and normalises.
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

constexpr int kAttnWaves = 4;

template <typename E, int D, int GMAX>
__global__ __launch_bounds__(256) void attn_splitk_kernel(
    const uint8_t *__restrict__ q, const uint8_t *__restrict__ pool_k, const uint8_t *__restrict__ pool_v, int C,
    const int32_t *__restrict__ sel_blocks, const int32_t *__restrict__ sel_slot,
    const int32_t *__restrict__ sel_count, const int32_t *__restrict__ seq_lens, int Hq, int Hkv, int k,
    int splits, int per_split, float scale_log2, float *__restrict__ ws) {
    constexpr int LPT = D * E::bytes / 16;
    constexpr int TPL = 64 / LPT;
    constexpr int LPB = 16 / TPL;
    constexpr int EPL = E::EPL;
    __shared__ float sm[kAttnWaves][GMAX][D + 2];

    const int row = blockIdx.y, split = blockIdx.x;
    const int b = row / Hkv, j = row - b * Hkv;
    const int G = Hq / Hkv;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
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
    const size_t block_bytes = (size_t)16 * D * E::bytes;

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
        const int nv = min(max(len - blk * 16, 0), 16);
        if (nv == 0)
            continue;
        const size_t base = ((size_t)row * C + s) * block_bytes;
        u32x4 kv[LPB], vv[LPB];
#pragma unroll
        for (int li = 0; li < LPB; ++li)
            kv[li] = load16(pool_k + base + ((size_t)(li * TPL + tg) * D + sub * EPL) * E::bytes);
#pragma unroll
        for (int li = 0; li < LPB; ++li)
            vv[li] = load16(pool_v + base + ((size_t)(li * TPL + tg) * D + sub * EPL) * E::bytes);

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

    // combine the token groups of the wave, then the waves through LDS
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
    float *wout = ws + ((size_t)row * splits + split) * G * (D + 2);
    for (int idx = threadIdx.x; idx < G * (D + 2); idx += 256) {
        const int g = idx / (D + 2), c = idx - g * (D + 2);
        float M = -__builtin_inff();
#pragma unroll
        for (int w = 0; w < kAttnWaves; ++w)
            M = fmaxf(M, sm[w][g][D]);
        float r;
        if (c == D) {
            r = M;
        } else if (M == -__builtin_inff()) {
            r = 0.0f;
        } else {
            r = 0.0f;
#pragma unroll
            for (int w = 0; w < kAttnWaves; ++w) {
                const float f = exp2f(sm[w][g][D] - M);
                r = __builtin_fmaf(f, c == D + 1 ? sm[w][g][D + 1] : sm[w][g][c], r);
            }
        }
        wout[idx] = r;
    }
}

// one workgroup per (b, h); thread d owns output element d
__global__ __launch_bounds__(128) void attn_merge_kernel(const float *__restrict__ ws, int Hq, int Hkv, int D,
                                                         int splits, float *__restrict__ out,
                                                         float *__restrict__ lse) {
    const int bh = blockIdx.x;
    const int b = bh / Hq, h = bh - b * Hq;
    const int G = Hq / Hkv;
    const int j = h / G, g = h - j * G;
    const int row = b * Hkv + j;
    const float *p = ws + (size_t)row * splits * G * (D + 2) + (size_t)g * (D + 2);
    const size_t stride = (size_t)G * (D + 2);
    float M = -__builtin_inff();
    for (int s = 0; s < splits; ++s)
        M = fmaxf(M, p[s * stride + D]);
    float L = 0.0f;
    if (M != -__builtin_inff())
        for (int s = 0; s < splits; ++s)
            L = __builtin_fmaf(exp2f(p[s * stride + D] - M), p[s * stride + D + 1], L);
    const bool empty = !(L > 0.0f);
    for (int d = threadIdx.x; d < D; d += blockDim.x) {
        float a = 0.0f;
        if (!empty)
            for (int s = 0; s < splits; ++s)
                a = __builtin_fmaf(exp2f(p[s * stride + D] - M), p[s * stride + d], a);
        out[(size_t)bh * D + d] = empty ? 0.0f : a / L;
    }
    if (lse && threadIdx.x == 0)
        lse[bh] = empty ? -__builtin_inff() : M * 0.69314718055994531f + logf(L);
}

int attention_auto_splits(int rows, int k) {
    int s = (1024 + rows - 1) / rows;
    const int cap = k / 4 > 1 ? k / 4 : 1;
    if (s > cap)
        s = cap;
    return s < 1 ? 1 : s;
}

size_t attention_ws_bytes(int rows, int G, int D, int splits) {
    size_t b = (size_t)rows * splits * G * (D + 2) * sizeof(float);
    return (b + 255) & ~(size_t)255;
}

template <typename E, int D, int GMAX>
static hipError_t attn_t(const Dims &d, const void *q, const void *pk, const void *pv, int cap, const int32_t *sb,
                         const int32_t *ss, const int32_t *sc, const int32_t *lens, int k, float scale, int splits,
                         float *out, float *lse, float *ws, hipStream_t st) {
    const int per = (k + splits - 1) / splits;
    const float scale_log2 = scale * 1.4426950408889634f;
    hipLaunchKernelGGL((attn_splitk_kernel<E, D, GMAX>), dim3(splits, d.rows()), dim3(256), 0, st,
                       (const uint8_t *)q, (const uint8_t *)pk, (const uint8_t *)pv, cap, sb, ss, sc, lens, d.Hq,
                       d.Hkv, k, splits, per, scale_log2, ws);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess)
        return e;
    hipLaunchKernelGGL(attn_merge_kernel, dim3(d.B * d.Hq), dim3(128), 0, st, (const float *)ws, d.Hq, d.Hkv, D,
                       splits, out, lse);
    return hipGetLastError();
}

template <typename E, int D>
static hipError_t attn_g(const Dims &d, const void *q, const void *pk, const void *pv, int cap, const int32_t *sb,
                         const int32_t *ss, const int32_t *sc, const int32_t *lens, int k, float scale, int splits,
                         float *out, float *lse, float *ws, hipStream_t st) {
    const int G = d.G();
    if (G <= 4)
        return attn_t<E, D, 4>(d, q, pk, pv, cap, sb, ss, sc, lens, k, scale, splits, out, lse, ws, st);
    if (G <= 8)
        return attn_t<E, D, 8>(d, q, pk, pv, cap, sb, ss, sc, lens, k, scale, splits, out, lse, ws, st);
    return attn_t<E, D, 16>(d, q, pk, pv, cap, sb, ss, sc, lens, k, scale, splits, out, lse, ws, st);
}

hipError_t launch_attention(const Dims &d, const void *q, const void *pk, const void *pv, int cap,
                            const int32_t *sb, const int32_t *ss, const int32_t *sc, const int32_t *lens, int k,
                            float scale, int splits, float *out, float *lse, float *ws, hipStream_t st) {
    if (d.dtype == 1)
        return d.D == 128 ? attn_g<BF16, 128>(d, q, pk, pv, cap, sb, ss, sc, lens, k, scale, splits, out, lse, ws, st)
                          : attn_g<BF16, 64>(d, q, pk, pv, cap, sb, ss, sc, lens, k, scale, splits, out, lse, ws, st);
    return d.D == 128 ? attn_g<F32, 128>(d, q, pk, pv, cap, sb, ss, sc, lens, k, scale, splits, out, lse, ws, st)
                      : attn_g<F32, 64>(d, q, pk, pv, cap, sb, ss, sc, lens, k, scale, splits, out, lse, ws, st);
}

}  // namespace skv
