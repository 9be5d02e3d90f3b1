// Decode-time KV append on gfx950.
//
// The pages place the method's gains where the KV cache grows during
// decoding ("KV Cache 塞不进 HBM 了", intro and §1).  One call stores each
// sequence's new key and value rows (one token per kv head) at token
// seq_lens[b], keeps the Quest min/max box of the block that token falls in
// exact without rescanning it (a new block starts from the token itself,
// else the element-wise min/max with it; the box of stored values is made of
// stored values, so this is bit-exact), refreshes the pool copy of that block
// when it is resident in the row's working set (so a resident slot always
// holds its block's bytes), and grows seq_lens[b] by one.  A full sequence
// (seq_lens[b] >= T) is left as it is.
//
// One workgroup per sequence, so that every kv head of the sequence reads
// the old length before thread 0 writes the new one; inside it one wave per
// kv head.  The first D*e/16 lanes of the wave own 16-byte slices of the row
// (coalesced copies); the whole wave scans the row's slot table 64 slots at a
// time and refreshes every slot that holds the block.
#include "skv_device.h"
#include "skv_launch.h"

namespace skv {

constexpr int kAppendThreads = 512;

template <typename E, int D>
__global__ __launch_bounds__(kAppendThreads) void append_kernel(
    const uint8_t *__restrict__ new_k, const uint8_t *__restrict__ new_v, int32_t *__restrict__ seq_lens,
    uint8_t *__restrict__ keys, uint8_t *__restrict__ values, uint8_t *__restrict__ meta, int Hkv, int T,
    const int32_t *__restrict__ slot_block, int C, uint8_t *__restrict__ pool_k, uint8_t *__restrict__ pool_v) {
    constexpr int ROWB = D * E::bytes;  // bytes of one token's row
    constexpr int LPR = ROWB / 16;      // lanes per row
    static_assert(LPR <= 64, "one wave holds a row");
    const int b = blockIdx.x;
    const int len = seq_lens[b];
    const int NB = T / 16;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    if (len >= 0 && len < T) {
        const int blk = len >> 4, tok = len & 15;
        const bool owner = lane < LPR;
        for (int j = wave; j < Hkv; j += kAppendThreads / 64) {
            const size_t r = (size_t)b * Hkv + j;
            u32x4 kv{}, vv{};
            if (owner) {
                kv = load16(new_k + r * ROWB + lane * 16);
                vv = load16(new_v + r * ROWB + lane * 16);
                store16(keys + (r * T + len) * ROWB + lane * 16, kv);
                store16(values + (r * T + len) * ROWB + lane * 16, vv);
            }
            if (meta && owner) {
                uint8_t *lo = meta + ((r * NB + blk) * 2) * ROWB + lane * 16;
                uint8_t *hi = lo + ROWB;
                u32x4 a = kv, c = kv;
                if (tok != 0) {
                    const u32x4 ol = load16(lo), oh = load16(hi);
#pragma unroll
                    for (int w = 0; w < 4; ++w) {
                        if constexpr (E::bytes == 2) {
                            // per 16-bit half: keep the stored value that is smaller / larger
                            const float k0 = bf16_lo(kv[w]), k1 = bf16_hi(kv[w]);
                            const uint32_t l0 = k0 < bf16_lo(ol[w]) ? kv[w] : ol[w];
                            const uint32_t l1 = k1 < bf16_hi(ol[w]) ? kv[w] : ol[w];
                            const uint32_t h0 = k0 > bf16_lo(oh[w]) ? kv[w] : oh[w];
                            const uint32_t h1 = k1 > bf16_hi(oh[w]) ? kv[w] : oh[w];
                            a[w] = (l0 & 0xffffu) | (l1 & 0xffff0000u);
                            c[w] = (h0 & 0xffffu) | (h1 & 0xffff0000u);
                        } else {
                            const float kf = __uint_as_float(kv[w]);
                            a[w] = kf < __uint_as_float(ol[w]) ? kv[w] : ol[w];
                            c[w] = kf > __uint_as_float(oh[w]) ? kv[w] : oh[w];
                        }
                    }
                }
                store16(lo, a);
                store16(hi, c);
            }
            if (slot_block) {
                for (int s0 = 0; s0 < C; s0 += 64) {
                    const bool hit = s0 + lane < C && slot_block[r * C + s0 + lane] == blk;
                    for (uint64_t m = __builtin_amdgcn_ballot_w64(hit); m; m &= m - 1) {
                        const int s = s0 + __builtin_ctzll(m);
                        if (owner) {
                            const size_t po = ((r * C + s) * 16 + tok) * ROWB + lane * 16;
                            store16(pool_k + po, kv);
                            store16(pool_v + po, vv);
                        }
                    }
                }
            }
        }
        __syncthreads();
        if (threadIdx.x == 0)
            seq_lens[b] = len + 1;
    }
}

template <typename E, int D>
static hipError_t append_t(const Dims &d, const void *nk, const void *nv, int32_t *lens, void *k, void *v, void *meta,
                           const int32_t *sb, int cap, void *pk, void *pv, hipStream_t st) {
    hipLaunchKernelGGL((append_kernel<E, D>), dim3(d.B), dim3(kAppendThreads), 0, st, (const uint8_t *)nk,
                       (const uint8_t *)nv, lens, (uint8_t *)k, (uint8_t *)v, (uint8_t *)meta, d.Hkv, d.T, sb, cap,
                       (uint8_t *)pk, (uint8_t *)pv);
    return hipGetLastError();
}

hipError_t launch_append(const Dims &d, const void *new_k, const void *new_v, int32_t *seq_lens, void *keys,
                         void *values, void *meta, const int32_t *slot_block, int cap, void *pool_k, void *pool_v,
                         hipStream_t st) {
    if (d.dtype == 1)
        return d.D == 128 ? append_t<BF16, 128>(d, new_k, new_v, seq_lens, keys, values, meta, slot_block, cap,
                                                pool_k, pool_v, st)
                          : append_t<BF16, 64>(d, new_k, new_v, seq_lens, keys, values, meta, slot_block, cap,
                                               pool_k, pool_v, st);
    return d.D == 128 ? append_t<F32, 128>(d, new_k, new_v, seq_lens, keys, values, meta, slot_block, cap, pool_k,
                                           pool_v, st)
                      : append_t<F32, 64>(d, new_k, new_v, seq_lens, keys, values, meta, slot_block, cap, pool_k,
                                          pool_v, st);
}

}  // namespace skv
