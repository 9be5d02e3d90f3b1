// Stage 2: per-(sequence, kv-head) top-k under the KV budget on gfx950.
//
// Each row keeps its forced blocks (the ones covering the first sink tokens
// and the last recent tokens: sink + recent + top-scored, "KV Cache 塞不进 HBM
// 了" §2.3) and fills the rest of its budget (a per-head, per-step cap, same
// page §3 step 2) with the best-scored remaining valid blocks, ties broken
// towards the lower block id.  Output is ascending by block id.
//
// One workgroup per row: 512 threads up to 8192 blocks, 1024 up to 16384
// (measured: 512 threads take the 128K Quest rows' top-k from 13.1 to 11.5
// us, and are slower than 1024 beyond 8192 blocks).  Scores become order-preserving 32-bit
// keys held in registers (KPT per thread, thread t owns the contiguous ids
// [t*KPT, t*KPT+KPT)).  Four 8-bit radix passes with an LDS histogram find
// the key of the last block the budget admits and how many blocks with
// exactly that key still fit; one pass of two workgroup prefix sums then
// emits the chosen ids in ascending order (ties at the threshold go to the
// lowest ids because the equal-key rank is a prefix count in id order).
#include "skv_rowops.h"

namespace skv {

constexpr int kTopkLongThreads = 1024;

template <int THREADS, int KPT>
__global__ __launch_bounds__(THREADS) void topk_kernel(const float *__restrict__ scores,
                                                            const int32_t *__restrict__ seq_lens, int Hkv, int T,
                                                            int NB, int k, int sink, int recent,
                                                            int32_t *__restrict__ sel_blocks,
                                                            int32_t *__restrict__ sel_count) {
    __shared__ TopkScratch sc;
    const int row = blockIdx.x;
    const int len = min(max(seq_lens[row / Hkv], 0), T);
    const int n = topk_row<THREADS, KPT>(scores + (size_t)row * NB, len, NB, k, sink, recent,
                                              sel_blocks + (size_t)row * k, sc);
    if (threadIdx.x == 0)
        sel_count[row] = n;
}

// Rows longer than 16384 blocks: the long-row path (thread maxima bound the
// threshold, the exact select runs over the few keys that reach it).
__global__ __launch_bounds__(kTopkLongThreads) void topk_long_kernel(const float *__restrict__ scores,
                                                                 const int32_t *__restrict__ seq_lens, int Hkv, int T,
                                                                 int NB, int k, int sink, int recent,
                                                                 int32_t *__restrict__ sel_blocks,
                                                                 int32_t *__restrict__ sel_count) {
    __shared__ TopkLongScratch ls;
    const int row = blockIdx.x;
    const int len = min(max(seq_lens[row / Hkv], 0), T);
    const float *srow = scores + (size_t)row * NB;
    int32_t *out = sel_blocks + (size_t)row * k;
    const int n = topk_long_row<kTopkLongThreads>(srow, len, NB, k, sink, recent, out, ls);
    if (threadIdx.x == 0)
        sel_count[row] = n;
}

template <int THREADS, int KPT>
static hipError_t topk_t(const Dims &d, const float *scores, const int32_t *lens, int k, int sink, int recent,
                         int32_t *sel, int32_t *cnt, hipStream_t st) {
    hipLaunchKernelGGL((topk_kernel<THREADS, KPT>), dim3(d.rows()), dim3(THREADS), 0, st, scores, lens, d.Hkv, d.T,
                       d.NB, k, sink, recent, sel, cnt);
    return hipGetLastError();
}

hipError_t launch_topk(const Dims &d, const float *scores, const int32_t *lens, int k, int sink, int recent,
                       int32_t *sel, int32_t *cnt, hipStream_t st) {
    const int kpt = (d.NB + 511) / 512;  // keys per thread with 512 threads
    if (kpt <= 1)
        return topk_t<512, 1>(d, scores, lens, k, sink, recent, sel, cnt, st);
    if (kpt <= 2)
        return topk_t<512, 2>(d, scores, lens, k, sink, recent, sel, cnt, st);
    if (kpt <= 4)
        return topk_t<512, 4>(d, scores, lens, k, sink, recent, sel, cnt, st);
    if (kpt <= 8)
        return topk_t<512, 8>(d, scores, lens, k, sink, recent, sel, cnt, st);
    if (kpt <= 16)
        return topk_t<512, 16>(d, scores, lens, k, sink, recent, sel, cnt, st);
    if (kpt <= 32)
        return topk_t<1024, 16>(d, scores, lens, k, sink, recent, sel, cnt, st);
    hipLaunchKernelGGL(topk_long_kernel, dim3(d.rows()), dim3(kTopkLongThreads), 0, st, scores, lens, d.Hkv, d.T, d.NB, k,
                       sink, recent, sel, cnt);
    return hipGetLastError();
}

}  // namespace skv
