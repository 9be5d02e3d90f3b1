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
//
// Rows over 16384 blocks run in two launches (topk_chunk_kernel, then
// topk_long_kernel; see long_row_select): one workgroup per chunk of
// 1024-4096 blocks keeps the chunk's best blocks in the caller's workspace,
// then one workgroup per row selects from those candidates.  On 8 rows of
// 65536 blocks (k = 128) the two launches take 6.0 and 4.9 us; the
// selection with the working-set plan (sparse_kv_select) 22 us over both,
// against 36 us for one workgroup per row streaming the whole row.
#include "skv_rowops.h"

namespace skv {

template <int THREADS, int KPT>
__global__ __launch_bounds__(THREADS) void topk_kernel(const float *__restrict__ scores,
                                                            const int32_t *__restrict__ seq_lens, int Hkv, int T,
                                                            int NB, int k, int sink, int recent,
                                                            int32_t *__restrict__ sel_blocks,
                                                            int32_t *__restrict__ sel_count) {
    __shared__ TopkScratch sc;
    const int row = blockIdx.x;
    TopkScores<KPT> pre;  // issued before the length is known
    topk_load<KPT>(scores + (size_t)row * NB, NB, pre);
    const int len = min(max(seq_lens[row / Hkv], 0), T);
    const int n = topk_row<THREADS, KPT>(pre, len, NB, k, sink, recent, sel_blocks + (size_t)row * k, sc);
    if (threadIdx.x == 0)
        sel_count[row] = n;
}

// Long rows, phase A: grid (chunks, rows), one workgroup of THREADS per
// chunk of THREADS * KPT blocks (rows placed on XCDs as the scoring kernels
// place them).  ws: per row, chunks * stride scores, then as many ids.
template <int THREADS, int KPT>
__global__ __launch_bounds__(THREADS) void topk_chunk_kernel(const float *__restrict__ scores,
                                                             const int32_t *__restrict__ seq_lens, int Hkv, int T,
                                                             int NB, int k, int sink, int recent,
                                                             float *__restrict__ ws) {
    __shared__ TopkScratch sc;
    int row, chunk;
    xcd_row_part(row, chunk);
    float v[KPT];  // issued before the length is known
    chunk_load<THREADS, KPT>(scores + (size_t)row * NB, NB, chunk, v);
    const int len = min(max(seq_lens[row / Hkv], 0), T);
    const int nvalid = min(nb_of(len), NB);
    // uniform: a row of at most k valid blocks takes them all without its
    // candidates, and phase B reads no entry of a chunk past the valid part
    if (nvalid <= k || chunk * THREADS * KPT >= nvalid)
        return;
    const size_t nc = (size_t)gridDim.x * long_row_stride(k);
    float *wrow = ws + (size_t)row * 2 * nc;
    const size_t off = (size_t)chunk * long_row_stride(k);
    chunk_candidates<THREADS, KPT>(v, len, NB, k, sink, recent, chunk, wrow + off,
                                   reinterpret_cast<int32_t *>(wrow + nc) + off, sc);
}

// The candidates phase B reads for a row: the chunks that hold valid blocks.
__device__ __forceinline__ int long_row_ncand(int len, int NB, int k, int chunk_blocks) {
    return (min(nb_of(len), NB) + chunk_blocks - 1) / chunk_blocks * long_row_stride(k);
}

// Long rows, phase B of the top-k: one workgroup of kLongRowThreads per row.
template <int KPT>
__global__ __launch_bounds__(kLongRowThreads) void topk_long_kernel(const int32_t *__restrict__ seq_lens, int Hkv,
                                                                    int T, int NB, int k, int sink, int recent,
                                                                    int chunk_blocks, int nchunks,
                                                                    const float *__restrict__ ws,
                                                                    int32_t *__restrict__ sel_blocks,
                                                                    int32_t *__restrict__ sel_count) {
    __shared__ TopkScratch sc;
    __shared__ int32_t sS[kMaxK];
    const int row = blockIdx.x;
    const int nc = nchunks * long_row_stride(k);
    const float *wrow = ws + (size_t)row * 2 * nc;
    LongCands<KPT> cands;  // issued before the length is known
    long_row_load<KPT>(wrow, reinterpret_cast<const int32_t *>(wrow + nc), nc, cands);
    const int len = min(max(seq_lens[row / Hkv], 0), T);
    const int n = long_row_select<kLongRowThreads, KPT>(cands, long_row_ncand(len, NB, k, chunk_blocks), len, NB, k,
                                                        sink, recent, sS, sc);
    for (int i = threadIdx.x; i < k; i += kLongRowThreads)
        sel_blocks[(size_t)row * k + i] = sS[i];
    if (threadIdx.x == 0)
        sel_count[row] = n;
}

size_t long_row_ws_bytes(const Dims &d, int k) {
    return d.NB > kLongRowBlocks ? (size_t)d.rows() * long_row_chunks(d.NB, k) * long_row_stride(k) * 8 : 0;
}

hipError_t launch_topk_chunks(const Dims &d, const float *scores, const int32_t *lens, int k, int sink, int recent,
                              float *ws, hipStream_t st) {
    const int ch = long_row_chunk(d.NB, k);
    const dim3 grid(long_row_chunks(d.NB, k), d.rows());
    if (ch == 1024)
        hipLaunchKernelGGL((topk_chunk_kernel<kChunkThreads, 4>), grid, dim3(kChunkThreads), 0, st, scores, lens,
                           d.Hkv, d.T, d.NB, k, sink, recent, ws);
    else if (ch == 2048)
        hipLaunchKernelGGL((topk_chunk_kernel<kChunkThreads, 8>), grid, dim3(kChunkThreads), 0, st, scores, lens,
                           d.Hkv, d.T, d.NB, k, sink, recent, ws);
    else
        hipLaunchKernelGGL((topk_chunk_kernel<kChunkThreads, 16>), grid, dim3(kChunkThreads), 0, st, scores, lens,
                           d.Hkv, d.T, d.NB, k, sink, recent, ws);
    return hipGetLastError();
}

// Keys per thread of phase B for a row's candidate count: 4, 8 or 32.  (No
// row of 16385 to 65536 blocks with k <= 1024 has 4097 to 8192 candidates:
// a chunk size that fails the 4096 bound and meets the 16384 one gives more
// than 8192.)
int long_row_kpt(const Dims &d, int k) {
    const int ncand = long_row_chunks(d.NB, k) * long_row_stride(k);
    return ncand <= 4 * kLongRowThreads ? 4 : ncand <= 8 * kLongRowThreads ? 8 : 32;
}

template <int THREADS, int KPT>
static hipError_t topk_t(const Dims &d, const float *scores, const int32_t *lens, int k, int sink, int recent,
                         int32_t *sel, int32_t *cnt, hipStream_t st) {
    hipLaunchKernelGGL((topk_kernel<THREADS, KPT>), dim3(d.rows()), dim3(THREADS), 0, st, scores, lens, d.Hkv, d.T,
                       d.NB, k, sink, recent, sel, cnt);
    return hipGetLastError();
}

hipError_t launch_topk(const Dims &d, const float *scores, const int32_t *lens, int k, int sink, int recent,
                       int32_t *sel, int32_t *cnt, void *ws, hipStream_t st) {
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
    hipError_t e = launch_topk_chunks(d, scores, lens, k, sink, recent, static_cast<float *>(ws), st);
    if (e != hipSuccess)
        return e;
    const int ch = long_row_chunk(d.NB, k), nch = long_row_chunks(d.NB, k);
    const float *w = static_cast<const float *>(ws);
#define SKV_TOPK_LONG(KP)                                                                                         \
    hipLaunchKernelGGL(topk_long_kernel<KP>, dim3(d.rows()), dim3(kLongRowThreads), 0, st, lens, d.Hkv, d.T, d.NB, \
                       k, sink, recent, ch, nch, w, sel, cnt)
    switch (long_row_kpt(d, k)) {
    case 4:
        SKV_TOPK_LONG(4);
        break;
    case 8:
        SKV_TOPK_LONG(8);
        break;
    default:
        SKV_TOPK_LONG(32);
    }
#undef SKV_TOPK_LONG
    return hipGetLastError();
}

}  // namespace skv
