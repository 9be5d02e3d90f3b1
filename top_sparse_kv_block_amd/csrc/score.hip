// Stage 1: block scoring on gfx950.
//
// Exact block-max: a block's score is scale times the largest q.k over its
// valid tokens, the GQA group's heads ("KV Cache 塞不进 HBM 了", §3 step 3:
// element-wise max inside the group) and the scoring queries (lookahead
// drafts: OasisKV summary, key module 2).
// Quest bound: sum_d max(q_d*min_d, q_d*max_d) over a block's element-wise key
// box, an upper bound of every q.k in the block.
//
// Layout on the chip.  A (b, kv-head) row of keys is T*D contiguous
// elements; one 16-token block is 16*D*e contiguous bytes (4 KiB for bf16,
// D=128).  bf16 keys are scored on the matrix cores (see the MFMA kernel
// below); float32 keys on the vector ALU as follows.
// A wave reads a block with fully coalesced 16-byte lane loads:
// LPT = D*e/16 lanes share a token (each holds EPL consecutive elements),
// TPL = 64/LPT tokens per wave load, 16/TPL loads per block.  Each lane
// keeps the matching 16-byte slice of every query row in registers, forms
// partial dot products (packed bf16 dot2 or fp32 FMA), and the LPT-lane
// partials are summed with DPP row rotations; no LDS is used.  The work is
// HBM-bound (about 4 flop per byte at G=4), so the kernel is organised
// around keeping many 16-byte loads in flight: the waves of a workgroup walk
// interleaved blocks of one row, non-temporal loads for the key stream.
#include "skv_device.h"
#include "skv_launch.h"

namespace skv {

template <int LPT> __device__ __forceinline__ float groups_max(float v);
template <> __device__ __forceinline__ float groups_max<8>(float v) {
    v = fmaxf(v, dpp<DPP_ROW_ROR8>(v));
    return rows_max(v);
}
template <> __device__ __forceinline__ float groups_max<16>(float v) { return rows_max(v); }
template <> __device__ __forceinline__ float groups_max<32>(float v) { return xor32_max(v); }

// Workgroups of 4 waves (the vector kernel walks 4 blocks per wave, the
// matrix-core kernel the counts below); non-temporal loads for the key
// stream were worth 20% on the 32K workload.
constexpr int kScoreWaves = 4;
constexpr int kScoreBlocksPerWave = 4;
// matrix-core scan: blocks per wave with one operand tile (up to 16 query
// rows) and with two.  Measured with 4-wave workgroups: 32K, one tile, one
// block per wave 72.8 us (2 blocks: 78.3); 1M with 4 drafts, two tiles, 4
// blocks per wave 300-308 us (16 blocks: 316-321).  Workgroups of 16 waves
// were slower at every setting (32K: 75-77 us; 1M: 314-350 us), as were 8
// (73.7-74.6 / 308-312), 2 (78.2 / 303-305) and 1 (80.1-80.6 / 300).
constexpr int kMfmaBlocksPerWave1 = 1;
constexpr int kMfmaBlocksPerWave2 = 4;
template <int NT> constexpr int mfma_blocks_per_wave() { return NT > 1 ? kMfmaBlocksPerWave2 : kMfmaBlocksPerWave1; }
constexpr int kScoreThreads = 64 * kScoreWaves;
// the Quest scan keeps 8 boxes in flight per lane (76 VGPRs): smaller
// workgroups let six waves per SIMD stay resident
constexpr int kQuestWaves = 4;
constexpr int kQuestThreads = 64 * kQuestWaves;
constexpr int kQuestBlocksPerWave = 4;  // wave iterations, each BPL blocks
// matrix-core Quest scan: one tile of 16 boxes per wave, two waves per
// workgroup.  Measured on the 128K workload (32 rows x 8192 boxes, 134 MB):
// 20.9 us with 2 waves, 21.1 with 1, 21.5 with 8, 22.4 with 4; two tiles per
// wave 24.0; the box operand loaded straight from memory (64 bytes per box
// per instruction) instead of through LDS 24.3-31.4.
constexpr int kQuestMfmaWaves = 2;

template <typename E, int D, int RMAX>
__global__ __launch_bounds__(kScoreThreads) void score_blockmax_kernel(const uint8_t *__restrict__ q,
                                                             const uint8_t *__restrict__ keys,
                                                             const int32_t *__restrict__ seq_lens,
                                                             float *__restrict__ scores, int Hq, int Hkv, int NQ,
                                                             int T, int NB, float scale) {
    constexpr int LPT = D * E::bytes / 16;
    constexpr int TPL = 64 / LPT;
    constexpr int LPB = 16 / TPL;
    int row, wgp;
    xcd_row_part(row, wgp);
    const int b = row / Hkv, j = row - b * Hkv;
    const int G = Hq / Hkv;
    const int R = NQ * G;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int sub = lane % LPT, tg = lane / LPT;

    // unconditional loads: under a uniform branch each ends in a wait for
    // all loads at the branch's join, which serialises them
    u32x4 qf[RMAX];
#pragma unroll
    for (int r = 0; r < RMAX; ++r) {
        const int rr = min(r, R - 1);
        const int rq = rr / G, g = rr - rq * G;
        const u32x4 v = load16(q + ((((size_t)b * NQ + rq) * Hq + (size_t)j * G + g) * D + sub * E::EPL) * E::bytes);
        qf[r] = r < R ? v : u32x4{0, 0, 0, 0};
    }
    const int len = min(max(seq_lens[b], 0), T);
    const int nvalid = nb_of(len);
    const uint8_t *krow = keys + (size_t)row * T * D * E::bytes;
    float *srow = scores + (size_t)row * NB;
    const int n0 = wgp * (kScoreWaves * kScoreBlocksPerWave);
    const int n1 = min(n0 + kScoreWaves * kScoreBlocksPerWave, NB);

    for (int n = n0 + wave; n < n1; n += kScoreWaves) {
        if (n >= nvalid) {
            if (lane == 0)
                srow[n] = -__builtin_inff();
            continue;
        }
        u32x4 kv[LPB];
#pragma unroll
        for (int i = 0; i < LPB; ++i)
            kv[i] = load_nt(krow + ((size_t)(n * 16 + i * TPL + tg) * D + sub * E::EPL) * E::bytes);
        float m = -__builtin_inff();
#pragma unroll
        for (int i = 0; i < LPB; ++i) {
            float best = -__builtin_inff();
#pragma unroll
            for (int r = 0; r < RMAX; ++r) {
                const float v = group_sum<LPT>(dot_chunk<E>(kv[i], qf[r], 0.0f));
                best = r < R ? fmaxf(best, v) : best;
            }
            if (n * 16 + i * TPL + tg < len)
                m = fmaxf(m, best);
        }
        m = groups_max<LPT>(m);
        if (lane == 0)
            srow[n] = m * scale;
    }
}

// bf16 block max on the matrix cores, for many query rows (lookahead
// drafts x GQA heads).  One v_mfma_f32_16x16x32_bf16 per 32 dims and per
// tile of 16 query rows gives S[token][query] for a whole block.  The MFMA
// wants each lane to hold 16 contiguous bytes of token l%16 (the A operand:
// dims 32c + 8(l/16) .. +8), which as a global load would read only 64
// contiguous bytes per token per instruction; so the wave reads the block
// with the fully coalesced lane layout of the vector kernel (4 tokens x
// 256 bytes per instruction), writes it to its own LDS tile (rows padded by
// 16 bytes, so both access patterns are free of bank conflicts) and reads
// the A operand back from there.  The query rows are the B operand (row
// 16t + l%16, same dims).  Lane l then holds S for tokens 4(l/16) .. +4 of
// query row 16t + l%16; the block's score is the max over the valid tokens
// and real query rows, one wave reduction.
template <int D, int NT>
__global__ __launch_bounds__(kScoreThreads) void score_blockmax_mfma_kernel(const uint8_t *__restrict__ q,
                                                                  const uint8_t *__restrict__ keys,
                                                                  const int32_t *__restrict__ seq_lens,
                                                                  float *__restrict__ scores, int Hq, int Hkv,
                                                                  int NQ, int T, int NB, float scale) {
    constexpr int KCH = D / 32;
    constexpr int TB = D * 2;          // bytes of one token
    constexpr int ROW = TB + 16;       // padded LDS row
    constexpr int LPT = TB / 16;       // lanes per token in the coalesced layout
    constexpr int TPL = 64 / LPT;      // tokens per load instruction
    constexpr int LPB = 16 / TPL;      // load instructions per block
    __shared__ __attribute__((aligned(16))) uint8_t tile[kScoreWaves][16 * ROW];
    int row, wgp;
    xcd_row_part(row, wgp);
    const int b = row / Hkv, j = row - b * Hkv;
    const int G = Hq / Hkv;
    const int R = NQ * G;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int col = lane & 15, rsub = lane >> 4;
    const int sub = lane % LPT, tg = lane / LPT;
    uint8_t *my = tile[wave];

    u32x4 qf[NT][KCH];
#pragma unroll
    for (int t = 0; t < NT; ++t) {
        const int r = 16 * t + col;
        const int rq = r / G, g = r - rq * G;
#pragma unroll
        for (int c = 0; c < KCH; ++c)
            qf[t][c] = r < R ? load16(q + ((((size_t)b * NQ + rq) * Hq + (size_t)j * G + g) * D + c * 32 + rsub * 8) * 2)
                             : u32x4{0, 0, 0, 0};
    }
    const int len = min(max(seq_lens[b], 0), T);
    const int nvalid = nb_of(len);
    const uint8_t *krow = keys + (size_t)row * T * TB;
    float *srow = scores + (size_t)row * NB;
    const int n0 = wgp * (kScoreWaves * mfma_blocks_per_wave<NT>());
    const int n1 = min(n0 + kScoreWaves * mfma_blocks_per_wave<NT>(), NB);

    for (int n = n0 + wave; n < n1; n += kScoreWaves) {
        if (n >= nvalid) {
            if (lane == 0)
                srow[n] = -__builtin_inff();
            continue;
        }
        u32x4 kv[LPB];
#pragma unroll
        for (int i = 0; i < LPB; ++i)
            kv[i] = load_nt(krow + (size_t)(n * 16 + i * TPL + tg) * TB + sub * 16);
#pragma unroll
        for (int i = 0; i < LPB; ++i)
            *reinterpret_cast<u32x4 *>(my + (i * TPL + tg) * ROW + sub * 16) = kv[i];
        __builtin_amdgcn_wave_barrier();
        u32x4 kf[KCH];
#pragma unroll
        for (int c = 0; c < KCH; ++c)
            kf[c] = *reinterpret_cast<const u32x4 *>(my + col * ROW + c * 64 + rsub * 16);
        __builtin_amdgcn_wave_barrier();  // the tile is rewritten by the next block
        float m = -__builtin_inff();
#pragma unroll
        for (int t = 0; t < NT; ++t) {
            f32x4 st = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
            for (int c = 0; c < KCH; ++c)
                st = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, kf[c]),
                                                              __builtin_bit_cast(bf16x8, qf[t][c]), st, 0, 0, 0);
            if (16 * t + col < R) {
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    if (n * 16 + 4 * rsub + i < len)
                        m = fmaxf(m, st[i]);
            }
        }
        m = wave_max(m);
        if (lane == 0)
            srow[n] = m * scale;
    }
}

// Quest bound.  max(q*lo, q*hi) = q * (q >= 0 ? hi : lo), so each lane
// selects, per element, the box corner the query's sign points to (one
// bit-select per packed word) and takes a plain dot product with q.
template <typename E> __device__ __forceinline__ uint32_t neg_mask(uint32_t qw);
template <> __device__ __forceinline__ uint32_t neg_mask<BF16>(uint32_t qw) {
    typedef short s16x2 __attribute__((ext_vector_type(2)));
    return __builtin_bit_cast(uint32_t, __builtin_bit_cast(s16x2, qw) >> (s16x2){15, 15});  // one packed shift
}
template <> __device__ __forceinline__ uint32_t neg_mask<F32>(uint32_t qw) {
    return (uint32_t)((int32_t)qw >> 31);
}

template <typename E, int D, int RMAX>
__global__ __launch_bounds__(kQuestThreads) void score_quest_kernel(const uint8_t *__restrict__ q,
                                                          const uint8_t *__restrict__ meta,
                                                          const int32_t *__restrict__ seq_lens,
                                                          float *__restrict__ scores, int Hq, int Hkv, int NQ, int T,
                                                          int NB, float scale) {
    constexpr int LPT = D * E::bytes / 16;  // lanes covering one D-vector
    constexpr int BPL = 64 / LPT;           // blocks per wave iteration
    int row, wgp;
    xcd_row_part(row, wgp);
    const int b = row / Hkv, j = row - b * Hkv;
    const int G = Hq / Hkv;
    const int R = NQ * G;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int sub = lane % LPT, bg = lane / LPT;

    // the query rows are loaded unconditionally (rows past R repeat row R - 1
    // and are zeroed afterwards): loads under a uniform branch each end in a
    // wait for all loads at the branch's join, which serialised these loads
    // and delayed the boxes' (27.1 against 21.x us per 128K scan)
    u32x4 qf[RMAX];
#pragma unroll
    for (int r = 0; r < RMAX; ++r) {
        const int rr = min(r, R - 1);
        const int rq = rr / G, g = rr - rq * G;
        const u32x4 v = load16(q + ((((size_t)b * NQ + rq) * Hq + (size_t)j * G + g) * D + sub * E::EPL) * E::bytes);
        qf[r] = r < R ? v : u32x4{0, 0, 0, 0};
    }
    const int len = min(max(seq_lens[b], 0), T);
    const int nvalid = nb_of(len);
    const size_t vec_bytes = (size_t)D * E::bytes;
    const uint8_t *mrow = meta + (size_t)row * NB * 2 * vec_bytes;
    float *srow = scores + (size_t)row * NB;
    const int per_wg = kQuestWaves * BPL * kQuestBlocksPerWave;
    const int n0 = wgp * per_wg;
    const int n1 = min(n0 + per_wg, NB);

    // all of the wave's boxes are loaded before any is used, so each wave
    // keeps kQuestBlocksPerWave loads in flight instead of one
    u32x4 lo[kQuestBlocksPerWave], hi[kQuestBlocksPerWave];
#pragma unroll
    for (int i = 0; i < kQuestBlocksPerWave; ++i) {
        const int n = n0 + (i * kQuestWaves + wave) * BPL + bg;
        lo[i] = hi[i] = u32x4{0, 0, 0, 0};
        if (n < n1 && n < nvalid) {
            lo[i] = load_nt(mrow + (size_t)n * 2 * vec_bytes + sub * 16);
            hi[i] = load_nt(mrow + (size_t)n * 2 * vec_bytes + vec_bytes + sub * 16);
        }
    }
#pragma unroll
    for (int i = 0; i < kQuestBlocksPerWave; ++i) {
        const int n = n0 + (i * kQuestWaves + wave) * BPL + bg;
        const bool in = n < n1 && n < nvalid;
        float best = -__builtin_inff();
#pragma unroll
        for (int r = 0; r < RMAX; ++r) {
            // computed for every row, kept only for real ones (a select, not
            // a branch: no wait at a join)
            u32x4 corner;
#pragma unroll
            for (int w = 0; w < 4; ++w) {
                const uint32_t m = neg_mask<E>(qf[r][w]);
                corner[w] = (lo[i][w] & m) | (hi[i][w] & ~m);
            }
            const float v = group_sum<LPT>(dot_chunk<E>(corner, qf[r], 0.0f));
            best = r < R ? fmaxf(best, v) : best;
        }
        if (sub == 0 && n < n1)
            srow[n] = in ? best * scale : -__builtin_inff();
    }
}

// Quest bound on the matrix cores (bf16).  Per element the bound takes
// q*hi where q >= 0 and q*lo where q < 0, which is q+ * hi + q- * lo with
// q+ = max(q, 0), q- = min(q, 0) (one of the two products is zero, and the
// other is exact in fp32).  So a block's bound for query row r is one dot
// product over 2D elements: the block's box as stored, [lo; hi], against
// [q-; q+] of the row, and a tile of 16 blocks x 16 query rows is a plain
// matrix product, 2D/32 v_mfma_f32_16x16x32_bf16 per tile.  Each wave reads
// its tile of 16 boxes (16 x 4D bytes) with fully coalesced 16-byte lane
// loads, stages it in its own LDS tile (rows padded by 16 bytes: both access
// patterns free of bank conflicts) and reads the B operand (block l%16,
// elements 32c + 8(l/16) .. +8) back from there; the A operand holds the
// same elements of [q-; q+] for query row 16t + l%16, built once from q.
// With the query tile as the product's left operand and the boxes as its
// right one, lane l holds the bounds of query rows 16t + 4(l/16) .. +4 for
// block l%16: the max over the group's rows is taken in the lane (and
// across the four 16-lane rows only when there are more than four query
// rows).  The vector kernel above spent as much time on its per-element
// selects and lane reductions as on its loads; with the boxes as the left
// operand the max over the rows cost four DPP steps per lane and score.
template <int D, int NT>
__global__ __launch_bounds__(64 * kQuestMfmaWaves) void score_quest_mfma_kernel(const uint8_t *__restrict__ q,
                                                               const uint8_t *__restrict__ meta,
                                                               const int32_t *__restrict__ seq_lens,
                                                               float *__restrict__ scores, int Hq, int Hkv, int NQ,
                                                               int T, int NB, float scale) {
    constexpr int KCH = 2 * D / 32;    // MFMA steps over the 2D elements of a box
    constexpr int BB = 4 * D;          // bytes of one box (lo and hi, bf16)
    constexpr int ROW = BB + 16;       // padded LDS row
    constexpr int LOADS = 16 * BB / 1024;  // 16-byte lane loads per tile
    constexpr int LPB = BB / 16;       // lanes per box in the coalesced layout
    __shared__ __attribute__((aligned(16))) uint8_t tile[kQuestMfmaWaves][16 * ROW];
    int row, wgp;
    xcd_row_part(row, wgp);
    const int b = row / Hkv, j = row - b * Hkv;
    const int G = Hq / Hkv;
    const int R = NQ * G;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int col = lane & 15, rsub = lane >> 4;
    uint8_t *my = tile[wave];

    // B operand: element e = 32c + 8*rsub + i of [q-; q+] for query row
    // 16t + col (rows past R: zeros, masked below).  Its loads go first
    // (unconditional), then the length, then the tile's box loads; the
    // operand is formed only once all of them are in flight.  (Formed
    // before the box loads, the compiler waited for the query before
    // issuing most of them, and each wave's tile arrived a full load
    // latency late.)
    constexpr int QL = D / 32;  // 16-byte query loads per lane and query tile
    u32x4 qv[NT][QL];
#pragma unroll
    for (int t = 0; t < NT; ++t) {
        const int rr = min(16 * t + col, R - 1);
        const int rq = rr / G, g = rr - rq * G;
        const uint8_t *qr = q + (((size_t)b * NQ + rq) * Hq + (size_t)j * G + g) * D * 2;
#pragma unroll
        for (int c = 0; c < QL; ++c)
            qv[t][c] = load16(qr + (32 * c + 8 * rsub) * 2);
    }
    const int len = min(max(seq_lens[b], 0), T);
    const int nvalid = nb_of(len);
    const uint8_t *mrow = meta + (size_t)row * NB * BB;
    float *srow = scores + (size_t)row * NB;
    const int n0 = (wgp * kQuestMfmaWaves + wave) * 16;  // this wave's tile of 16 boxes
    if (n0 >= NB)
        return;
    if (n0 >= nvalid) {  // uniform: no valid block in the tile
        if (lane < 16 && n0 + lane < NB)
            srow[n0 + lane] = -__builtin_inff();
        return;
    }
    u32x4 kv[LOADS];
    static_assert(64 % LPB == 0, "a lane reads the same 16 bytes of its box in every load");
    const uint32_t part = (uint32_t)(lane % LPB) * 16;
#pragma unroll
    for (int i = 0; i < LOADS; ++i) {
        const int bl = i * (64 / LPB) + lane / LPB;  // box of this lane's 16 bytes
        const uint32_t nb = (uint32_t)min(n0 + bl, NB - 1);  // a partial last tile re-reads the row's last box
        kv[i] = load_nt(mrow + (nb * (uint32_t)BB + part));  // a row's boxes span far less than 4 GiB
    }
    __builtin_amdgcn_sched_barrier(0);  // nothing below moves above the box loads
    // rows of a query tile past R hold row R - 1's query; their products
    // are never read (the maximum below skips them)
    u32x4 qf[NT][KCH];
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
        for (int c = 0; c < KCH; ++c) {
            const u32x4 v = qv[t][c % QL];
            u32x4 w;
#pragma unroll
            for (int x = 0; x < 4; ++x) {
                const uint32_t m = neg_mask<BF16>(v[x]);
                w[x] = c < QL ? (v[x] & m) : (v[x] & ~m);  // c < QL: q- (pairs with lo), else q+ (hi)
            }
            qf[t][c] = w;
        }
#pragma unroll
    for (int i = 0; i < LOADS; ++i) {
        const int bl = (i * 64 + lane) / LPB;
        *reinterpret_cast<u32x4 *>(my + bl * ROW + ((i * 64 + lane) % LPB) * 16) = kv[i];
    }
    __builtin_amdgcn_wave_barrier();
    u32x4 bf[KCH];
#pragma unroll
    for (int c = 0; c < KCH; ++c)
        bf[c] = *reinterpret_cast<const u32x4 *>(my + col * ROW + c * 64 + rsub * 16);
    // query rows x boxes: lane l holds the bounds of query rows
    // 16t + 4(l/16) .. +4 for block n0 + l%16
    float best = -__builtin_inff();
#pragma unroll
    for (int t = 0; t < NT; ++t) {
        f32x4 st = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int c = 0; c < KCH; ++c)
            st = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, qf[t][c]),
                                                          __builtin_bit_cast(bf16x8, bf[c]), st, 0, 0, 0);
#pragma unroll
        for (int i = 0; i < 4; ++i)
            best = 16 * t + 4 * rsub + i < R ? fmaxf(best, st[i]) : best;
    }
    if (R > 4)  // uniform: query rows in more than the first 16 lanes
        best = rows_max(best);
    if (lane < 16) {
        const int n = n0 + lane;
        if (n < NB)
            srow[n] = n < nvalid ? best * scale : -__builtin_inff();
    }
}

// Element-wise min / max of each block's valid keys (exact: the results are
// stored values).  One wave per block.
template <typename E, int D>
__global__ __launch_bounds__(256) void quest_meta_kernel(const uint8_t *__restrict__ keys,
                                                         const int32_t *__restrict__ seq_lens,
                                                         uint8_t *__restrict__ meta, int Hkv, int T, int NB) {
    constexpr int LPT = D * E::bytes / 16;
    constexpr int TPL = 64 / LPT;
    constexpr int LPB = 16 / TPL;
    const int row = blockIdx.y;
    const int b = row / Hkv;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int sub = lane % LPT, tg = lane / LPT;
    const int n = blockIdx.x * 4 + wave;
    if (n >= NB)
        return;
    const int len = min(max(seq_lens[b], 0), T);
    const size_t vec_bytes = (size_t)D * E::bytes;
    uint8_t *out = meta + ((size_t)row * NB + n) * 2 * vec_bytes;
    if (n >= nb_of(len)) {
        if (tg == 0) {
            store16(out + sub * 16, u32x4{0, 0, 0, 0});
            store16(out + vec_bytes + sub * 16, u32x4{0, 0, 0, 0});
        }
        return;
    }
    float lo[E::EPL], hi[E::EPL];
#pragma unroll
    for (int e = 0; e < E::EPL; ++e) {
        lo[e] = __builtin_inff();
        hi[e] = -__builtin_inff();
    }
    const uint8_t *krow = keys + (size_t)row * T * vec_bytes;
#pragma unroll
    for (int i = 0; i < LPB; ++i) {
        const int t = n * 16 + i * TPL + tg;
        if (t < len) {
            u32x4 v = load16(krow + (size_t)t * vec_bytes + sub * 16);
#pragma unroll
            for (int e = 0; e < E::EPL; ++e) {
                float x;
                if constexpr (E::bytes == 2)
                    x = (e & 1) ? bf16_hi(v[e >> 1]) : bf16_lo(v[e >> 1]);
                else
                    x = __uint_as_float(v[e]);
                lo[e] = fminf(lo[e], x);
                hi[e] = fmaxf(hi[e], x);
            }
        }
    }
    // combine the token groups of the wave (LPT-lane groups)
#pragma unroll
    for (int e = 0; e < E::EPL; ++e) {
        for (int off = LPT; off < 64; off <<= 1) {
            lo[e] = fminf(lo[e], __shfl_xor(lo[e], off));
            hi[e] = fmaxf(hi[e], __shfl_xor(hi[e], off));
        }
    }
    if (tg == 0) {
        u32x4 a, c;
        if constexpr (E::bytes == 2) {
#pragma unroll
            for (int w = 0; w < 4; ++w) {
                a[w] = (__float_as_uint(lo[2 * w]) >> 16) | (__float_as_uint(lo[2 * w + 1]) & 0xffff0000u);
                c[w] = (__float_as_uint(hi[2 * w]) >> 16) | (__float_as_uint(hi[2 * w + 1]) & 0xffff0000u);
            }
        } else {
#pragma unroll
            for (int w = 0; w < 4; ++w) {
                a[w] = __float_as_uint(lo[w]);
                c[w] = __float_as_uint(hi[w]);
            }
        }
        store16(out + sub * 16, a);
        store16(out + vec_bytes + sub * 16, c);
    }
}

// ------------------------------------------------------------------ launch
template <typename E, int D, int RMAX>
static hipError_t blockmax_t(const Dims &d, const void *q, int nq, const void *keys, const int32_t *lens,
                             float scale, float *scores, hipStream_t st) {
    const int per_wg = kScoreWaves * kScoreBlocksPerWave;
    dim3 grid((d.NB + per_wg - 1) / per_wg, d.rows());
    hipLaunchKernelGGL((score_blockmax_kernel<E, D, RMAX>), grid, dim3(kScoreThreads), 0, st, (const uint8_t *)q,
                       (const uint8_t *)keys, lens, scores, d.Hq, d.Hkv, nq, d.T, d.NB, scale);
    return hipGetLastError();
}

template <int D, int NT>
static hipError_t blockmax_mfma_t(const Dims &d, const void *q, int nq, const void *keys, const int32_t *lens,
                                  float scale, float *scores, hipStream_t st) {
    const int per_wg = kScoreWaves * mfma_blocks_per_wave<NT>();
    dim3 grid((d.NB + per_wg - 1) / per_wg, d.rows());
    hipLaunchKernelGGL((score_blockmax_mfma_kernel<D, NT>), grid, dim3(kScoreThreads), 0, st, (const uint8_t *)q,
                       (const uint8_t *)keys, lens, scores, d.Hq, d.Hkv, nq, d.T, d.NB, scale);
    return hipGetLastError();
}

// bf16 keys take the matrix-core kernel: measured on the 32K workload (4
// query rows) it streams faster than the vector kernel, and with 32 query
// rows (1M context, 4 drafts) the vector kernel is ALU-bound.  The A/B
// build (SKV_AB_VALU_BF16, see build.py --ab-valu) sends bf16 to the vector
// kernel instead, for the kernel-trace comparison only.
template <typename E, int D>
static hipError_t blockmax_r(const Dims &d, const void *q, int nq, const void *keys, const int32_t *lens,
                             float scale, float *scores, hipStream_t st) {
    const int R = nq * d.G();
#ifdef SKV_AB_VALU_BF16
    constexpr bool kMatrixCores = false;
#else
    constexpr bool kMatrixCores = E::bytes == 2;
#endif
    if constexpr (kMatrixCores) {
        return R <= 16 ? blockmax_mfma_t<D, 1>(d, q, nq, keys, lens, scale, scores, st)
                       : blockmax_mfma_t<D, 2>(d, q, nq, keys, lens, scale, scores, st);
    } else {
        if (R <= 4)
            return blockmax_t<E, D, 4>(d, q, nq, keys, lens, scale, scores, st);
        if (R <= 8)
            return blockmax_t<E, D, 8>(d, q, nq, keys, lens, scale, scores, st);
        if (R <= 16)
            return blockmax_t<E, D, 16>(d, q, nq, keys, lens, scale, scores, st);
        return blockmax_t<E, D, 32>(d, q, nq, keys, lens, scale, scores, st);
    }
}

// Achievable-read anchor (a measurement helper, not part of the step): the
// block scan's launch shape and load form -- (NB / 4) x rows workgroups of 4
// waves placed by xcd_row_part, each wave one 16-token block of BB bytes in
// 16-byte non-temporal lane loads, all of a wave's loads issued before any
// is used -- and nothing else but a XOR of what was read.  Its rate is the
// HBM read rate the scan's access pattern can reach on this chip.  The one
// store happens only for a XOR value the data almost never produce; it keeps
// the loads alive.
template <int BB>
__global__ __launch_bounds__(kScoreThreads) void stream_read_kernel(const uint8_t *__restrict__ keys, int NB,
                                                                    uint32_t *__restrict__ sink) {
    constexpr int LPB = BB / 1024;  // 16-byte lane loads per block
    int row, wgp;
    xcd_row_part(row, wgp);
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int n = wgp * kScoreWaves + wave;
    if (n >= NB)
        return;
    const uint8_t *p = keys + ((size_t)row * NB + n) * BB + lane * 16;
    u32x4 v[LPB];
#pragma unroll
    for (int i = 0; i < LPB; ++i)
        v[i] = load_nt(p + i * 1024);
    uint32_t x = 0;
#pragma unroll
    for (int i = 0; i < LPB; ++i)
        x ^= v[i][0] ^ v[i][1] ^ v[i][2] ^ v[i][3];
    if (x == 0x9e3779b9u)
        sink[0] = x;
}

hipError_t launch_stream_read(const Dims &d, const void *keys, uint32_t *sink, hipStream_t st) {
    dim3 grid((d.NB + kScoreWaves - 1) / kScoreWaves, d.rows());
    const int bb = 16 * d.D * d.elem_bytes();
    const uint8_t *k = (const uint8_t *)keys;
    if (bb == 2048)
        hipLaunchKernelGGL(stream_read_kernel<2048>, grid, dim3(kScoreThreads), 0, st, k, d.NB, sink);
    else if (bb == 4096)
        hipLaunchKernelGGL(stream_read_kernel<4096>, grid, dim3(kScoreThreads), 0, st, k, d.NB, sink);
    else
        hipLaunchKernelGGL(stream_read_kernel<8192>, grid, dim3(kScoreThreads), 0, st, k, d.NB, sink);
    return hipGetLastError();
}

hipError_t launch_score_blockmax(const Dims &d, const void *q, int nq, const void *keys, const int32_t *lens,
                                 float scale, float *scores, hipStream_t st) {
    if (d.dtype == 1)
        return d.D == 128 ? blockmax_r<BF16, 128>(d, q, nq, keys, lens, scale, scores, st)
                          : blockmax_r<BF16, 64>(d, q, nq, keys, lens, scale, scores, st);
    return d.D == 128 ? blockmax_r<F32, 128>(d, q, nq, keys, lens, scale, scores, st)
                      : blockmax_r<F32, 64>(d, q, nq, keys, lens, scale, scores, st);
}

template <typename E, int D, int RMAX>
static hipError_t quest_t(const Dims &d, const void *q, int nq, const void *meta, const int32_t *lens, float scale,
                          float *scores, hipStream_t st) {
    constexpr int LPT = D * E::bytes / 16;
    const int per_wg = kQuestWaves * (64 / LPT) * kQuestBlocksPerWave;
    dim3 grid((d.NB + per_wg - 1) / per_wg, d.rows());
    hipLaunchKernelGGL((score_quest_kernel<E, D, RMAX>), grid, dim3(kQuestThreads), 0, st, (const uint8_t *)q,
                       (const uint8_t *)meta, lens, scores, d.Hq, d.Hkv, nq, d.T, d.NB, scale);
    return hipGetLastError();
}

template <int D, int NT>
static hipError_t quest_mfma_t(const Dims &d, const void *q, int nq, const void *meta, const int32_t *lens,
                               float scale, float *scores, hipStream_t st) {
    const int per_wg = kQuestMfmaWaves * 16;
    dim3 grid((d.NB + per_wg - 1) / per_wg, d.rows());
    hipLaunchKernelGGL((score_quest_mfma_kernel<D, NT>), grid, dim3(64 * kQuestMfmaWaves), 0, st, (const uint8_t *)q,
                       (const uint8_t *)meta, lens, scores, d.Hq, d.Hkv, nq, d.T, d.NB, scale);
    return hipGetLastError();
}

// bf16 boxes take the matrix-core kernel (the A/B build sends them to the
// vector kernel, as for the block max).
template <typename E, int D>
static hipError_t quest_r(const Dims &d, const void *q, int nq, const void *meta, const int32_t *lens, float scale,
                          float *scores, hipStream_t st) {
    const int R = nq * d.G();
#ifdef SKV_AB_VALU_BF16
    constexpr bool kMatrixCores = false;
#else
    constexpr bool kMatrixCores = E::bytes == 2;
#endif
    if constexpr (kMatrixCores)
        return R <= 16 ? quest_mfma_t<D, 1>(d, q, nq, meta, lens, scale, scores, st)
                       : quest_mfma_t<D, 2>(d, q, nq, meta, lens, scale, scores, st);
    if (R <= 4)
        return quest_t<E, D, 4>(d, q, nq, meta, lens, scale, scores, st);
    if (R <= 8)
        return quest_t<E, D, 8>(d, q, nq, meta, lens, scale, scores, st);
    if (R <= 16)
        return quest_t<E, D, 16>(d, q, nq, meta, lens, scale, scores, st);
    return quest_t<E, D, 32>(d, q, nq, meta, lens, scale, scores, st);
}

hipError_t launch_score_quest(const Dims &d, const void *q, int nq, const void *meta, const int32_t *lens,
                              float scale, float *scores, hipStream_t st) {
    if (d.dtype == 1)
        return d.D == 128 ? quest_r<BF16, 128>(d, q, nq, meta, lens, scale, scores, st)
                          : quest_r<BF16, 64>(d, q, nq, meta, lens, scale, scores, st);
    return d.D == 128 ? quest_r<F32, 128>(d, q, nq, meta, lens, scale, scores, st)
                      : quest_r<F32, 64>(d, q, nq, meta, lens, scale, scores, st);
}

template <typename E, int D>
static hipError_t meta_t(const Dims &d, const void *keys, const int32_t *lens, void *meta, hipStream_t st) {
    dim3 grid((d.NB + 3) / 4, d.rows());
    hipLaunchKernelGGL((quest_meta_kernel<E, D>), grid, dim3(256), 0, st, (const uint8_t *)keys, lens,
                       (uint8_t *)meta, d.Hkv, d.T, d.NB);
    return hipGetLastError();
}

hipError_t launch_quest_meta(const Dims &d, const void *keys, const int32_t *lens, void *meta, hipStream_t st) {
    if (d.dtype == 1)
        return d.D == 128 ? meta_t<BF16, 128>(d, keys, lens, meta, st) : meta_t<BF16, 64>(d, keys, lens, meta, st);
    return d.D == 128 ? meta_t<F32, 128>(d, keys, lens, meta, st) : meta_t<F32, 64>(d, keys, lens, meta, st);
}

}  // namespace skv
