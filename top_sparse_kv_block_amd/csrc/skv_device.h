// Device-side helpers shared by the gfx950 kernels: element traits for
// float32 / bf16 storage, 16-byte vector loads, and wave64 cross-lane
// reductions built on DPP row operations (lanes are grouped in rows of 16).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

namespace skv {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

// Element storage traits.  EPL = elements in one 16-byte lane load.
struct F32 {
    static constexpr int bytes = 4;
    static constexpr int EPL = 4;
};
struct BF16 {
    static constexpr int bytes = 2;
    static constexpr int EPL = 8;
};

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// Streaming 16-byte load that should not displace reused lines.
__device__ __forceinline__ u32x4 load_nt(const void *p) {
    return __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(p));
}
__device__ __forceinline__ u32x4 load16(const void *p) { return *reinterpret_cast<const u32x4 *>(p); }
__device__ __forceinline__ void store16(void *p, u32x4 v) { *reinterpret_cast<u32x4 *>(p) = v; }

// Dot product of one 16-byte chunk of keys with the matching chunk of a
// query row, accumulated into acc.  bf16 uses the packed dot2 instruction
// (products of bf16 values are exact in fp32); float32 uses FMAs.
template <typename E> __device__ __forceinline__ float dot_chunk(u32x4 k, u32x4 q, float acc);

// The whole 16-byte vector is reinterpreted as 8 bf16 and split into pairs
// with shuffles.  (Bit-casting the individual 32-bit elements instead makes
// this compiler feed element 0 to all four dot2 instructions.)
template <> __device__ __forceinline__ float dot_chunk<BF16>(u32x4 k, u32x4 q, float acc) {
    const bf16x8 kb = __builtin_bit_cast(bf16x8, k), qb = __builtin_bit_cast(bf16x8, q);
    acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(kb, kb, 0, 1), __builtin_shufflevector(qb, qb, 0, 1),
                                          acc, false);
    acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(kb, kb, 2, 3), __builtin_shufflevector(qb, qb, 2, 3),
                                          acc, false);
    acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(kb, kb, 4, 5), __builtin_shufflevector(qb, qb, 4, 5),
                                          acc, false);
    acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(kb, kb, 6, 7), __builtin_shufflevector(qb, qb, 6, 7),
                                          acc, false);
    return acc;
}

template <> __device__ __forceinline__ float dot_chunk<F32>(u32x4 k, u32x4 q, float acc) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
        acc = __builtin_fmaf(__uint_as_float(k[i]), __uint_as_float(q[i]), acc);
    return acc;
}

// DPP controls (gfx9 encoding)
enum : int {
    DPP_QUAD_XOR1 = 0xB1,  // quad_perm [1,0,3,2]
    DPP_QUAD_XOR2 = 0x4E,  // quad_perm [2,3,0,1]
    DPP_ROW_ROR1 = 0x121,
    DPP_ROW_ROR2 = 0x122,
    DPP_ROW_ROR4 = 0x124,
    DPP_ROW_ROR8 = 0x128,
    DPP_ROW_HALF_MIRROR = 0x141,
};

template <int CTRL> __device__ __forceinline__ float dpp(float v) {
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xf, 0xf, false));
}

// Cross-row exchange in registers (gfx950 v_permlane16/32_swap): the pair
// returned holds this lane's value and that of lane l^16 (resp. l^32).
__device__ __forceinline__ float xor16_max(float v) {
    const auto p = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return fmaxf(__uint_as_float(p[0]), __uint_as_float(p[1]));
}
__device__ __forceinline__ float xor32_max(float v) {
    const auto p = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return fmaxf(__uint_as_float(p[0]), __uint_as_float(p[1]));
}
__device__ __forceinline__ float xor16_sum(float v) {
    const auto p = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return __uint_as_float(p[0]) + __uint_as_float(p[1]);
}
__device__ __forceinline__ float xor32_sum(float v) {
    const auto p = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return __uint_as_float(p[0]) + __uint_as_float(p[1]);
}

// Sum over aligned groups of L lanes (L = 8, 16 or 32); every lane of the
// group receives the group's total.  The order of the additions is fixed,
// so the result is deterministic.
template <int L> __device__ __forceinline__ float group_sum(float v);

template <> __device__ __forceinline__ float group_sum<16>(float v) {
    v += dpp<DPP_ROW_ROR8>(v);
    v += dpp<DPP_ROW_ROR4>(v);
    v += dpp<DPP_ROW_ROR2>(v);
    v += dpp<DPP_ROW_ROR1>(v);
    return v;
}

template <> __device__ __forceinline__ float group_sum<8>(float v) {
    v += dpp<DPP_ROW_HALF_MIRROR>(v);
    v += dpp<DPP_QUAD_XOR2>(v);
    v += dpp<DPP_QUAD_XOR1>(v);
    return v;
}

template <> __device__ __forceinline__ float group_sum<32>(float v) { return xor16_sum(group_sum<16>(v)); }

// max / sum across the lanes l, l^16, l^32, l^48 (the four rows of the wave)
__device__ __forceinline__ float rows_max(float v) { return xor32_max(xor16_max(v)); }
__device__ __forceinline__ float rows_sum(float v) { return xor32_sum(xor16_sum(v)); }

// max over the whole wave (all lanes receive it)
__device__ __forceinline__ float wave_max(float v) {
    v = fmaxf(v, dpp<DPP_ROW_ROR8>(v));
    v = fmaxf(v, dpp<DPP_ROW_ROR4>(v));
    v = fmaxf(v, dpp<DPP_ROW_ROR2>(v));
    v = fmaxf(v, dpp<DPP_ROW_ROR1>(v));
    return rows_max(v);
}

// min / max of an unsigned value over the whole wave (all lanes receive it)
template <bool MAX> __device__ __forceinline__ uint32_t wave_minmax_u32(uint32_t v) {
    auto pick = [](uint32_t a, uint32_t b) { return MAX ? (a > b ? a : b) : (a < b ? a : b); };
    v = pick(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, DPP_ROW_ROR8, 0xf, 0xf, false));
    v = pick(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, DPP_ROW_ROR4, 0xf, 0xf, false));
    v = pick(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, DPP_ROW_ROR2, 0xf, 0xf, false));
    v = pick(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, DPP_ROW_ROR1, 0xf, 0xf, false));
    auto p = __builtin_amdgcn_permlane16_swap(v, v, false, false);
    v = pick(p[0], p[1]);
    p = __builtin_amdgcn_permlane32_swap(v, v, false, false);
    return pick(p[0], p[1]);
}
__device__ __forceinline__ uint32_t wave_min_u32(uint32_t v) { return wave_minmax_u32<false>(v); }
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) { return wave_minmax_u32<true>(v); }

// Inclusive prefix sum over the 64 lanes of a wave with DPP row shifts and
// row broadcasts (no LDS round trips).
template <int CTRL, int ROWMASK> __device__ __forceinline__ uint32_t dpp_zero(uint32_t v) {
    return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, ROWMASK, 0xf, false);
}
__device__ __forceinline__ uint32_t wave_incl_scan(uint32_t v) {
    v += dpp_zero<0x111, 0xf>(v);  // row_shr:1
    v += dpp_zero<0x112, 0xf>(v);  // row_shr:2
    v += dpp_zero<0x114, 0xf>(v);  // row_shr:4
    v += dpp_zero<0x118, 0xf>(v);  // row_shr:8
    v += dpp_zero<0x142, 0xa>(v);  // row_bcast:15 into rows 1 and 3
    v += dpp_zero<0x143, 0xc>(v);  // row_bcast:31 into rows 2 and 3
    return v;
}

// Every lane of a 16-lane row gets lane N of that row (DPP row_newbcast).
template <int N> __device__ __forceinline__ float row_bcast(float v) {
    static_assert(N >= 0 && N < 16, "lane within a row");
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x150 + N, 0xf, 0xf,
                                                                 false));
}

// Calls f(std::integral_constant<int, i>) for i = I .. N-1 (compile-time lane
// or head indices for DPP controls).
template <int I, int N> struct StaticFor {
    template <typename F> __device__ __forceinline__ static void run(F &&f) {
        f(std::integral_constant<int, I>{});
        StaticFor<I + 1, N>::run(f);
    }
};
template <int N> struct StaticFor<N, N> {
    template <typename F> __device__ __forceinline__ static void run(F &&) {}
};

// fast exp2 for arguments <= 0 (v_exp_f32; results below the smallest
// normal flush to zero, which is what the softmax wants)
__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ int nb_of(int len) { return (len + 15) >> 4; }

// Workgroup barrier that orders LDS accesses only: each wave waits for its
// own LDS operations, not for its global loads and stores, so global loads
// issued before it stay in flight across it.  For barriers whose only
// purpose is to share LDS data (the row routines' scans and histograms).
__device__ __forceinline__ void lds_barrier() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// (row, part) handled by this workgroup of a (parts x rows) grid.  The
// dispatcher deals workgroups to the 8 XCDs in turn, so with rows % 8 == 0
// the parts of one row are laid out 8 apart in dispatch order: they run on
// one XCD and share its L2 (the row's scores, slot state and partials
// written by one kernel are then read from that L2 by the next, whose
// workgroups follow the same rule).  Any other row count is row-major.
// Only the placement depends on this; every mapping is a bijection.
__device__ __forceinline__ void xcd_row_part(int &row, int &part) {
    const int parts = gridDim.x, rows = gridDim.y;
    const int L = blockIdx.y * parts + blockIdx.x;  // dispatch order
    if ((rows & 7) == 0) {
        const int x = L & 7, r8 = L >> 3;
        row = 8 * (r8 / parts) + x;
        part = r8 - (r8 / parts) * parts;
    } else {
        row = blockIdx.y;
        part = blockIdx.x;
    }
}

}  // namespace skv
