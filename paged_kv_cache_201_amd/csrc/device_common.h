// Device helpers for gfx950 (CDNA4, wave64): cross-lane XOR shuffles built
// from DPP, bf16 / fp8 packing, and small vector types.
#pragma once

#include <hip/hip_runtime.h>
#include <cstdint>
#include <type_traits>
#include <utility>

namespace pkv {

// Compile-time loop: f(std::integral_constant<int, I>{}) for I = 0..N-1.
template <typename F, int... I>
__device__ __forceinline__ void static_for_impl(F&& f, std::integer_sequence<int, I...>) {
    (f(std::integral_constant<int, I>{}), ...);
}
template <int N, typename F>
__device__ __forceinline__ void static_for(F&& f) {
    static_for_impl(f, std::make_integer_sequence<int, N>{});
}

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

// Explicit global-memory (address space 1) pointers, for loads whose base is
// computed in scalar registers.
typedef const char __attribute__((address_space(1)))* gbytes_t;

__device__ __forceinline__ gbytes_t as_global(const void* p) { return (gbytes_t)p; }

template <typename T>
__device__ __forceinline__ T load_global(gbytes_t p) {
    return *(const T __attribute__((address_space(1)))*)p;
}

// Streaming load: the data is used once, so mark it non-temporal.
template <typename T>
__device__ __forceinline__ T load_global_stream(gbytes_t p) {
    return __builtin_nontemporal_load((const T __attribute__((address_space(1)))*)p);
}

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// ---------------------------------------------------------------------------
// XOR shuffles.  lane ^ M for M < 16 stays inside a DPP row of 16 lanes.
// Directly available: 1, 2, 3 (quad_perm), 7 (row_half_mirror), 8
// (row_ror:8), 15 (row_mirror); every other M < 16 is one of those XOR one of
// {1, 2, 3}, so it takes two DPP moves.  Masks with bit 4 or 5 set add one
// ds_bpermute for the bits that cross rows.
// ---------------------------------------------------------------------------
template <int CTRL>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t x) {
    return (uint32_t)__builtin_amdgcn_mov_dpp((int)x, CTRL, 0xF, 0xF, true);
}

template <int M>
__device__ __forceinline__ uint32_t xor_shfl_u32(uint32_t x) {
    static_assert(M >= 0 && M < 64, "lane mask");
    if constexpr (M == 0) {
        return x;
    } else if constexpr (M >= 16) {
        const int lane = __lane_id();
        const uint32_t y = xor_shfl_u32<(M & 15)>(x);
        return (uint32_t)__builtin_amdgcn_ds_bpermute(((lane ^ (M & 48)) << 2), (int)y);
    } else if constexpr (M == 1) {
        return dpp_u32<0xB1>(x);           // quad_perm [1,0,3,2]
    } else if constexpr (M == 2) {
        return dpp_u32<0x4E>(x);           // quad_perm [2,3,0,1]
    } else if constexpr (M == 3) {
        return dpp_u32<0x1B>(x);           // quad_perm [3,2,1,0]
    } else if constexpr (M == 7) {
        return dpp_u32<0x141>(x);          // row_half_mirror
    } else if constexpr (M == 8) {
        return dpp_u32<0x128>(x);          // row_ror:8
    } else if constexpr (M == 15) {
        return dpp_u32<0x140>(x);          // row_mirror
    } else if constexpr ((M ^ 7) < 4) {
        return xor_shfl_u32<(M ^ 7)>(dpp_u32<0x141>(x));
    } else if constexpr ((M ^ 8) < 4) {
        return xor_shfl_u32<(M ^ 8)>(dpp_u32<0x128>(x));
    } else {
        return xor_shfl_u32<(M ^ 15)>(dpp_u32<0x140>(x));
    }
}

template <int M>
__device__ __forceinline__ float xor_shfl(float x) {
    return __uint_as_float(xor_shfl_u32<M>(__float_as_uint(x)));
}

// ---------------------------------------------------------------------------
// Reduction bases.  A row of LPH lanes is reduced with a sequence of XOR
// partner masks whose highest set bits are distinct (a triangular basis of
// the lane index space), chosen so that each is one DPP move.
// ---------------------------------------------------------------------------
template <int LPH>
struct LaneBasis;
template <>
struct LaneBasis<4> {
    static constexpr int n = 2;
    static constexpr int m[5] = {2, 1, 0, 0, 0};
};
template <>
struct LaneBasis<8> {
    static constexpr int n = 3;
    static constexpr int m[5] = {7, 2, 1, 0, 0};
};
template <>
struct LaneBasis<16> {
    static constexpr int n = 4;
    static constexpr int m[5] = {8, 7, 2, 1, 0};
};
template <>
struct LaneBasis<32> {
    static constexpr int n = 5;
    static constexpr int m[5] = {16, 8, 7, 2, 1};
};

constexpr int highest_bit(int x) {
    int h = -1;
    while (x) {
        x >>= 1;
        ++h;
    }
    return h;
}

constexpr int ilog2(int x) { return highest_bit(x); }

// Coordinates of lane index l (within its row) in the basis: bit s of the
// result is the coefficient of basis mask s.
template <int LPH>
__host__ __device__ constexpr int basis_coords(int l) {
    int c = 0;
    for (int s = 0; s < LaneBasis<LPH>::n; ++s) {
        const int m = LaneBasis<LPH>::m[s];
        if ((l >> highest_bit(m)) & 1) {
            c |= 1 << s;
            l ^= m;
        }
    }
    return c;
}

// The first S = log2(G) basis masks split G per-lane partial sums across the
// row (a reduce-scatter); the remaining masks all-reduce.  Afterwards lane l
// holds the sum for value index head_of_lane(l); before, its value slot u
// must hold the partial for index u ^ head_of_lane(l).
template <int LPH, int G>
__host__ __device__ constexpr int head_of_lane(int l) {
    constexpr int S = ilog2(G);
    const int c = basis_coords<LPH>(l);
    int f = 0;
    for (int s = 0; s < S; ++s)
        if ((c >> s) & 1) f |= 1 << (S - 1 - s);
    return f;
}

// Lane mask that reaches, from lane l, a lane whose head is head_of_lane(l) ^ u.
template <int LPH, int G>
__host__ __device__ constexpr int lane_mask_for_head_xor(int u) {
    constexpr int S = ilog2(G);
    int m = 0;
    for (int s = 0; s < S; ++s)
        if ((u >> (S - 1 - s)) & 1) m ^= LaneBasis<LPH>::m[s];
    return m;
}

// Reduce-scatter + all-reduce of G partial sums over a row of LPH lanes
// (G <= LPH).  v[u] on entry: this lane's partial for index u ^ head_of_lane.
// Returns the row total for index head_of_lane(lane).
template <int LPH, int G>
__device__ __forceinline__ float row_reduce_scatter(float (&v)[G]) {
    static_assert(G <= LPH, "one value per lane after the scatter");
    constexpr int S = ilog2(G);
    constexpr int N = LaneBasis<LPH>::n;
    static_for<S>([&](auto sc) {
        constexpr int s = decltype(sc)::value;
        constexpr int half = G >> (s + 1);
        constexpr int M = LaneBasis<LPH>::m[s];
#pragma unroll
        for (int i = 0; i < half; ++i) v[i] += xor_shfl<M>(v[i + half]);
    });
    float x = v[0];
    static_for<N - S>([&](auto sc) {
        constexpr int M = LaneBasis<LPH>::m[S + decltype(sc)::value];
        x += xor_shfl<M>(x);
    });
    return x;
}

// ---------------------------------------------------------------------------
// Conversions.
// ---------------------------------------------------------------------------
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    f32x2_t f = {lo, hi};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f, bf16x2_t));
}

__device__ __forceinline__ uint16_t to_bf16_bits(float x) {
    return __builtin_bit_cast(uint16_t, (__bf16)x);
}

__device__ __forceinline__ float bf16_lo(uint32_t x) { return __uint_as_float(x << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t x) { return __uint_as_float(x & 0xFFFF0000u); }

// two fp8 e4m3 codes (bytes 0,1 or 2,3 of x) -> bf16x2, exact
template <bool HI>
__device__ __forceinline__ uint32_t fp8x2_to_bf16x2(uint32_t x) {
    return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)x, 1.0f, HI));
}

// a.lo*b.lo + a.hi*b.hi with a zero accumulator, as the three-operand VOP3P
// form: the two-operand accumulate form would need the destination zeroed
// by a separate move first.
__device__ __forceinline__ float dot2_bf16_first(uint32_t a, uint32_t b) {
    float r;
    asm("v_dot2_f32_bf16 %0, %1, %2, 0" : "=v"(r) : "v"(a), "v"(b));
    return r;
}

// sum of a.lo*b.lo + a.hi*b.hi + c, bf16 pairs with fp32 accumulation
__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float c) {
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a),
                                           __builtin_bit_cast(bf16x2_t, b), c, false);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float fast_log2(float x) { return __builtin_amdgcn_logf(x); }

}  // namespace pkv
