// Device helpers for gfx950 (CDNA4, wave64): DPP row reductions, storage
// conversions and vector loads.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <utility>

namespace pkv {

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float float2_t __attribute__((ext_vector_type(2)));

// Compile-time loop: f(std::integral_constant<int, i>) for i = 0 .. N-1.
template <int N, typename F>
__device__ __forceinline__ void static_for(F&& f) {
    [&]<int... I>(std::integer_sequence<int, I...>) { (f(std::integral_constant<int, I>{}), ...); }(
        std::make_integer_sequence<int, N>{});
}

// DPP controls (row = 16 lanes).
constexpr int kDppRowMirror = 0x140;      // lane i <- lane 15 - i
constexpr int kDppRowHalfMirror = 0x141;  // lane i <- lane 7 - i within each half row (i ^ 7)
constexpr int kDppQuadXor2 = 0x4E;        // quad_perm [2,3,0,1]
constexpr int kDppQuadXor1 = 0xB1;        // quad_perm [1,0,3,2]
constexpr int kDppRowRor = 0x120;         // + n (rotate right): lane i <- lane (i - n) mod 16
constexpr int kDppRowNewBcast = 0x150;    // + n: every lane of the row <- lane n of the row

template <int CTRL>
__device__ __forceinline__ float dpp_f32(float x) {
    return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), CTRL, 0xF, 0xF, true));
}

// Sum over the 16 lanes of each row; every lane of the row gets the total.
// mirror, half-mirror, xor 2, xor 1: each step pairs classes of lanes that
// have not been added yet, so four steps cover all sixteen.
__device__ __forceinline__ float row16_sum(float x) {
    x += dpp_f32<kDppRowMirror>(x);
    x += dpp_f32<kDppRowHalfMirror>(x);
    x += dpp_f32<kDppQuadXor2>(x);
    x += dpp_f32<kDppQuadXor1>(x);
    return x;
}

// Broadcast lane N of each row to the whole row.
template <int N>
__device__ __forceinline__ float row_bcast(float x) {
    return dpp_f32<kDppRowNewBcast + N>(x);
}

// Butterfly reduce-scatter over the 16 lanes of a row: on entry every lane
// holds 16 partial sums a[v]; on return lane c holds the row's total of
// a[c].  Step k pairs each lane with one that differs in bit 3-k of its
// index (ror 8 = xor 8, half mirror = xor 7, xor 2, xor 1).  The first step
// adds both halves across the pair and then keeps the half selected by bit 3;
// each later step keeps the half selected by its bit and adds the partner's
// copy of that half.
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef float f32x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

// Per-lane select: m all ones -> x_set, all zeros -> x_clear.  One v_bfi_b32
// with the mask in a VGPR, so that the compiler cannot turn the selects of
// the butterfly below into dynamically indexed vector reads.  Two rules for
// its callers, both about what the compiler cannot see inside inline asm:
// the mask is a per-lane 32-bit value (a 64-bit lane-mask constant handed
// over as an SGPR pair has been materialised with only its low word set), and
// no operand may come straight from a v_dot* (the wait states a dot result
// needs before another VALU reads it are not inserted for an asm reader).
__device__ __forceinline__ float lane_select(float x_clear, float x_set, uint32_t m) {
    uint32_t r;
    asm("v_bfi_b32 %0, %1, %2, %3" : "=v"(r) : "v"(m), "v"(__float_as_uint(x_set)), "v"(__float_as_uint(x_clear)));
    return __uint_as_float(r);
}

// All ones in the lanes whose index within the 16-lane row has bit K set.
template <int K>
__device__ __forceinline__ uint32_t row_bit_mask() {
    return 0u - ((__lane_id() >> K) & 1u);
}

__device__ __forceinline__ float row16_reduce_scatter(const f32x16_t a) {
    const uint32_t m3 = row_bit_mask<3>();
    const uint32_t m2 = row_bit_mask<2>();
    const uint32_t m1 = row_bit_mask<1>();
    const uint32_t m0 = row_bit_mask<0>();
    f32x8_t s1;
    static_for<8>([&](auto jc) {
        constexpr int j = decltype(jc)::value;
        const float lo = a[j] + dpp_f32<kDppRowRor + 8>(a[j]);
        const float hi = a[j + 8] + dpp_f32<kDppRowRor + 8>(a[j + 8]);
        s1[j] = lane_select(lo, hi, m3);
    });
    f32x4_t s2;
    static_for<4>([&](auto jc) {
        constexpr int j = decltype(jc)::value;
        s2[j] = lane_select(s1[j], s1[j + 4], m2) + dpp_f32<kDppRowHalfMirror>(lane_select(s1[j + 4], s1[j], m2));
    });
    float2_t s3;
    static_for<2>([&](auto jc) {
        constexpr int j = decltype(jc)::value;
        s3[j] = lane_select(s2[j], s2[j + 2], m1) + dpp_f32<kDppQuadXor2>(lane_select(s2[j + 2], s2[j], m1));
    });
    return lane_select(s3[0], s3[1], m0) + dpp_f32<kDppQuadXor1>(lane_select(s3[1], s3[0], m0));
}

// Max / sum over the lanes of a row whose index is congruent mod STRIDE
// (STRIDE a power of two <= 8): rotations by STRIDE, 2 STRIDE, ... 8.
template <int STRIDE>
__device__ __forceinline__ float row_group_max(float x) {
    if constexpr (STRIDE <= 8) {
        x = fmaxf(x, dpp_f32<kDppRowRor + STRIDE>(x));
        if constexpr (STRIDE * 2 <= 8) return row_group_max<STRIDE * 2>(x);
    }
    return x;
}
template <int STRIDE>
__device__ __forceinline__ float row_group_sum(float x) {
    if constexpr (STRIDE <= 8) {
        x += dpp_f32<kDppRowRor + STRIDE>(x);
        if constexpr (STRIDE * 2 <= 8) return row_group_sum<STRIDE * 2>(x);
    }
    return x;
}

// Across the four rows of a wave (lanes i, i^16, i^32, i^48).
__device__ __forceinline__ float rows4_max(float x) {
    x = fmaxf(x, __shfl_xor(x, 16));
    x = fmaxf(x, __shfl_xor(x, 32));
    return x;
}
__device__ __forceinline__ float rows4_sum(float x) {
    x += __shfl_xor(x, 16);
    x += __shfl_xor(x, 32);
    return x;
}

__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

// bf16 halves of a 32-bit word as fp32 (exact).
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// fp32 -> bf16 bits, round to nearest even; NaN -> quiet NaN with its sign.
__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f) {
    const uint32_t u = __float_as_uint(f);
    if ((u & 0x7FFFFFFFu) > 0x7F800000u) return ((u >> 16) & 0x8000u) | 0x7FC0u;
    return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

// OCP E4M3 code of y: nearest value, ties to even, |y| >= 448 -> 448,
// NaN -> 0x7F.  Integer rounding of the fp32 fields.
__device__ __forceinline__ uint32_t f32_to_e4m3_sat(float y) {
    const uint32_t u = __float_as_uint(y);
    const uint32_t sign = (u >> 24) & 0x80u;
    const uint32_t mag = u & 0x7FFFFFFFu;
    if (mag > 0x7F800000u) return 0x7Fu;     // NaN
    if (mag >= 0x43E00000u) return sign | 0x7Eu;  // |y| >= 448 (and inf)
    if (mag < 0x3C800000u) {                 // |y| < 2^-6: subnormal codes m * 2^-9
        const float m = rintf(__uint_as_float(mag) * 512.0f);  // exact scale, ties to even
        return sign | static_cast<uint32_t>(m);                  // m == 8 is the smallest normal
    }
    uint32_t e = (mag >> 23) - 127u + 7u;    // 1 .. 15
    uint32_t keep = (mag >> 20) & 7u;        // top three mantissa bits
    const uint32_t rest = mag & 0xFFFFFu;    // 20 bits below them
    if (rest > 0x80000u || (rest == 0x80000u && (keep & 1u))) ++keep;
    if (keep == 8u) {
        keep = 0;
        ++e;
    }
    return sign | (e << 3) | keep;
}

// Read-only data the kernels never write (plan records, lengths, block
// tables) is read through the constant address space: uniform addresses then
// become scalar loads, which wait on their own counter instead of behind the
// K/V vector loads in flight.
template <typename T>
using const_ptr = const __attribute__((address_space(4))) T*;

template <typename T>
__device__ __forceinline__ const_ptr<T> as_const(const T* p) {
    return (const_ptr<T>)(p);
}

// Vector loads of N 32-bit words (N = 1, 2, 4, 8) from 4N-byte aligned memory.
template <int N>
struct Words {
    uint32_t w[N];
};

template <int N>
__device__ __forceinline__ Words<N> load_words(const void* p) {
    Words<N> r;
    if constexpr (N == 8) {
        const uint4 a = reinterpret_cast<const uint4*>(p)[0];
        const uint4 b = reinterpret_cast<const uint4*>(p)[1];
        r.w[0] = a.x; r.w[1] = a.y; r.w[2] = a.z; r.w[3] = a.w;
        r.w[4] = b.x; r.w[5] = b.y; r.w[6] = b.z; r.w[7] = b.w;
    } else if constexpr (N == 4) {
        const uint4 a = *reinterpret_cast<const uint4*>(p);
        r.w[0] = a.x; r.w[1] = a.y; r.w[2] = a.z; r.w[3] = a.w;
    } else if constexpr (N == 2) {
        const uint2 a = *reinterpret_cast<const uint2*>(p);
        r.w[0] = a.x; r.w[1] = a.y;
    } else {
        static_assert(N == 1, "1, 2, 4 or 8 words");
        r.w[0] = *reinterpret_cast<const uint32_t*>(p);
    }
    return r;
}

// Streaming variant: non-temporal loads for data read exactly once.
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

template <int N>
__device__ __forceinline__ Words<N> load_words_nt(const void* p) {
    Words<N> r;
    if constexpr (N == 8 || N == 4) {
#pragma unroll
        for (int h = 0; h < N / 4; ++h) {
            const u32x4_t a = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p) + h);
            r.w[4 * h] = a.x; r.w[4 * h + 1] = a.y; r.w[4 * h + 2] = a.z; r.w[4 * h + 3] = a.w;
        }
    } else if constexpr (N == 2) {
        const u32x2_t a = __builtin_nontemporal_load(reinterpret_cast<const u32x2_t*>(p));
        r.w[0] = a.x; r.w[1] = a.y;
    } else {
        r.w[0] = __builtin_nontemporal_load(reinterpret_cast<const uint32_t*>(p));
    }
    return r;
}

template <int N>
__device__ __forceinline__ void store_words(void* p, const Words<N>& r) {
    if constexpr (N == 8) {
        reinterpret_cast<uint4*>(p)[0] = make_uint4(r.w[0], r.w[1], r.w[2], r.w[3]);
        reinterpret_cast<uint4*>(p)[1] = make_uint4(r.w[4], r.w[5], r.w[6], r.w[7]);
    } else if constexpr (N == 4) {
        *reinterpret_cast<uint4*>(p) = make_uint4(r.w[0], r.w[1], r.w[2], r.w[3]);
    } else if constexpr (N == 2) {
        *reinterpret_cast<uint2*>(p) = make_uint2(r.w[0], r.w[1]);
    } else {
        static_assert(N == 1, "1, 2, 4 or 8 words");
        *reinterpret_cast<uint32_t*>(p) = r.w[0];
    }
}

}  // namespace pkv
