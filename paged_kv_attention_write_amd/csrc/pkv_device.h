// Device helpers for gfx950 (CDNA4, wave64): DPP row reductions, storage
// conversions and vector loads.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pkv {

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float float2_t __attribute__((ext_vector_type(2)));

// DPP controls (row = 16 lanes).
constexpr int kDppRowMirror = 0x140;      // lane i <- lane 15 - i
constexpr int kDppRowHalfMirror = 0x141;  // lane i <- lane 7 - i within each half row
constexpr int kDppQuadXor2 = 0x4E;        // quad_perm [2,3,0,1]
constexpr int kDppQuadXor1 = 0xB1;        // quad_perm [1,0,3,2]

template <int CTRL>
__device__ __forceinline__ float dpp_f32(float x) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, false));
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
