// paged_kv_write: scatter this step's K/V rows into the block pool by slot.
//
// "nanoserve", "One engine step" (steps 2-3): each new token's cache slot is
// computed from its block table once per step and every layer writes the
// token's K/V there before attending; "How to design an LLM serving system",
// "PagedAttention": slot_mapping names the physical slot of each new token.
//
// One thread moves 8 consecutive elements of one (token, kv head) row: a
// 16-byte (bf16) or 32-byte (fp32) load and an 8/16/32-byte store, so a wave
// writes 64 x 8 contiguous elements of the destination slot's row.  The
// cache row of slot s starts at element s * H_kv * D.
#include "pkv_attention.h"

namespace pkv {
namespace {

template <int NEW_DT, int CACHE_DT>
__device__ __forceinline__ Words<dt_bytes(CACHE_DT) * 2> convert8(const Words<dt_bytes(NEW_DT) * 2>& in,
                                                                    float scale) {
    constexpr int NI = dt_bytes(NEW_DT) * 2;
    constexpr int NO = dt_bytes(CACHE_DT) * 2;
    Words<NO> out;
    if constexpr (NEW_DT == CACHE_DT) {
#pragma unroll
        for (int i = 0; i < NI; ++i) out.w[i] = in.w[i];
    } else {
        float x[8];
        if constexpr (NEW_DT == PKV_DTYPE_F32) {
#pragma unroll
            for (int i = 0; i < 8; ++i) x[i] = __uint_as_float(in.w[i]);
        } else {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                x[2 * i] = bf16_lo(in.w[i]);
                x[2 * i + 1] = bf16_hi(in.w[i]);
            }
        }
        if constexpr (CACHE_DT == PKV_DTYPE_BF16) {
#pragma unroll
            for (int i = 0; i < 4; ++i) out.w[i] = f32_to_bf16_rne(x[2 * i]) | (f32_to_bf16_rne(x[2 * i + 1]) << 16);
        } else {
            static_assert(CACHE_DT == PKV_DTYPE_FP8_E4M3, "fp8 cache");
            uint32_t c[8];
#pragma unroll
            for (int i = 0; i < 8; ++i) c[i] = f32_to_e4m3_sat(x[i] / scale);  // IEEE fp32 division
            out.w[0] = c[0] | (c[1] << 8) | (c[2] << 16) | (c[3] << 24);
            out.w[1] = c[4] | (c[5] << 8) | (c[6] << 16) | (c[7] << 24);
        }
    }
    return out;
}

template <int NEW_DT, int CACHE_DT>
__global__ __launch_bounds__(256) void kv_write_kernel(const char* __restrict__ k_new, const char* __restrict__ v_new,
                                                       int64_t new_stride_bytes, const int32_t* __restrict__ slots,
                                                       int64_t num_tokens, char* __restrict__ k_cache,
                                                       char* __restrict__ v_cache, int64_t num_slots,
                                                       int32_t chunks_per_token, float k_scale, float v_scale) {
    constexpr int NI = dt_bytes(NEW_DT) * 2;   // words of 8 new elements
    constexpr int NO = dt_bytes(CACHE_DT) * 2; // words of 8 cache elements
    const int64_t idx = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
    const int64_t t = idx / chunks_per_token;
    if (t >= num_tokens) return;
    const int32_t c = static_cast<int32_t>(idx - t * chunks_per_token);
    const int64_t slot = slots[t];
    if (slot < 0 || slot >= num_slots) return;
    const int64_t row_elems = static_cast<int64_t>(chunks_per_token) * 8;
    const int64_t src = t * new_stride_bytes + static_cast<int64_t>(c) * 8 * dt_bytes(NEW_DT);
    const int64_t dst = (slot * row_elems + static_cast<int64_t>(c) * 8) * dt_bytes(CACHE_DT);
    const Words<NI> kin = load_words<NI>(k_new + src);
    const Words<NI> vin = load_words<NI>(v_new + src);
    store_words<NO>(k_cache + dst, convert8<NEW_DT, CACHE_DT>(kin, k_scale));
    store_words<NO>(v_cache + dst, convert8<NEW_DT, CACHE_DT>(vin, v_scale));
}

template <int NEW_DT, int CACHE_DT>
int launch(const void* k_new, const void* v_new, int64_t stride_elems, const int32_t* slots, int64_t T,
           void* kc, void* vc, int64_t num_slots, int32_t hd, float ks, float vs, hipStream_t stream) {
    const int32_t cpt = hd / 8;
    const int64_t threads = T * cpt;
    const int64_t blocks = (threads + 255) / 256;
    if (blocks > 0x7FFFFFFF) return PKV_ERR_SHAPE;
    hipLaunchKernelGGL((kv_write_kernel<NEW_DT, CACHE_DT>), dim3(static_cast<uint32_t>(blocks)), dim3(256), 0, stream,
                       static_cast<const char*>(k_new), static_cast<const char*>(v_new),
                       stride_elems * dt_bytes(NEW_DT), slots, T, static_cast<char*>(kc), static_cast<char*>(vc),
                       num_slots, cpt, ks, vs);
    return hipGetLastError() == hipSuccess ? PKV_OK : PKV_ERR_HIP;
}

}  // namespace

int launch_kv_write(const void* k_new, const void* v_new, int32_t new_dtype, int64_t stride_elems,
                    const int32_t* slots, int64_t T, void* kc, void* vc, int32_t cache_dtype, int64_t num_slots,
                    int32_t hd, float ks, float vs, void* stream) {
    hipStream_t st = static_cast<hipStream_t>(stream);
    if (new_dtype == PKV_DTYPE_F32 && cache_dtype == PKV_DTYPE_F32)
        return launch<PKV_DTYPE_F32, PKV_DTYPE_F32>(k_new, v_new, stride_elems, slots, T, kc, vc, num_slots, hd, ks, vs, st);
    if (new_dtype == PKV_DTYPE_BF16 && cache_dtype == PKV_DTYPE_BF16)
        return launch<PKV_DTYPE_BF16, PKV_DTYPE_BF16>(k_new, v_new, stride_elems, slots, T, kc, vc, num_slots, hd, ks, vs, st);
    if (new_dtype == PKV_DTYPE_F32 && cache_dtype == PKV_DTYPE_BF16)
        return launch<PKV_DTYPE_F32, PKV_DTYPE_BF16>(k_new, v_new, stride_elems, slots, T, kc, vc, num_slots, hd, ks, vs, st);
    if (new_dtype == PKV_DTYPE_BF16 && cache_dtype == PKV_DTYPE_FP8_E4M3)
        return launch<PKV_DTYPE_BF16, PKV_DTYPE_FP8_E4M3>(k_new, v_new, stride_elems, slots, T, kc, vc, num_slots, hd, ks, vs, st);
    if (new_dtype == PKV_DTYPE_F32 && cache_dtype == PKV_DTYPE_FP8_E4M3)
        return launch<PKV_DTYPE_F32, PKV_DTYPE_FP8_E4M3>(k_new, v_new, stride_elems, slots, T, kc, vc, num_slots, hd, ks, vs, st);
    return PKV_ERR_UNSUPPORTED;
}

}  // namespace pkv
