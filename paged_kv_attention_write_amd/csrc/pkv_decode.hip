// Paged decode attention and the merge of split pieces (gfx950).
//
// One workgroup per planner queue (persistent: it walks its queue's units
// with the decode unit), then the pieces of a cut sequence are merged by
// their log-sum-exp ("How Easy Is It to Start Serving LLMs?", Phase 4 §3).
#include "pkv_decode_unit.h"

namespace pkv {
namespace {

template <int QDT, int KVDT, int D, int G, int NW, bool UNIFORM_PAGE, int WPE>
__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(WPE)))
void decode_kernel(AttnArgs a) {
    __shared__ DecodeLds<D, G, NW> lds;
    const const_ptr<Unit> units = as_const(a.units);
    const const_ptr<int32_t> qoff = as_const(a.queue_off);
    const int u_begin = qoff[blockIdx.x];
    const int u_end = qoff[blockIdx.x + 1];
    for (int ui = u_begin; ui < u_end; ++ui) {
        const Unit un = load_unit(units, ui);
        decode_unit<QDT, KVDT, D, G, NW, UNIFORM_PAGE>(a, un, lds);
    }
}

// Merge of the partial results of cut sequences.  One wave per (merge record,
// row, head): lane c reads part c's lse (log2 units), a wave max and sum give
// the part weights w_c = 2^(lse_c - M) / sum, then every lane accumulates its
// D/64 elements over the parts with independent loads.  Grid: (merge record,
// row of the record, group of kMergeWaves heads).
constexpr int kMergeWaves = 4;

template <int QDT, int D>
__global__ __launch_bounds__(kMergeWaves * 64) void merge_kernel(const Merge* __restrict__ merges,
                                                                 const float* __restrict__ po,
                                                                 const float* __restrict__ pl,
                                                                 void* __restrict__ out, int hq, float v_scale) {
    constexpr int E = D / 64;  // elements per lane
    const Merge mg = merges[blockIdx.x];
    const int r = blockIdx.y;
    const int lane = threadIdx.x & 63;
    const int h = blockIdx.z * kMergeWaves + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    if (h >= hq || r >= mg.nrows) return;
    const int64_t hd = static_cast<int64_t>(hq) * D;
    {
        // weights of the parts, 64 at a time
        float M = -INFINITY;
        bool nan = false;
        for (int c0 = 0; c0 < mg.parts; c0 += 64) {
            const int c = c0 + lane;
            const float x = c < mg.parts ? pl[static_cast<int64_t>(mg.prow0 + c * mg.nrows + r) * hq + h] : -INFINITY;
            nan |= (x != x);
            M = fmaxf(M, x);
        }
        for (int o = 32; o >= 1; o >>= 1) M = fmaxf(M, __shfl_xor(M, o));
        nan = __any(nan);
        float acc[E];
#pragma unroll
        for (int e = 0; e < E; ++e) acc[e] = 0.f;
        float sw = 0.f;
        if (!nan && M != -INFINITY) {
            for (int c0 = 0; c0 < mg.parts; c0 += 64) {
                const int c = c0 + lane;
                const float w = c < mg.parts
                                    ? exp2_fast(pl[static_cast<int64_t>(mg.prow0 + c * mg.nrows + r) * hq + h] - M)
                                    : 0.f;
                float ws = w;
                for (int o = 32; o >= 1; o >>= 1) ws += __shfl_xor(ws, o);
                sw += ws;
                const int n = min(64, mg.parts - c0);
                int j = 0;
                for (; j + 4 <= n; j += 4) {
                    float v[4][E];
                    float wj[4];
#pragma unroll
                    for (int k = 0; k < 4; ++k) {
                        wj[k] = __shfl(w, j + k);
                        const float* src = po + static_cast<int64_t>(mg.prow0 + (c0 + j + k) * mg.nrows + r) * hd +
                                           static_cast<int64_t>(h) * D + lane * E;
#pragma unroll
                        for (int e = 0; e < E; ++e) v[k][e] = src[e];
                    }
#pragma unroll
                    for (int k = 0; k < 4; ++k)
#pragma unroll
                        for (int e = 0; e < E; ++e) acc[e] = fmaf(wj[k], v[k][e], acc[e]);
                }
                for (; j < n; ++j) {
                    const float wj = __shfl(w, j);
                    const float* src = po + static_cast<int64_t>(mg.prow0 + (c0 + j) * mg.nrows + r) * hd +
                                       static_cast<int64_t>(h) * D + lane * E;
#pragma unroll
                    for (int e = 0; e < E; ++e) acc[e] = fmaf(wj, src[e], acc[e]);
                }
            }
        }
        float o[E];
        const float scale = (sw > 0.f) ? v_scale / sw : 0.f;
#pragma unroll
        for (int e = 0; e < E; ++e) o[e] = nan ? NAN : acc[e] * scale;
        const int64_t oi = static_cast<int64_t>(mg.row0 + r) * hd + static_cast<int64_t>(h) * D + lane * E;
        if constexpr (QDT == PKV_DTYPE_F32) {
#pragma unroll
            for (int e = 0; e < E; ++e) static_cast<float*>(out)[oi + e] = o[e];
        } else {
#pragma unroll
            for (int e = 0; e < E; ++e) static_cast<uint16_t*>(out)[oi + e] = static_cast<uint16_t>(f32_to_bf16_rne(o[e]));
        }
    }
}

// Launch shape: one persistent workgroup per queue.  8 waves (one per kv head
// of the 8-head workloads) stream bf16 / fp32 K/V on whole-tile pages (one
// workgroup per CU: more loads in flight per CU lower the read rate of this
// pattern).  16 waves (two per kv head, alternate tiles, <= 128 VGPRs) hide
// the extra latency of per-token page lookups and the fp8 conversion work.
// Group 8 (eight q heads per lane), group 1 (sixteen tokens in flight per
// lane) and fp32 K/V need more registers and keep 8 waves at two waves per
// SIMD.
template <int QDT, int KVDT, int D, int G>
int launch_decode_t(const AttnArgs& a, int num_queues, bool uniform, hipStream_t st) {
    constexpr bool kSmallRegs = !(G == 8 || G == 1 || KVDT == PKV_DTYPE_F32);
    const dim3 grid(num_queues);
    if constexpr (kSmallRegs) {
        if constexpr (KVDT == PKV_DTYPE_FP8_E4M3) {
            if (uniform)
                hipLaunchKernelGGL((decode_kernel<QDT, KVDT, D, G, 16, true, 4>), grid, dim3(16 * 64), 0, st,
                                   a);
            else
                hipLaunchKernelGGL((decode_kernel<QDT, KVDT, D, G, 16, false, 4>), grid, dim3(16 * 64), 0, st,
                                   a);
        } else if (uniform) {
            hipLaunchKernelGGL((decode_kernel<QDT, KVDT, D, G, 8, true, 4>), grid, dim3(8 * 64), 0, st, a);
        } else {
            hipLaunchKernelGGL((decode_kernel<QDT, KVDT, D, G, 16, false, 4>), grid, dim3(16 * 64), 0, st, a);
        }
    } else {
        if (uniform)
            hipLaunchKernelGGL((decode_kernel<QDT, KVDT, D, G, 8, true, 2>), grid, dim3(8 * 64), 0, st, a);
        else
            hipLaunchKernelGGL((decode_kernel<QDT, KVDT, D, G, 8, false, 2>), grid, dim3(8 * 64), 0, st, a);
    }
    return hipGetLastError() == hipSuccess ? PKV_OK : PKV_ERR_HIP;
}

template <int QDT, int KVDT, int D>
int launch_decode_g(const AttnArgs& a, int group, int num_queues, bool uniform, hipStream_t st) {
    switch (group) {
        case 1: return launch_decode_t<QDT, KVDT, D, 1>(a, num_queues, uniform, st);
        case 2: return launch_decode_t<QDT, KVDT, D, 2>(a, num_queues, uniform, st);
        case 4: return launch_decode_t<QDT, KVDT, D, 4>(a, num_queues, uniform, st);
        case 8: return launch_decode_t<QDT, KVDT, D, 8>(a, num_queues, uniform, st);
        default: return PKV_ERR_UNSUPPORTED;
    }
}

template <int QDT, int KVDT>
int launch_decode_d(const AttnArgs& a, int d, int group, int num_queues, bool uniform, hipStream_t st) {
    if (d == 64) return launch_decode_g<QDT, KVDT, 64>(a, group, num_queues, uniform, st);
    if (d == 128) return launch_decode_g<QDT, KVDT, 128>(a, group, num_queues, uniform, st);
    return PKV_ERR_UNSUPPORTED;
}

}  // namespace

int launch_decode(const AttnArgs& a, int q_dtype, int kv_dtype, int head_dim, int group, int num_queues,
                  void* stream) {
    hipStream_t st = static_cast<hipStream_t>(stream);
    const bool uniform = (a.block_size % kTileTokens) == 0;
    if (q_dtype == PKV_DTYPE_F32 && kv_dtype == PKV_DTYPE_F32)
        return launch_decode_d<PKV_DTYPE_F32, PKV_DTYPE_F32>(a, head_dim, group, num_queues, uniform, st);
    if (q_dtype == PKV_DTYPE_BF16 && kv_dtype == PKV_DTYPE_BF16)
        return launch_decode_d<PKV_DTYPE_BF16, PKV_DTYPE_BF16>(a, head_dim, group, num_queues, uniform, st);
    if (q_dtype == PKV_DTYPE_BF16 && kv_dtype == PKV_DTYPE_FP8_E4M3)
        return launch_decode_d<PKV_DTYPE_BF16, PKV_DTYPE_FP8_E4M3>(a, head_dim, group, num_queues, uniform, st);
    return PKV_ERR_UNSUPPORTED;
}

int launch_merge(const AttnArgs& a, const Merge* merges, int num_merges, int max_rows, int q_dtype, int head_dim,
                 void* stream) {
    if (num_merges == 0) return PKV_OK;
    hipStream_t st = static_cast<hipStream_t>(stream);
    const dim3 grid(num_merges, max_rows, (a.hq + kMergeWaves - 1) / kMergeWaves);
    const dim3 block(kMergeWaves * 64);
    if (q_dtype == PKV_DTYPE_F32 && head_dim == 64)
        hipLaunchKernelGGL((merge_kernel<PKV_DTYPE_F32, 64>), grid, block, 0, st, merges, a.partial_o, a.partial_lse,
                           a.out, a.hq, a.v_scale);
    else if (q_dtype == PKV_DTYPE_F32)
        hipLaunchKernelGGL((merge_kernel<PKV_DTYPE_F32, 128>), grid, block, 0, st, merges, a.partial_o, a.partial_lse,
                           a.out, a.hq, a.v_scale);
    else if (head_dim == 64)
        hipLaunchKernelGGL((merge_kernel<PKV_DTYPE_BF16, 64>), grid, block, 0, st, merges, a.partial_o, a.partial_lse,
                           a.out, a.hq, a.v_scale);
    else
        hipLaunchKernelGGL((merge_kernel<PKV_DTYPE_BF16, 128>), grid, block, 0, st, merges, a.partial_o, a.partial_lse,
                           a.out, a.hq, a.v_scale);
    return hipGetLastError() == hipSuccess ? PKV_OK : PKV_ERR_HIP;
}

}  // namespace pkv
