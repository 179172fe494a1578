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
// row, head): the parts' lse values (log2 units, wave-uniform: scalar loads)
// and each lane's D/64 elements of every part are loaded together, up to
// kMergeBatch parts at a time, so a record of up to that many parts costs one
// round trip to memory; batches combine by an online log-sum-exp.  Grid:
// (merge record, row of the record, group of kMergeWaves heads).
constexpr int kMergeWaves = 4;
constexpr int kMergeBatch = 8;

template <int QDT, int D>
__global__ __launch_bounds__(kMergeWaves * 64) void merge_kernel(const Merge* __restrict__ merges,
                                                                 const float* __restrict__ po,
                                                                 const float* __restrict__ pl,
                                                                 void* __restrict__ out, int hq, float v_scale) {
    constexpr int E = D / 64;  // elements per lane
    constexpr int B = kMergeBatch;
    const const_ptr<int32_t> mw = reinterpret_cast<const_ptr<int32_t>>(as_const(merges) + blockIdx.x);
    const int row0 = mw[0], nrows = mw[1], prow0 = mw[2], parts = mw[3];
    const int r = blockIdx.y;
    const int lane = threadIdx.x & 63;
    const int h = blockIdx.z * kMergeWaves + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    if (h >= hq || r >= nrows) return;
    const int64_t hd = static_cast<int64_t>(hq) * D;
    const const_ptr<float> lse = as_const(pl);
    float M = -INFINITY;  // running maximum of the lse values seen
    float sw = 0.f;       // sum of 2^(lse - M)
    float acc[E];
#pragma unroll
    for (int e = 0; e < E; ++e) acc[e] = 0.f;
    bool nan = false;
    for (int c0 = 0; c0 < parts; c0 += B) {
        float l[B];
        float x[B][E];
#pragma unroll
        for (int b = 0; b < B; ++b) {
            const int64_t prow = prow0 + static_cast<int64_t>(min(c0 + b, parts - 1)) * nrows + r;
            l[b] = lse[prow * hq + h];
            const float* src = po + prow * hd + static_cast<int64_t>(h) * D + lane * E;
#pragma unroll
            for (int e = 0; e < E; ++e) x[b][e] = src[e];
        }
        float mb = M;
#pragma unroll
        for (int b = 0; b < B; ++b) {
            if (c0 + b >= parts) l[b] = -INFINITY;  // a repeated last part counts once
            nan |= l[b] != l[b];
            mb = fmaxf(mb, l[b]);
        }
        if (mb == -INFINITY) continue;  // every part so far is empty
        const float f = exp2_fast(M - mb);  // 0 while M is -inf
        sw *= f;
#pragma unroll
        for (int e = 0; e < E; ++e) acc[e] *= f;
#pragma unroll
        for (int b = 0; b < B; ++b) {
            const float w = exp2_fast(l[b] - mb);  // 0 for an empty part
            sw += w;
#pragma unroll
            for (int e = 0; e < E; ++e) acc[e] = fmaf(w, x[b][e], acc[e]);
        }
        M = mb;
    }
    const float scale = sw > 0.f ? v_scale / sw : 0.f;
    float o[E];
#pragma unroll
    for (int e = 0; e < E; ++e) o[e] = nan ? NAN : acc[e] * scale;
    const int64_t oi = static_cast<int64_t>(row0 + r) * hd + static_cast<int64_t>(h) * D + lane * E;
    if constexpr (QDT == PKV_DTYPE_F32) {
#pragma unroll
        for (int e = 0; e < E; ++e) static_cast<float*>(out)[oi + e] = o[e];
    } else {
#pragma unroll
        for (int e = 0; e < E; ++e) static_cast<uint16_t*>(out)[oi + e] = static_cast<uint16_t>(f32_to_bf16_rne(o[e]));
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
