// Paged decode attention and the merge of split pieces (gfx950).
//
// One workgroup per planner queue (persistent: it walks its queue's units
// with the decode unit), then the pieces of a cut sequence are merged by
// their log-sum-exp ("How Easy Is It to Start Serving LLMs?", Phase 4 §3).
#include "pkv_decode_unit.h"

namespace pkv {
namespace {

template <int QDT, int KVDT, int D, int G, int NW, int PK, int WPE, bool WR = false>
__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(WPE)))
void decode_kernel(AttnArgs a) {
    __shared__ DecodeLds<D, G, NW> lds;
    const const_ptr<Unit> units = as_const(a.units);
    const const_ptr<int32_t> qoff = as_const(a.queue_off);
    const int u_begin = qoff[blockIdx.x];
    const int u_end = qoff[blockIdx.x + 1];
    for (int ui = u_begin; ui < u_end; ++ui) {
        const Unit un = load_unit(units, ui);
        decode_unit<QDT, KVDT, D, G, NW, PK, WR>(a, un, lds);
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

// Running merge state of one wave over some parts of one (row, q head): the
// largest LSE seen, the sum of 2^(lse - M), and the lane's D/64 elements of
// the weighted sum of the parts' normalised outputs.
template <int E>
struct MergeState {
    float M = -INFINITY;
    float sw = 0.f;
    float acc[E] = {};
    bool nan = false;
};

// Fold parts c0, c0 + step, ... (< parts) of row r, q head h into st,
// kMergeBatch parts per round trip: every part's LSE and its elements are
// loaded before any is used.  A NaN LSE (a bad block id in some piece) makes
// the row NaN; empty parts (lse = -inf) drop out.
template <int D>
__device__ __forceinline__ void merge_fold(MergeState<D / 64>& st, const float* __restrict__ po,
                                           const_ptr<float> lse, int hq, int prow0, int nrows, int parts, int r, int h,
                                           int c0, int step, int lane) {
    constexpr int E = D / 64;
    constexpr int B = kMergeBatch;
    const int64_t hd = static_cast<int64_t>(hq) * D;
    for (int cb = c0; cb < parts; cb += B * step) {
        float l[B];
        float x[B][E];
#pragma unroll
        for (int b = 0; b < B; ++b) {
            const int64_t prow = prow0 + static_cast<int64_t>(min(cb + b * step, parts - 1)) * nrows + r;
            l[b] = lse[prow * hq + h];
            const float* src = po + prow * hd + static_cast<int64_t>(h) * D + lane * E;
#pragma unroll
            for (int e = 0; e < E; ++e) x[b][e] = src[e];
        }
        float mb = st.M;
#pragma unroll
        for (int b = 0; b < B; ++b) {
            if (cb + b * step >= parts) l[b] = -INFINITY;  // a repeated last part counts once
            st.nan |= l[b] != l[b];
            mb = fmaxf(mb, l[b]);
        }
        if (mb == -INFINITY) continue;  // every part so far is empty
        const float f = exp2_fast(st.M - mb);  // 0 while M is -inf
        st.sw *= f;
#pragma unroll
        for (int e = 0; e < E; ++e) st.acc[e] *= f;
#pragma unroll
        for (int b = 0; b < B; ++b) {
            const float w = exp2_fast(l[b] - mb);  // 0 for an empty part
            st.sw += w;
#pragma unroll
            for (int e = 0; e < E; ++e) st.acc[e] = fmaf(w, x[b][e], st.acc[e]);
        }
        st.M = mb;
    }
}

// The row-block and few-piece records fold with every lane taking 4
// consecutive elements of one (row, q head), one 16-byte load per part: a
// wave covers 256 / D heads, a workgroup kMergeWaves times that.
template <int D>
constexpr int kMergeHeadsPerWave = 256 / D;

// Fold all parts of row r of a record for the lane's 4 elements of q head h
// (h clamped into range for the loads; the caller drops lanes past hq), in
// the same order and arithmetic as merge_fold.
template <int D>
__device__ __forceinline__ void merge_fold4(float& M, float& sw, float (&acc)[4], bool& nan,
                                            const float* __restrict__ po, const float* __restrict__ pl, int hq,
                                            int prow0, int nrows, int parts, int r, int h, int e0) {
    constexpr int B = kMergeBatch;
    const int64_t hd = static_cast<int64_t>(hq) * D;
    for (int cb = 0; cb < parts; cb += B) {
        float l[B];
        float4 x[B];
#pragma unroll
        for (int b = 0; b < B; ++b) {
            const int64_t prow = prow0 + static_cast<int64_t>(min(cb + b, parts - 1)) * nrows + r;
            l[b] = pl[prow * hq + h];
            x[b] = *reinterpret_cast<const float4*>(po + prow * hd + static_cast<int64_t>(h) * D + e0);
        }
        float mb = M;
#pragma unroll
        for (int b = 0; b < B; ++b) {
            if (cb + b >= parts) l[b] = -INFINITY;  // a repeated last part counts once
            nan |= l[b] != l[b];
            mb = fmaxf(mb, l[b]);
        }
        if (mb == -INFINITY) continue;  // every part so far is empty
        const float f = exp2_fast(M - mb);  // 0 while M is -inf
        sw *= f;
#pragma unroll
        for (int e = 0; e < 4; ++e) acc[e] *= f;
#pragma unroll
        for (int b = 0; b < B; ++b) {
            const float w = exp2_fast(l[b] - mb);  // 0 for an empty part
            sw += w;
            acc[0] = fmaf(w, x[b].x, acc[0]);
            acc[1] = fmaf(w, x[b].y, acc[1]);
            acc[2] = fmaf(w, x[b].z, acc[2]);
            acc[3] = fmaf(w, x[b].w, acc[3]);
        }
        M = mb;
    }
}

template <int QDT, int D>
__device__ __forceinline__ void merge_store(void* __restrict__ out, int64_t oi, const float (&acc)[D / 64], float sw,
                                            bool nan, float v_scale) {
    constexpr int E = D / 64;
    const float scale = sw > 0.f ? v_scale / sw : 0.f;
    float o[E];
#pragma unroll
    for (int e = 0; e < E; ++e) o[e] = nan ? NAN : acc[e] * scale;
    if constexpr (QDT == PKV_DTYPE_F32) {
#pragma unroll
        for (int e = 0; e < E; ++e) static_cast<float*>(out)[oi + e] = o[e];
    } else {
#pragma unroll
        for (int e = 0; e < E; ++e) static_cast<uint16_t*>(out)[oi + e] = static_cast<uint16_t>(f32_to_bf16_rne(o[e]));
    }
}

// One launch over all merge records (a 1-D grid of kMergeWaves-wave
// workgroups).  The plan lists its records in three kinds:
//  - wide (one row, at least kWideMergeParts pieces): the first
//    wide_slots * hq blocks give each (record, q head) a workgroup whose wave
//    w folds parts w, w + kMergeWaves, ..., the waves' states then combining
//    through LDS (each scaled by 2^(m_w - M), an empty wave adding nothing);
//  - row blocks of chunk rows, then one-row records with few pieces: the
//    next block_slots * max_rows * hgroups blocks and the last
//    row_slots * hgroups blocks give each (record, row, group of
//    kMergeWaves * kMergeHeadsPerWave<D> q heads) a workgroup, every lane
//    folding all parts of 4 elements of one head.
// The live numbers of records come from `counts` in the workspace when it is
// given (a launch sized for what any plan with these q_lens can hold, made
// once and replayed for later plans), else from the arguments; blocks past
// them exit.
template <int QDT, int D>
__global__ __launch_bounds__(kMergeWaves * 64) void merge_kernel(const Merge* __restrict__ merges,
                                                                 const float* __restrict__ po,
                                                                 const float* __restrict__ pl,
                                                                 void* __restrict__ out, int hq, float v_scale,
                                                                 const int32_t* __restrict__ counts, int num_merges,
                                                                 int num_wide, int num_block, int wide_slots,
                                                                 int block_slots, int max_rows) {
    constexpr int E = D / 64;
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int64_t hd = static_cast<int64_t>(hq) * D;
    const const_ptr<float> lse = as_const(pl);
    if (counts != nullptr) {
        const const_ptr<int32_t> c = as_const(counts);
        num_merges = c[0];
        num_wide = c[1];
        num_block = c[2];
    }
    const int b = blockIdx.x;
    const int wide_blocks = wide_slots * hq;
    if (b < wide_blocks) {
        if (b / hq >= num_wide) return;
        __shared__ float sh_m[kMergeWaves], sh_s[kMergeWaves];
        __shared__ int sh_nan[kMergeWaves];
        __shared__ float sh_acc[kMergeWaves][D];
        const int rec = b / hq, h = b % hq;
        const const_ptr<int32_t> mw = reinterpret_cast<const_ptr<int32_t>>(as_const(merges) + rec);
        const int row0 = mw[0], prow0 = mw[2], parts = mw[3];
        MergeState<E> st;
        merge_fold<D>(st, po, lse, hq, prow0, 1, parts, 0, h, wave, kMergeWaves, lane);
        if (lane == 0) {
            sh_m[wave] = st.M;
            sh_s[wave] = st.sw;
            sh_nan[wave] = st.nan ? 1 : 0;
        }
#pragma unroll
        for (int e = 0; e < E; ++e) sh_acc[wave][lane * E + e] = st.acc[e];
        __syncthreads();
        if (wave != 0) return;
        float Mt = -INFINITY;
        bool nan = false;
#pragma unroll
        for (int w = 0; w < kMergeWaves; ++w) {
            Mt = fmaxf(Mt, sh_m[w]);
            nan |= sh_nan[w] != 0;
        }
        float sw = 0.f;
        float acc[E] = {};
#pragma unroll
        for (int w = 0; w < kMergeWaves; ++w) {
            const float f = sh_m[w] == -INFINITY ? 0.f : exp2_fast(sh_m[w] - Mt);
            sw = fmaf(f, sh_s[w], sw);
#pragma unroll
            for (int e = 0; e < E; ++e) acc[e] = fmaf(f, sh_acc[w][lane * E + e], acc[e]);
        }
        merge_store<QDT, D>(out, static_cast<int64_t>(row0) * hd + static_cast<int64_t>(h) * D + lane * E, acc, sw,
                            nan, v_scale);
        return;
    }
    constexpr int HPW = kMergeHeadsPerWave<D>;
    constexpr int LPH = 64 / HPW;  // lanes per head
    const int hgroups = (hq + kMergeWaves * HPW - 1) / (kMergeWaves * HPW);
    const int b2 = b - wide_blocks;
    const int block_blocks = block_slots * max_rows * hgroups;
    int rec, r;
    if (b2 < block_blocks) {
        rec = num_wide + b2 / (max_rows * hgroups);
        if (rec >= num_wide + num_block) return;
        r = (b2 / hgroups) % max_rows;
    } else {
        rec = num_wide + num_block + (b2 - block_blocks) / hgroups;
        if (rec >= num_merges) return;
        r = 0;
    }
    const int h = (b2 % hgroups) * kMergeWaves * HPW + wave * HPW + lane / LPH;
    const int e0 = (lane % LPH) * 4;
    const const_ptr<int32_t> mw = reinterpret_cast<const_ptr<int32_t>>(as_const(merges) + rec);
    const int row0 = mw[0], nrows = mw[1], prow0 = mw[2], parts = mw[3];
    if (r >= nrows) return;
    float M = -INFINITY, sw = 0.f;
    float acc[4] = {0.f, 0.f, 0.f, 0.f};
    bool nan = false;
    merge_fold4<D>(M, sw, acc, nan, po, pl, hq, prow0, nrows, parts, r, min(h, hq - 1), e0);
    if (h >= hq) return;
    const float scale = sw > 0.f ? v_scale / sw : 0.f;
    float o[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) o[e] = nan ? NAN : acc[e] * scale;
    store_out<QDT, 4>(static_cast<char*>(out) +
                          (static_cast<int64_t>(row0 + r) * hd + static_cast<int64_t>(h) * D + e0) * dt_bytes(QDT),
                      o);
}

// Launch shape: one persistent workgroup per queue.  8 waves (one per kv head
// of the 8-head workloads) stream bf16 / fp32 K/V on whole-tile pages (one
// workgroup per CU: more loads in flight per CU lower the read rate of this
// pattern).  One 8-wave workgroup per CU is two waves per SIMD, so those
// kernels are built for two (up to 256 VGPRs): the register room lets the
// compiler schedule the loads of a tile earlier than a 128-VGPR build does,
// which measured 2.4 % faster on the 64-sequence decode batch.  16 waves
// (two per kv head, alternate tiles, <= 128 VGPRs) hide the extra latency
// of per-lane page lookups (page sizes other than 1, 4, 8 and multiples of
// 16) and the fp8 conversion work.  Group 8 (eight q heads per lane), group
// 1 (sixteen tokens in flight per lane), group 2 on per-lane pages at
// D = 128 and fp32 K/V need more registers and keep 8 waves at two waves per
// SIMD.
template <int QDT, int KVDT, int D, int G, int NW, int PK, int WPE>
void launch_decode_kernel(const AttnArgs& a, int num_queues, hipStream_t st) {
    hipLaunchKernelGGL((decode_kernel<QDT, KVDT, D, G, NW, PK, WPE>), dim3(num_queues), dim3(NW * 64), 0, st, a);
}

// A decode kernel shape for every page kind it serves: whole tiles, groups
// of 4 or 8 tokens, one-token pages (ONE: groups 2 to 8 with the register
// room for a wave-tile's next entries; otherwise they take the kPageAny
// kernel) and any other size.
template <int QDT, int KVDT, int D, int G, int NW, int WPE, bool ONE>
void launch_decode_pk(const AttnArgs& a, int num_queues, int pk, hipStream_t st) {
    if (pk == kPageTile)
        launch_decode_kernel<QDT, KVDT, D, G, NW, kPageTile, WPE>(a, num_queues, st);
    else if (pk == kPageGroup)
        launch_decode_kernel<QDT, KVDT, D, G, NW, kPageGroup, WPE>(a, num_queues, st);
    else if (ONE && pk == kPageOne)
        launch_decode_kernel<QDT, KVDT, D, G, NW, (ONE ? kPageOne : kPageAny), WPE>(a, num_queues, st);
    else
        launch_decode_kernel<QDT, KVDT, D, G, NW, kPageAny, WPE>(a, num_queues, st);
}

template <int QDT, int KVDT, int D, int G>
int launch_decode_t(const AttnArgs& a, int num_queues, int pk, hipStream_t st) {
    constexpr bool kSmallRegs = !(G == 8 || G == 1 || KVDT == PKV_DTYPE_F32);
    if constexpr (kSmallRegs) {
        if constexpr (KVDT == PKV_DTYPE_FP8_E4M3) {
            launch_decode_pk<QDT, KVDT, D, G, 16, 4, false>(a, num_queues, pk, st);
        } else if (pk != kPageAny) {
            launch_decode_pk<QDT, KVDT, D, G, 8, 2, true>(a, num_queues, pk, st);
        } else if constexpr (G == 2 && D == 128) {
            // eight tokens per lane and wave-tile need more than 128 registers
            launch_decode_kernel<QDT, KVDT, D, G, 8, kPageAny, 2>(a, num_queues, st);
        } else {
            launch_decode_kernel<QDT, KVDT, D, G, 16, kPageAny, 4>(a, num_queues, st);
        }
    } else {
        launch_decode_pk<QDT, KVDT, D, G, 8, 2, (G >= 2 && KVDT != PKV_DTYPE_F32)>(a, num_queues, pk, st);
    }
    return hipGetLastError() == hipSuccess ? PKV_OK : PKV_ERR_HIP;
}

template <int QDT, int KVDT, int D>
int launch_decode_g(const AttnArgs& a, int group, int num_queues, int pk, hipStream_t st) {
    switch (group) {
        case 1: return launch_decode_t<QDT, KVDT, D, 1>(a, num_queues, pk, st);
        case 2: return launch_decode_t<QDT, KVDT, D, 2>(a, num_queues, pk, st);
        case 4: return launch_decode_t<QDT, KVDT, D, 4>(a, num_queues, pk, st);
        case 8: return launch_decode_t<QDT, KVDT, D, 8>(a, num_queues, pk, st);
        default: return PKV_ERR_UNSUPPORTED;
    }
}

template <int QDT, int KVDT>
int launch_decode_d(const AttnArgs& a, int d, int group, int num_queues, int pk, hipStream_t st) {
    if (d == 64) return launch_decode_g<QDT, KVDT, 64>(a, group, num_queues, pk, st);
    if (d == 128) return launch_decode_g<QDT, KVDT, 128>(a, group, num_queues, pk, st);
    return PKV_ERR_UNSUPPORTED;
}

}  // namespace

int launch_decode(const AttnArgs& a, int q_dtype, int kv_dtype, int head_dim, int group, int num_queues,
                  void* stream) {
    hipStream_t st = static_cast<hipStream_t>(stream);
    // the page kind: whole 16-token tiles, groups of 4 tokens, one token,
    // anything else
    const int bs = a.block_size;
    const int pk = bs % kTileTokens == 0 ? kPageTile
                   : (bs == 4 || bs == 8) ? kPageGroup
                   : (bs == 1 && group >= 2) ? kPageOne
                                             : kPageAny;
    if (q_dtype == PKV_DTYPE_F32 && kv_dtype == PKV_DTYPE_F32)
        return launch_decode_d<PKV_DTYPE_F32, PKV_DTYPE_F32>(a, head_dim, group, num_queues, pk, st);
    if (q_dtype == PKV_DTYPE_BF16 && kv_dtype == PKV_DTYPE_BF16)
        return launch_decode_d<PKV_DTYPE_BF16, PKV_DTYPE_BF16>(a, head_dim, group, num_queues, pk, st);
    if (q_dtype == PKV_DTYPE_BF16 && kv_dtype == PKV_DTYPE_FP8_E4M3)
        return launch_decode_d<PKV_DTYPE_BF16, PKV_DTYPE_FP8_E4M3>(a, head_dim, group, num_queues, pk, st);
    return PKV_ERR_UNSUPPORTED;
}

// The decode kernel that also writes the step's new tokens (a.slot_mapping):
// bf16 q and K/V on pages of whole 16-token tiles, the shape the serving
// step uses; a separate build so that the plain decode kernel carries none
// of it.
int launch_decode_write(const AttnArgs& a, int head_dim, int group, int num_queues, void* stream) {
    hipStream_t st = static_cast<hipStream_t>(stream);
    if (a.block_size % kTileTokens != 0 || a.slot_mapping == nullptr) return PKV_ERR_UNSUPPORTED;
    constexpr int BF = PKV_DTYPE_BF16;
    auto go = [&](auto d, auto g) {
        constexpr int D = decltype(d)::value, G = decltype(g)::value;
        hipLaunchKernelGGL((decode_kernel<BF, BF, D, G, 8, kPageTile, 2, true>), dim3(num_queues), dim3(8 * 64), 0,
                           st, a);
        return hipGetLastError() == hipSuccess ? PKV_OK : PKV_ERR_HIP;
    };
    using D64 = std::integral_constant<int, 64>;
    using D128 = std::integral_constant<int, 128>;
    auto by_group = [&](auto d) {
        switch (group) {
            case 1: return go(d, std::integral_constant<int, 1>{});
            case 2: return go(d, std::integral_constant<int, 2>{});
            case 4: return go(d, std::integral_constant<int, 4>{});
            case 8: return go(d, std::integral_constant<int, 8>{});
            default: return static_cast<int>(PKV_ERR_UNSUPPORTED);
        }
    };
    if (head_dim == 64) return by_group(D64{});
    if (head_dim == 128) return by_group(D128{});
    return PKV_ERR_UNSUPPORTED;
}

int launch_merge(const AttnArgs& a, const pkv_plan* plan, const void* workspace, int max_rows, int q_dtype,
                 int head_dim, void* stream) {
    hipStream_t st = static_cast<hipStream_t>(stream);
    const Merge* merges = reinterpret_cast<const Merge*>(static_cast<const char*>(workspace) + plan->off_merges);
    // A launch made while the stream is being captured is replayed for later
    // plans of the same room: it covers every record the room can hold and
    // reads the live counts from the workspace.
    hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
    const bool capturing = hipStreamIsCapturing(st, &cs) == hipSuccess && cs == hipStreamCaptureStatusActive;
    const int32_t* counts = nullptr;
    int64_t wide_slots = plan->num_wide_merges;
    int64_t block_slots = plan->num_block_merges;
    int64_t row_slots = static_cast<int64_t>(plan->num_merges) - wide_slots - block_slots;
    if (capturing) {
        counts = reinterpret_cast<const int32_t*>(static_cast<const char*>(workspace) + plan->off_queues) +
                 plan_counts_index(plan->num_queues);
        wide_slots = plan->max_row_merges;
        block_slots = plan->max_block_merges;
        row_slots = plan->max_row_merges;
    }
    const int64_t hpg = static_cast<int64_t>(kMergeWaves) * (head_dim == 64 ? kMergeHeadsPerWave<64>
                                                                              : kMergeHeadsPerWave<128>);
    const int64_t hgroups = (a.hq + hpg - 1) / hpg;
    const int64_t blocks = wide_slots * a.hq + block_slots * max_rows * hgroups + row_slots * hgroups;
    if (blocks == 0) return PKV_OK;
    if (blocks > 0x7FFFFFFF) return PKV_ERR_SHAPE;
    const dim3 grid(static_cast<uint32_t>(blocks));
    const dim3 block(kMergeWaves * 64);
    const int nm = plan->num_merges, nw = plan->num_wide_merges, nb = plan->num_block_merges;
    const int ws = static_cast<int>(wide_slots), bsl = static_cast<int>(block_slots);
    if (q_dtype == PKV_DTYPE_F32 && head_dim == 64)
        hipLaunchKernelGGL((merge_kernel<PKV_DTYPE_F32, 64>), grid, block, 0, st, merges, a.partial_o, a.partial_lse,
                           a.out, a.hq, a.v_scale, counts, nm, nw, nb, ws, bsl, max_rows);
    else if (q_dtype == PKV_DTYPE_F32)
        hipLaunchKernelGGL((merge_kernel<PKV_DTYPE_F32, 128>), grid, block, 0, st, merges, a.partial_o, a.partial_lse,
                           a.out, a.hq, a.v_scale, counts, nm, nw, nb, ws, bsl, max_rows);
    else if (head_dim == 64)
        hipLaunchKernelGGL((merge_kernel<PKV_DTYPE_BF16, 64>), grid, block, 0, st, merges, a.partial_o, a.partial_lse,
                           a.out, a.hq, a.v_scale, counts, nm, nw, nb, ws, bsl, max_rows);
    else
        hipLaunchKernelGGL((merge_kernel<PKV_DTYPE_BF16, 128>), grid, block, 0, st, merges, a.partial_o, a.partial_lse,
                           a.out, a.hq, a.v_scale, counts, nm, nw, nb, ws, bsl, max_rows);
    return hipGetLastError() == hipSuccess ? PKV_OK : PKV_ERR_HIP;
}

}  // namespace pkv
