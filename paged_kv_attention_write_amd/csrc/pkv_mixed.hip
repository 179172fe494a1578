// Mixed chunked-prefill + decode step (gfx950).
//
// One persistent workgroup per planner queue walks its units: a decode unit
// (one row, every kv head) runs the decode unit code unchanged; a prefill unit
// (a block of rows of one chunk, one kv head, one key piece) runs the
// matrix-core tile below.  ("nanoserve", packed batches and chunked prefill:
// the decode rows and the prefill chunk of a mixed step go to their own
// kernels' code paths, the decode rows never through a gather.)
//
// Prefill tile.  The unit's kPrefillQRows (row, q head) pairs of kv head h
// are spread over the 8 waves, 16 per wave: pair x = 16 w + n is row x / G,
// q head h G + x % G, so the G heads that share K/V sit side by side.  Per
// tile of 32 keys the workgroup stages K (row-major) and V (transposed, keys
// in the order the second product consumes them) in LDS, then every wave
// computes, with v_mfma_f32_16x16x32_bf16,
//   S^T[key][pair] = K Q^T   (A = K from LDS, B = its q slice in registers)
//   O^T[d][pair]  += V^T P^T (A = V^T from LDS, B = P straight from the
//                             registers that hold S^T, rounded to bf16)
// The transposed forms put one pair per lane column in both results: lane l
// holds pair l % 16 for keys / dimensions 4 (l / 16) + i, so the online
// softmax state of a pair lives in the lanes that accumulate its output and
// no data moves between the two products.  Row maxima and sums combine the
// four lanes of a pair (l, l^16, l^32, l^48).  Keys are masked bottom-right
// causally: row r of the chunk sits at position pos0 + r and sees keys up to
// it.  fp8 K/V are widened to bf16 (exactly) when staged.
#include "pkv_decode_unit.h"

namespace pkv {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));

constexpr int kPfWaves = 8;
constexpr int kPfPairsPerWave = 16;  // MFMA N
constexpr int kPfKeys = 32;          // keys per staged tile
static_assert(kPfWaves * kPfPairsPerWave == kPrefillQRows, "one 16-pair slice per wave");

template <int D>
struct PrefillLds {
    uint16_t k[kPfKeys][D + 8];   // K tile, row-major; rows padded by 16 bytes
    uint16_t vt[D][kPfKeys + 8];  // V^T tile, keys in operand slot order; rows padded by 16 bytes
};

// Slot of key kk (0..31) in a V^T row.  The second product's k index s = 8 g
// + j of lane group g is the key (j / 4) * 16 + 4 g + j % 4, which is where
// the first product left that key's score in lane group g.
__device__ __forceinline__ int vt_slot(int kk) { return ((kk & 15) >> 2) * 8 + (kk >> 4) * 4 + (kk & 3); }

// Global K/V bytes of one staged item (8 elements).
template <int KVDT>
struct PfItem {
    static constexpr int W = KVDT == PKV_DTYPE_FP8_E4M3 ? 2 : 4;  // 32-bit words
};

// 8 K/V elements as 8 bf16 (4 words); fp8 codes widen exactly.
template <int KVDT>
__device__ __forceinline__ Words<4> item_to_bf16(const Words<PfItem<KVDT>::W>& r) {
    if constexpr (KVDT == PKV_DTYPE_BF16) {
        return r;
    } else {
        Words<4> o;
#pragma unroll
        for (int w = 0; w < 2; ++w) {
            const float2_t lo = __builtin_amdgcn_cvt_pk_f32_fp8(static_cast<int>(r.w[w]), false);
            const float2_t hi = __builtin_amdgcn_cvt_pk_f32_fp8(static_cast<int>(r.w[w]), true);
            o.w[2 * w] = (__float_as_uint(lo.x) >> 16) | (__float_as_uint(lo.y) & 0xFFFF0000u);
            o.w[2 * w + 1] = (__float_as_uint(hi.x) >> 16) | (__float_as_uint(hi.y) & 0xFFFF0000u);
        }
        return o;
    }
}

template <int KVDT, int D>
struct PfStage {
    static constexpr int ITEMS = kPfKeys * D / 8;              // per tensor
    static constexpr int PER_THREAD = 2 * ITEMS / (kPfWaves * 64);  // K and V items of one thread
    static_assert(2 * ITEMS % (kPfWaves * 64) == 0, "items split evenly");
    Words<PfItem<KVDT>::W> raw[PER_THREAD];
    bool ok[PER_THREAD];
};

// Issue the loads of the tile at key t0: item it < ITEMS is K, else V; item
// (key kk, group dg) holds elements 8 dg .. 8 dg + 7 of key t0 + kk.  Keys at
// or past kend and pages outside the pool load nothing (zeros are staged).
template <int KVDT, int D>
__device__ __forceinline__ void pf_load(PfStage<KVDT, D>& st, const AttnArgs& a, const_ptr<int32_t> tbl, int h,
                                        int t0, int kend, bool& bad) {
    using S = PfStage<KVDT, D>;
    constexpr int KVB = dt_bytes(KVDT);
    constexpr int W = PfItem<KVDT>::W;
    const uint32_t nblocks = static_cast<uint32_t>(a.num_blocks < 0x7FFFFFFF ? a.num_blocks : 0x7FFFFFFF);
#pragma unroll
    for (int i = 0; i < S::PER_THREAD; ++i) {
        const int it = static_cast<int>(threadIdx.x) + i * kPfWaves * 64;
        const bool is_v = it >= S::ITEMS;
        const int item = is_v ? it - S::ITEMS : it;
        const int kk = item / (D / 8);
        const int dg = item % (D / 8);
        const int t = t0 + kk;
        const bool tv = t < kend;
        const int pidx = t / a.block_size;
        const uint32_t page = static_cast<uint32_t>((tv && pidx < a.max_blocks) ? tbl[pidx] : -1);
        const bool ok = tv && page < nblocks;  // a negative id wraps to >= 2^31
        bad |= tv && !ok;
        st.ok[i] = ok;
        if (ok) {
            const int64_t slot = static_cast<int64_t>(page) * a.block_size + (t - pidx * a.block_size);
            const char* base = static_cast<const char*>(is_v ? a.v_cache : a.k_cache);
            st.raw[i] = load_words<W>(base + ((slot * a.hkv + h) * D + dg * 8) * KVB);
        } else {
#pragma unroll
            for (int w = 0; w < W; ++w) st.raw[i].w[w] = 0u;
        }
    }
}

template <int KVDT, int D>
__device__ __forceinline__ void pf_stage(const PfStage<KVDT, D>& st, PrefillLds<D>& lds) {
    using S = PfStage<KVDT, D>;
#pragma unroll
    for (int i = 0; i < S::PER_THREAD; ++i) {
        const int it = static_cast<int>(threadIdx.x) + i * kPfWaves * 64;
        const bool is_v = it >= S::ITEMS;
        const int item = is_v ? it - S::ITEMS : it;
        const int kk = item / (D / 8);
        const int dg = item % (D / 8);
        Words<4> w = item_to_bf16<KVDT>(st.raw[i]);
#pragma unroll
        for (int j = 0; j < 4; ++j) w.w[j] = st.ok[i] ? w.w[j] : 0u;
        if (!is_v) {
            store_words<4>(&lds.k[kk][dg * 8], w);
        } else {
            const int s = vt_slot(kk);
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                lds.vt[dg * 8 + 2 * j][s] = static_cast<uint16_t>(w.w[j] & 0xFFFFu);
                lds.vt[dg * 8 + 2 * j + 1][s] = static_cast<uint16_t>(w.w[j] >> 16);
            }
        }
    }
}

__device__ __forceinline__ bf16x8_t lds_bf16x8(const uint16_t* p) {
    return __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const uint4*>(p));
}

// One prefill unit (kind >= 1) on the calling workgroup.
template <int KVDT, int D, int G>
__device__ __forceinline__ void prefill_unit(const AttnArgs& a, const Unit& un, PrefillLds<D>& lds) {
    constexpr int QB = 2;  // bf16 queries
    constexpr int NS = D / 32;  // k steps of the first product
    constexpr int ND = D / 16;  // 16-row blocks of O^T
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int n = lane & 15;  // pair column of this lane
    const int g4 = lane >> 4;
    const int h = un.kind - kUnitPrefill;

    const int x = wave * kPfPairsPerWave + n;
    const int r = x / G;  // row of the chunk block
    const int hq_idx = h * G + x % G;
    const bool row_ok = r < un.nrows;
    const int pos = un.pos0 + r;
    // rows of this wave: positions pos0 + wr0 .. pos0 + wr1
    const int wr0 = (wave * kPfPairsPerWave) / G;
    const int wr1 = min(un.nrows - 1, (wave * kPfPairsPerWave + kPfPairsPerWave - 1) / G);
    const bool wave_has_rows = wr0 < un.nrows;
    const int wave_last_pos = un.pos0 + wr1;

    const int n_ctx = as_const(a.context_lens)[un.seq];
    const int kend = min(min(un.kv_end, n_ctx), un.pos0 + un.nrows);  // no row sees past its position
    const const_ptr<int32_t> tbl = as_const(a.block_tables) + static_cast<int64_t>(un.seq) * a.max_blocks;

    // q slice of this lane's pair: elements 32 s + 8 g4 .. + 7
    bf16x8_t qb[NS];
    {
        const char* qrow = static_cast<const char*>(a.q) +
                           (static_cast<int64_t>(un.row0 + r) * a.q_stride + static_cast<int64_t>(hq_idx) * D) * QB;
#pragma unroll
        for (int s = 0; s < NS; ++s) {
            Words<4> w;
            if (row_ok) {
                w = load_words<4>(qrow + (32 * s + 8 * g4) * QB);
            } else {
#pragma unroll
                for (int j = 0; j < 4; ++j) w.w[j] = 0u;
            }
            qb[s] = __builtin_bit_cast(bf16x8_t, make_uint4(w.w[0], w.w[1], w.w[2], w.w[3]));
        }
    }

    f32x4_t acc[ND];
#pragma unroll
    for (int b = 0; b < ND; ++b) acc[b] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    float m_run = -INFINITY;  // running max of this lane's pair (its four lanes agree)
    float l_run = 0.f;        // this lane's share of the running sum
    bool bad = false;

    __syncthreads();  // the LDS of the previous unit is free
    PfStage<KVDT, D> st;
    pf_load<KVDT, D>(st, a, tbl, h, un.kv_begin, kend, bad);
    for (int t0 = un.kv_begin; t0 < kend; t0 += kPfKeys) {
        pf_stage<KVDT, D>(st, lds);
        __syncthreads();
        if (t0 + kPfKeys < kend) pf_load<KVDT, D>(st, a, tbl, h, t0 + kPfKeys, kend, bad);
        if (wave_has_rows && t0 <= wave_last_pos) {
            // S^T for keys t0 + 16 kb2 + 4 g4 + i, pair n
            float sv[8];
#pragma unroll
            for (int kb2 = 0; kb2 < 2; ++kb2) {
                f32x4_t c = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int s = 0; s < NS; ++s)
                    c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(lds_bf16x8(&lds.k[16 * kb2 + n][32 * s + 8 * g4]),
                                                                qb[s], c, 0, 0, 0);
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int kp = t0 + 16 * kb2 + 4 * g4 + i;
                    sv[4 * kb2 + i] = (row_ok && kp < kend && kp <= pos) ? c[i] * a.qk_scale : -INFINITY;
                }
            }
            float mt = sv[0];
#pragma unroll
            for (int j = 1; j < 8; ++j) mt = fmaxf(mt, sv[j]);
            mt = fmaxf(mt, __shfl_xor(mt, 16));
            mt = fmaxf(mt, __shfl_xor(mt, 32));
            // lazy rescale, as in the decode unit: scores at most 2^8 above
            // the running maximum are taken against it
            const bool need = mt > m_run + 8.0f;
            if (__any(need)) {
                const float m_new = need ? mt : m_run;
                const float alpha = need ? exp2_fast(m_run - m_new) : 1.f;
                l_run *= alpha;
                m_run = m_new;
#pragma unroll
                for (int b = 0; b < ND; ++b) acc[b] *= alpha;
            }
            const float mb = (m_run == -INFINITY) ? 0.f : m_run;
            uint32_t pw[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const uint32_t lo = f32_to_bf16_rne(exp2_fast(sv[2 * j] - mb));
                const uint32_t hi = f32_to_bf16_rne(exp2_fast(sv[2 * j + 1] - mb));
                l_run += __uint_as_float(lo << 16) + __uint_as_float(hi << 16);  // the weights P V uses
                pw[j] = lo | (hi << 16);
            }
            const bf16x8_t pb = __builtin_bit_cast(bf16x8_t, make_uint4(pw[0], pw[1], pw[2], pw[3]));
#pragma unroll
            for (int b = 0; b < ND; ++b)
                acc[b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(lds_bf16x8(&lds.vt[16 * b + n][8 * g4]), pb, acc[b],
                                                                 0, 0, 0);
        }
        __syncthreads();
    }
    bad = __syncthreads_or(bad) != 0;

    float l_tot = l_run + __shfl_xor(l_run, 16);
    l_tot += __shfl_xor(l_tot, 32);
    if (!row_ok) return;
    const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
    if (un.prow < 0) {
        uint16_t* dst = static_cast<uint16_t*>(a.out) +
                        (static_cast<int64_t>(un.row0 + r) * a.hq + hq_idx) * D + 4 * g4;
        const float sc = inv * a.v_scale;
#pragma unroll
        for (int b = 0; b < ND; ++b) {
            float o[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) o[i] = bad ? NAN : acc[b][i] * sc;
            store_out<PKV_DTYPE_BF16, 4>(reinterpret_cast<char*>(dst + 16 * b), o);
        }
    } else {
        const int64_t prow = static_cast<int64_t>(un.prow) + r;
        float* dst = a.partial_o + (prow * a.hq + hq_idx) * D + 4 * g4;
#pragma unroll
        for (int b = 0; b < ND; ++b) {
            const float4 o = bad ? make_float4(NAN, NAN, NAN, NAN)
                                 : make_float4(acc[b][0] * inv, acc[b][1] * inv, acc[b][2] * inv, acc[b][3] * inv);
            *reinterpret_cast<float4*>(dst + 16 * b) = o;
        }
        if (g4 == 0)
            a.partial_lse[prow * a.hq + hq_idx] = bad ? NAN : (l_tot > 0.f ? m_run + __log2f(l_tot) : -INFINITY);
    }
}

template <int D, int G>
constexpr size_t mixed_lds_bytes() {
    return sizeof(DecodeLds<D, G, kPfWaves>) > sizeof(PrefillLds<D>) ? sizeof(DecodeLds<D, G, kPfWaves>)
                                                                      : sizeof(PrefillLds<D>);
}

template <int KVDT, int D, int G, bool UNIFORM_PAGE, int WPE>
__global__ __launch_bounds__(kPfWaves * 64) __attribute__((amdgpu_waves_per_eu(WPE)))
void mixed_kernel(AttnArgs a) {
    __shared__ __attribute__((aligned(16))) char smem[mixed_lds_bytes<D, G>()];
    const const_ptr<Unit> units = as_const(a.units);
    const const_ptr<int32_t> qoff = as_const(a.queue_off);
    const int u_begin = qoff[blockIdx.x];
    const int u_end = qoff[blockIdx.x + 1];
    for (int ui = u_begin; ui < u_end; ++ui) {
        const Unit un = load_unit(units, ui);
        if (un.kind == kUnitDecode)
            decode_unit<PKV_DTYPE_BF16, KVDT, D, G, kPfWaves, UNIFORM_PAGE>(
                a, un, *reinterpret_cast<DecodeLds<D, G, kPfWaves>*>(smem));
        else
            prefill_unit<KVDT, D, G>(a, un, *reinterpret_cast<PrefillLds<D>*>(smem));
    }
}

template <int KVDT, int D, int G>
int launch_mixed_t(const AttnArgs& a, int num_queues, bool uniform, hipStream_t st) {
    constexpr int WPE = (G == 8 || G == 1) ? 2 : 4;
    if (uniform)
        hipLaunchKernelGGL((mixed_kernel<KVDT, D, G, true, WPE>), dim3(num_queues), dim3(kPfWaves * 64), 0, st, a);
    else
        hipLaunchKernelGGL((mixed_kernel<KVDT, D, G, false, WPE>), dim3(num_queues), dim3(kPfWaves * 64), 0, st, a);
    return hipGetLastError() == hipSuccess ? PKV_OK : PKV_ERR_HIP;
}

template <int KVDT, int D>
int launch_mixed_g(const AttnArgs& a, int group, int num_queues, bool uniform, hipStream_t st) {
    switch (group) {
        case 1: return launch_mixed_t<KVDT, D, 1>(a, num_queues, uniform, st);
        case 2: return launch_mixed_t<KVDT, D, 2>(a, num_queues, uniform, st);
        case 4: return launch_mixed_t<KVDT, D, 4>(a, num_queues, uniform, st);
        case 8: return launch_mixed_t<KVDT, D, 8>(a, num_queues, uniform, st);
        default: return PKV_ERR_UNSUPPORTED;
    }
}

template <int KVDT>
int launch_mixed_d(const AttnArgs& a, int d, int group, int num_queues, bool uniform, hipStream_t st) {
    if (d == 64) return launch_mixed_g<KVDT, 64>(a, group, num_queues, uniform, st);
    if (d == 128) return launch_mixed_g<KVDT, 128>(a, group, num_queues, uniform, st);
    return PKV_ERR_UNSUPPORTED;
}

}  // namespace

int launch_mixed(const AttnArgs& a, int q_dtype, int kv_dtype, int head_dim, int group, int num_queues,
                 void* stream) {
    hipStream_t st = static_cast<hipStream_t>(stream);
    const bool uniform = (a.block_size % kTileTokens) == 0;
    if (q_dtype != PKV_DTYPE_BF16) return PKV_ERR_UNSUPPORTED;  // the prefill tile is a bf16 product
    if (kv_dtype == PKV_DTYPE_BF16)
        return launch_mixed_d<PKV_DTYPE_BF16>(a, head_dim, group, num_queues, uniform, st);
    if (kv_dtype == PKV_DTYPE_FP8_E4M3)
        return launch_mixed_d<PKV_DTYPE_FP8_E4M3>(a, head_dim, group, num_queues, uniform, st);
    return PKV_ERR_UNSUPPORTED;
}

}  // namespace pkv
