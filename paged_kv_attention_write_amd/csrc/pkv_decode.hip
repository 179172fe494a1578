// Paged decode attention and the merge of split pieces (gfx950).
//
// What is computed: for each query row, softmax(scale * q K^T) V over the
// keys of its sequence, K/V read in place from the block pool through the
// sequence's block table with an online softmax ("nanoserve", Triton
// paged-attention decode bullet), the work split into pieces by the host
// planner and the pieces of a cut sequence merged by their log-sum-exp ("How
// Easy Is It to Start Serving LLMs?", Phase 4 §3).
//
// Mapping onto CDNA4:
// * One workgroup per planner queue (persistent: it walks its queue's units).
//   A workgroup has NW waves; a wave owns one kv head of the unit (NW / H_kv
//   waves share a head and take alternate 16-token tiles when H_kv < NW).
// * A wave reads 4 tokens per load instruction: lane (row r, col c) loads
//   elements [c*D/16, (c+1)*D/16) of token 4i + r, i.e. one coalesced
//   16-byte (bf16, D=128) slice per lane and a 256-byte row per 16 lanes.
//   The G = Hq/H_kv query heads of the group are held in registers and reuse
//   every K row once loaded.
// * q.k partial sums are reduced over the 16 lanes of a row with four DPP
//   steps; each row keeps its own online-softmax state (m, l, acc) over the
//   tokens it saw, so no cross-row traffic happens inside the loop; the four
//   rows (and the waves sharing a head) are merged once per unit.
// * Scores are kept in log2 units (scale * log2 e folded into one factor)
//   so the exponentials are single v_exp_f32 instructions.
#include <math.h>

#include "pkv_attention.h"

namespace pkv {
namespace {

template <int QDT, int KVDT, int D, int G>
struct DecodeRegs {
    static constexpr int EPL = D / 16;                           // elements per lane
    static constexpr int KW = EPL * dt_bytes(KVDT) / 4;          // K/V words per lane
    static constexpr int QW = EPL * dt_bytes(QDT) / 4;           // q words per lane
    static constexpr bool kDot2 = (QDT == PKV_DTYPE_BF16 && KVDT == PKV_DTYPE_BF16);
};

// Query slice of one head held by a lane: bf16 pairs (dot2 path) or fp32.
template <int QDT, int KVDT, int D>
struct QSlice {
    using R = DecodeRegs<QDT, KVDT, D, 1>;
    uint32_t w[R::kDot2 ? R::EPL / 2 : 1];
    float f[R::kDot2 ? 1 : R::EPL];
};

template <int QDT, int KVDT, int D>
__device__ __forceinline__ void load_q(QSlice<QDT, KVDT, D>& q, const char* p) {
    using R = DecodeRegs<QDT, KVDT, D, 1>;
    const Words<R::QW> raw = load_words<R::QW>(p);
    if constexpr (R::kDot2) {
#pragma unroll
        for (int j = 0; j < R::EPL / 2; ++j) q.w[j] = raw.w[j];
    } else if constexpr (QDT == PKV_DTYPE_F32) {
#pragma unroll
        for (int e = 0; e < R::EPL; ++e) q.f[e] = __uint_as_float(raw.w[e]);
    } else {
#pragma unroll
        for (int j = 0; j < R::EPL / 2; ++j) {
            q.f[2 * j] = bf16_lo(raw.w[j]);
            q.f[2 * j + 1] = bf16_hi(raw.w[j]);
        }
    }
}

// K/V slice of one token as fp32 (exact for every storage dtype).
template <int KVDT, int EPL, int KW>
__device__ __forceinline__ void kv_to_f32(float (&x)[EPL], const Words<KW>& r) {
    if constexpr (KVDT == PKV_DTYPE_F32) {
#pragma unroll
        for (int e = 0; e < EPL; ++e) x[e] = __uint_as_float(r.w[e]);
    } else if constexpr (KVDT == PKV_DTYPE_BF16) {
#pragma unroll
        for (int j = 0; j < EPL / 2; ++j) {
            x[2 * j] = bf16_lo(r.w[j]);
            x[2 * j + 1] = bf16_hi(r.w[j]);
        }
    } else {
#pragma unroll
        for (int w = 0; w < KW; ++w) {
            const float2_t lo = __builtin_amdgcn_cvt_pk_f32_fp8(static_cast<int>(r.w[w]), false);
            const float2_t hi = __builtin_amdgcn_cvt_pk_f32_fp8(static_cast<int>(r.w[w]), true);
            x[4 * w] = lo.x;
            x[4 * w + 1] = lo.y;
            x[4 * w + 2] = hi.x;
            x[4 * w + 3] = hi.y;
        }
    }
}

template <int QDT, int KVDT, int D, int G, int NW, bool UNIFORM_PAGE>
__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(4)))
void decode_kernel(AttnArgs a) {
    using R = DecodeRegs<QDT, KVDT, D, G>;
    constexpr int EPL = R::EPL;
    constexpr int KW = R::KW;
    constexpr int KVB = dt_bytes(KVDT);
    constexpr int QB = dt_bytes(QDT);

    __shared__ float lds_acc[NW][G][D];
    __shared__ float lds_ml[NW][G][2];
    __shared__ int lds_bad[NW];

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int row = lane >> 4;
    const int col = lane & 15;
    const int hkv = a.hkv;
    const int tp = (hkv <= NW && NW % hkv == 0) ? NW / hkv : 1;  // waves per kv head
    const int sub = wave % tp;
    const int head0 = wave / tp;
    const int hstep = NW / tp;
    const int bs = a.block_size;
    const int64_t hq_d = static_cast<int64_t>(a.hq) * D;

    const char* __restrict__ kc = static_cast<const char*>(a.k_cache);
    const char* __restrict__ vc = static_cast<const char*>(a.v_cache);

    const int u_begin = a.queue_off[blockIdx.x];
    const int u_end = a.queue_off[blockIdx.x + 1];
    for (int ui = u_begin; ui < u_end; ++ui) {
        const Unit u = a.units[ui];
        const int n = a.context_lens[u.seq];
        const int kb = u.kv_begin;
        const int ke = min(u.kv_end, n);
        const int32_t* __restrict__ tbl = a.block_tables + static_cast<int64_t>(u.seq) * a.max_blocks;

        for (int h = head0; h < hkv; h += hstep) {
            QSlice<QDT, KVDT, D> q[G];
            const char* qbase = static_cast<const char*>(a.q) +
                                (static_cast<int64_t>(u.row0) * a.q_stride + static_cast<int64_t>(h) * G * D +
                                 col * EPL) * QB;
#pragma unroll
            for (int g = 0; g < G; ++g) load_q<QDT, KVDT, D>(q[g], qbase + static_cast<int64_t>(g) * D * QB);

            float m[G], l[G], acc[G][EPL];
#pragma unroll
            for (int g = 0; g < G; ++g) {
                m[g] = -INFINITY;
                l[g] = 0.f;
#pragma unroll
                for (int e = 0; e < EPL; ++e) acc[g][e] = 0.f;
            }
            bool bad = false;

            for (int t0 = kb + sub * kTileTokens; t0 < ke; t0 += kTileTokens * tp) {
                Words<KW> kr[4], vr[4];
                bool valid[4];
                if constexpr (UNIFORM_PAGE) {
                    // the 16 tokens of the tile lie in one page
                    const int pidx = t0 / bs;
                    const int page = pidx < a.max_blocks ? tbl[pidx] : -1;
                    const bool pok = pidx < a.max_blocks && page >= 0 && page < a.num_blocks;
                    bad |= !pok;
                    const int64_t page_base = static_cast<int64_t>(page) * bs - static_cast<int64_t>(pidx) * bs;
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const int t = t0 + 4 * i + row;
                        valid[i] = pok && t < ke;
                        const int64_t off = ((page_base + t) * hkv + h) * D + col * EPL;
                        if (valid[i]) {
                            kr[i] = load_words<KW>(kc + off * KVB);
                            vr[i] = load_words<KW>(vc + off * KVB);
                        } else {
#pragma unroll
                            for (int w = 0; w < KW; ++w) kr[i].w[w] = vr[i].w[w] = 0u;
                        }
                    }
                } else {
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const int t = t0 + 4 * i + row;
                        const bool tv = t < ke;
                        const int pidx = t / bs;
                        const int page = (tv && pidx < a.max_blocks) ? tbl[pidx] : -1;
                        const bool pok = pidx < a.max_blocks && page >= 0 && page < a.num_blocks;
                        bad |= tv && !pok;
                        valid[i] = tv && pok;
                        const int64_t off =
                            ((static_cast<int64_t>(page) * bs + (t - pidx * bs)) * hkv + h) * D + col * EPL;
                        if (valid[i]) {
                            kr[i] = load_words<KW>(kc + off * KVB);
                            vr[i] = load_words<KW>(vc + off * KVB);
                        } else {
#pragma unroll
                            for (int w = 0; w < KW; ++w) kr[i].w[w] = vr[i].w[w] = 0u;
                        }
                    }
                }

                // scores of the 4 tokens x G heads (log2 units)
                float sc[4][G];
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    float part[G];
                    if constexpr (R::kDot2) {
#pragma unroll
                        for (int g = 0; g < G; ++g) {
                            float d = 0.f;
#pragma unroll
                            for (int j = 0; j < EPL / 2; ++j)
                                d = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, q[g].w[j]),
                                                                    __builtin_bit_cast(bf16x2_t, kr[i].w[j]), d, false);
                            part[g] = d;
                        }
                    } else {
                        float kf[EPL];
                        kv_to_f32<KVDT, EPL, KW>(kf, kr[i]);
#pragma unroll
                        for (int g = 0; g < G; ++g) {
                            float d = 0.f;
#pragma unroll
                            for (int e = 0; e < EPL; ++e) d = fmaf(q[g].f[e], kf[e], d);
                            part[g] = d;
                        }
                    }
#pragma unroll
                    for (int g = 0; g < G; ++g) {
                        const float s = row16_sum(part[g]) * a.qk_scale;
                        sc[i][g] = valid[i] ? s : -INFINITY;
                    }
                }

                // online softmax per head over this row's 4 tokens
                float p[4][G];
#pragma unroll
                for (int g = 0; g < G; ++g) {
                    const float mt = fmaxf(fmaxf(sc[0][g], sc[1][g]), fmaxf(sc[2][g], sc[3][g]));
                    const float mn = fmaxf(m[g], mt);
                    const float ms = (mn == -INFINITY) ? 0.f : mn;
                    const float alpha = exp2_fast(m[g] - ms);
                    float psum = 0.f;
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        p[i][g] = exp2_fast(sc[i][g] - ms);
                        psum += p[i][g];
                    }
                    l[g] = l[g] * alpha + psum;
                    m[g] = mn;
#pragma unroll
                    for (int e = 0; e < EPL; ++e) acc[g][e] *= alpha;
                }
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    float vf[EPL];
                    kv_to_f32<KVDT, EPL, KW>(vf, vr[i]);
#pragma unroll
                    for (int g = 0; g < G; ++g)
#pragma unroll
                        for (int e = 0; e < EPL; ++e) acc[g][e] = fmaf(p[i][g], vf[e], acc[g][e]);
                }
            }

            // merge the four rows of the wave
            bad = __any(bad);
#pragma unroll
            for (int g = 0; g < G; ++g) {
                const float M = rows4_max(m[g]);
                const float f = exp2_fast(m[g] - ((M == -INFINITY) ? 0.f : M));
                l[g] = rows4_sum(l[g] * f);
#pragma unroll
                for (int e = 0; e < EPL; ++e) acc[g][e] = rows4_sum(acc[g][e] * f);
                m[g] = M;
            }

            // merge the waves that shared this head
            if (tp > 1) {
                __syncthreads();
                if (row == 0) {
#pragma unroll
                    for (int g = 0; g < G; ++g)
#pragma unroll
                        for (int e = 0; e < EPL; ++e) lds_acc[wave][g][col * EPL + e] = acc[g][e];
                }
                if (lane == 0) {
#pragma unroll
                    for (int g = 0; g < G; ++g) {
                        lds_ml[wave][g][0] = m[g];
                        lds_ml[wave][g][1] = l[g];
                    }
                    lds_bad[wave] = bad ? 1 : 0;
                }
                __syncthreads();
                if (sub == 0) {
#pragma unroll
                    for (int g = 0; g < G; ++g) {
                        float M = -INFINITY;
                        for (int w = 0; w < tp; ++w) M = fmaxf(M, lds_ml[wave + w][g][0]);
                        const float Ms = (M == -INFINITY) ? 0.f : M;
                        float lt = 0.f;
                        float at[EPL];
#pragma unroll
                        for (int e = 0; e < EPL; ++e) at[e] = 0.f;
                        for (int w = 0; w < tp; ++w) {
                            const float f = exp2_fast(lds_ml[wave + w][g][0] - Ms);
                            lt += lds_ml[wave + w][g][1] * f;
#pragma unroll
                            for (int e = 0; e < EPL; ++e) at[e] = fmaf(lds_acc[wave + w][g][col * EPL + e], f, at[e]);
                        }
                        m[g] = M;
                        l[g] = lt;
#pragma unroll
                        for (int e = 0; e < EPL; ++e) acc[g][e] = at[e];
                    }
                    for (int w = 1; w < tp; ++w) bad |= lds_bad[wave + w] != 0;
                }
            }

            if (sub == 0 && row == 0) {
#pragma unroll
                for (int g = 0; g < G; ++g) {
                    const int hq_idx = h * G + g;
                    const float inv = l[g] > 0.f ? 1.f / l[g] : 0.f;
                    float o[EPL];
#pragma unroll
                    for (int e = 0; e < EPL; ++e) o[e] = bad ? NAN : acc[g][e] * inv;
                    if (u.prow < 0) {
                        char* dst = static_cast<char*>(a.out) +
                                    (static_cast<int64_t>(u.row0) * hq_d + static_cast<int64_t>(hq_idx) * D + col * EPL) * QB;
#pragma unroll
                        for (int e = 0; e < EPL; ++e) o[e] *= a.v_scale;
                        store_out<QDT, EPL>(dst, o);
                    } else {
                        float* dst = a.partial_o + (static_cast<int64_t>(u.prow) * a.hq + hq_idx) * D + col * EPL;
#pragma unroll
                        for (int e = 0; e < EPL; e += 4)
                            *reinterpret_cast<float4*>(dst + e) = make_float4(o[e], o[e + 1], o[e + 2], o[e + 3]);
                        if (col == 0)
                            a.partial_lse[static_cast<int64_t>(u.prow) * a.hq + hq_idx] =
                                bad ? NAN : (l[g] > 0.f ? m[g] + __log2f(l[g]) : -INFINITY);
                    }
                }
            }
        }
    }
}

// Merge of the partial results of cut sequences: one workgroup per merge
// record, one thread per (head, element); lse in log2 units.
template <int QDT>
__global__ __launch_bounds__(256) void merge_kernel(const Merge* __restrict__ merges, const float* __restrict__ po,
                                                   const float* __restrict__ pl, void* __restrict__ out, int hq,
                                                   int d, float v_scale) {
    const Merge mg = merges[blockIdx.x];
    const int hd = hq * d;
    for (int r = 0; r < mg.nrows; ++r) {
        for (int idx = threadIdx.x; idx < hd; idx += blockDim.x) {
            const int h = idx / d;
            float M = -INFINITY;
            bool nan = false;
            for (int c = 0; c < mg.parts; ++c) {
                const float x = pl[static_cast<int64_t>(mg.prow0 + c * mg.nrows + r) * hq + h];
                nan |= (x != x);
                M = fmaxf(M, x);
            }
            float o = 0.f;
            if (nan) {
                o = NAN;
            } else if (M != -INFINITY) {
                float sw = 0.f, acc = 0.f;
                for (int c = 0; c < mg.parts; ++c) {
                    const int64_t prow = mg.prow0 + c * mg.nrows + r;
                    const float w = exp2_fast(pl[prow * hq + h] - M);
                    sw += w;
                    acc = fmaf(w, po[prow * hd + idx], acc);
                }
                o = acc / sw * v_scale;
            }
            const int64_t oi = static_cast<int64_t>(mg.row0 + r) * hd + idx;
            if constexpr (QDT == PKV_DTYPE_F32) {
                static_cast<float*>(out)[oi] = o;
            } else {
                static_cast<uint16_t*>(out)[oi] = static_cast<uint16_t>(f32_to_bf16_rne(o));
            }
        }
    }
}

constexpr int kDecodeWaves = 8;

template <int QDT, int KVDT, int D, int G>
int launch_decode_t(const AttnArgs& a, int num_queues, bool uniform, hipStream_t st) {
    if (uniform)
        hipLaunchKernelGGL((decode_kernel<QDT, KVDT, D, G, kDecodeWaves, true>), dim3(num_queues),
                           dim3(kDecodeWaves * 64), 0, st, a);
    else
        hipLaunchKernelGGL((decode_kernel<QDT, KVDT, D, G, kDecodeWaves, false>), dim3(num_queues),
                           dim3(kDecodeWaves * 64), 0, st, a);
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

int launch_merge(const AttnArgs& a, const Merge* merges, int num_merges, int q_dtype, int head_dim, void* stream) {
    if (num_merges == 0) return PKV_OK;
    hipStream_t st = static_cast<hipStream_t>(stream);
    if (q_dtype == PKV_DTYPE_F32)
        hipLaunchKernelGGL((merge_kernel<PKV_DTYPE_F32>), dim3(num_merges), dim3(256), 0, st, merges, a.partial_o,
                           a.partial_lse, a.out, a.hq, head_dim, a.v_scale);
    else
        hipLaunchKernelGGL((merge_kernel<PKV_DTYPE_BF16>), dim3(num_merges), dim3(256), 0, st, merges, a.partial_o,
                           a.partial_lse, a.out, a.hq, head_dim, a.v_scale);
    return hipGetLastError() == hipSuccess ? PKV_OK : PKV_ERR_HIP;
}

}  // namespace pkv
