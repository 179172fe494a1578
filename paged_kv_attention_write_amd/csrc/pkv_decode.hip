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

// Loads of one wave-tile: U groups of 4 tokens (token t0 + 4u + row in lane
// row `row`).  With pages of a multiple of 16 tokens the page of every
// 16-token sub-tile is one scalar load and the group's base address is
// scalar; the per-lane part is a 32-bit byte offset.  FULL: every token of
// the tile is below ke.  Loads are never skipped: a token outside the piece
// (or on a page outside the pool) reads the first bytes of the pool instead,
// and its V is zeroed (its score is masked to -inf by the caller).
template <int KVDT, int D, int U, int KW, bool UNIFORM_PAGE, bool FULL>
__device__ __forceinline__ void load_tile(Words<KW> (&k)[U], Words<KW> (&v)[U], const AttnArgs& a,
                                          const_ptr<int32_t> tbl, const char* kc, const char* vc, int t0, int ke,
                                          int row, uint32_t lane_off, uint32_t head_off, int64_t tok_bytes,
                                          bool& bad) {
    const int bs = a.block_size;
    // block ids are int32: a pool of more than 2^31 - 1 blocks is addressed up to that many
    const uint32_t nblocks = static_cast<uint32_t>(a.num_blocks < 0x7FFFFFFF ? a.num_blocks : 0x7FFFFFFF);
    if constexpr (UNIFORM_PAGE) {
        constexpr int SUB = U >= 4 ? U / 4 : 1;
        constexpr int PER = U < 4 ? U : 4;
#pragma unroll
        for (int s = 0; s < SUB; ++s) {
            const int ts = t0 + 16 * s;
            const int pidx = ts / bs;
            const bool in = FULL || ts < ke;
            const uint32_t page = static_cast<uint32_t>((in && pidx < a.max_blocks) ? tbl[pidx] : -1);
            const bool pok = page < nblocks;  // a negative id wraps to >= 2^31
            if (in && !pok) bad = true;
            const int64_t slot0 =
                pok ? static_cast<int64_t>(static_cast<uint64_t>(page) * static_cast<uint32_t>(bs) +
                                           static_cast<uint32_t>(ts - pidx * bs))
                    : 0;
            const char* kb = kc + slot0 * tok_bytes;
            const char* vb = vc + slot0 * tok_bytes;
#pragma unroll
            for (int uu = 0; uu < PER; ++uu) {
                const int u = 4 * s + uu;
                if constexpr (FULL) {
                    k[u] = load_words_nt<KW>(kb + 4 * uu * tok_bytes + lane_off);
                    v[u] = load_words_nt<KW>(vb + 4 * uu * tok_bytes + lane_off);
                } else {
                    const bool ok = pok && t0 + 4 * u + row < ke;
                    const int64_t off = ok ? 4 * uu * tok_bytes + lane_off : 0;
                    k[u] = load_words<KW>(kb + off);
                    Words<KW> vv = load_words<KW>(vb + off);
#pragma unroll
                    for (int w = 0; w < KW; ++w) vv.w[w] = ok ? vv.w[w] : 0u;
                    v[u] = vv;
                }
            }
        }
    } else {
        // one lookup per token: lane row r reads the page of token t0 + 4u + r
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int t = t0 + 4 * u + row;
            const bool tv = FULL || t < ke;
            const int pidx = t / bs;
            const uint32_t page = static_cast<uint32_t>((tv && pidx < a.max_blocks) ? tbl[pidx] : -1);
            const bool ok = tv && page < nblocks;  // a negative id wraps to >= 2^31
            bad |= tv && !ok;
            const uint64_t slot = static_cast<uint64_t>(page) * static_cast<uint32_t>(bs) +
                                  static_cast<uint32_t>(t - pidx * bs);
            const int64_t off = ok ? static_cast<int64_t>(slot) * tok_bytes + head_off : 0;
            k[u] = load_words<KW>(kc + off);
            Words<KW> vv = load_words<KW>(vc + off);
#pragma unroll
            for (int w = 0; w < KW; ++w) vv.w[w] = ok ? vv.w[w] : 0u;
            v[u] = vv;
        }
    }
}

// Scores in log2 units above the running maximum by at most this much are
// accumulated against the stale maximum; the accumulator is rescaled only
// when a tile's maximum climbs further, so p <= 2^8 and nothing overflows.
constexpr float kRescaleThreshold = 8.0f;

// One wave-tile of the online softmax: scores of the 4U tokens x G heads,
// lazy rescale, P V accumulate.
template <int QDT, int KVDT, int D, int G, int U, int KW, int EPL>
__device__ __forceinline__ void process_tile(const Words<KW> (&k)[U], const Words<KW> (&v)[U],
                                             const QSlice<QDT, KVDT, D> (&q)[G], float (&acc)[G][EPL],
                                             float& m_run, float& l_run, float qk_scale, bool my_valid, int col) {
    using R = DecodeRegs<QDT, KVDT, D, G>;
    f32x16_t part;  // partial q.k of this lane's slice, index u * G + g
#pragma unroll
    for (int u = 0; u < U; ++u) {
        if constexpr (R::kDot2) {
#pragma unroll
            for (int g = 0; g < G; ++g) {
                float d = 0.f;
#pragma unroll
                for (int j = 0; j < EPL / 2; ++j)
                    d = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, q[g].w[j]),
                                                        __builtin_bit_cast(bf16x2_t, k[u].w[j]), d, false);
                part[u * G + g] = d;
            }
        } else {
            float kf[EPL];
            kv_to_f32<KVDT, EPL, KW>(kf, k[u]);
#pragma unroll
            for (int g = 0; g < G; ++g) {
                float d = 0.f;
#pragma unroll
                for (int e = 0; e < EPL; ++e) d = fmaf(q[g].f[e], kf[e], d);
                part[u * G + g] = d;
            }
        }
    }
    // lane col now holds the full score of (token 4 (col / G) + row, head col % G)
    float sc = row16_reduce_scatter(part) * qk_scale;
    sc = my_valid ? sc : -INFINITY;
    const float mt = row_group_max<G>(sc);
    const bool need = mt > m_run + kRescaleThreshold;
    if (__any(need)) {
        const float m_new = need ? mt : m_run;
        const float alpha = need ? exp2_fast(m_run - m_new) : 1.f;
        l_run *= alpha;
        m_run = m_new;
        static_for<G>([&](auto g) {
            const float al = row_bcast<g>(alpha);
#pragma unroll
            for (int e = 0; e < EPL; ++e) acc[g][e] *= al;
        });
    }
    const float p = exp2_fast(sc - ((m_run == -INFINITY) ? 0.f : m_run));
    l_run += row_group_sum<G>(p);
    static_for<U>([&](auto u) {
        float vf[EPL];
        kv_to_f32<KVDT, EPL, KW>(vf, v[u]);
        static_for<G>([&](auto g) {
            const float pb = row_bcast<u * G + g>(p);
#pragma unroll
            for (int e = 0; e < EPL; ++e) acc[g][e] = fmaf(pb, vf[e], acc[g][e]);
        });
    });
}

template <int QDT, int KVDT, int D, int G, int NW, bool UNIFORM_PAGE, int WPE>
__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(WPE)))
void decode_kernel(AttnArgs a) {
    using R = DecodeRegs<QDT, KVDT, D, G>;
    constexpr int EPL = R::EPL;
    constexpr int KW = R::KW;
    constexpr int QB = dt_bytes(QDT);
    constexpr int KVB = dt_bytes(KVDT);
    constexpr int U = 16 / G;  // tokens per lane per wave-tile
    constexpr int TT = 4 * U;  // tokens per wave-tile

    __shared__ float lds_acc[NW][G][D];
    __shared__ float lds_ml[NW][G][2];
    __shared__ int lds_bad[NW];

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int row = lane >> 4;
    const int col = lane & 15;
    const int my_tok = 4 * (col / G) + row;  // token offset in the tile of this lane's score
    const int hkv = a.hkv;
    const int tp = (hkv <= NW && NW % hkv == 0) ? NW / hkv : 1;  // waves per kv head
    const int sub = wave % tp;
    const int head0 = wave / tp;
    const int hstep = NW / tp;
    const int64_t hq_d = static_cast<int64_t>(a.hq) * D;
    const int64_t tok_bytes = static_cast<int64_t>(hkv) * D * KVB;  // one token, all kv heads
    const uint32_t row_bytes = static_cast<uint32_t>(tok_bytes);

    const char* __restrict__ kc = static_cast<const char*>(a.k_cache);
    const char* __restrict__ vc = static_cast<const char*>(a.v_cache);
    const const_ptr<Unit> units = as_const(a.units);
    const const_ptr<int32_t> qoff = as_const(a.queue_off);
    const const_ptr<int32_t> ctx = as_const(a.context_lens);

    const int u_begin = qoff[blockIdx.x];
    const int u_end = qoff[blockIdx.x + 1];
    for (int ui = u_begin; ui < u_end; ++ui) {
        const Unit un = load_unit(units, ui);
        const int n = ctx[un.seq];
        const int kb = un.kv_begin;
        const int ke = min(un.kv_end, n);
        const const_ptr<int32_t> tbl = as_const(a.block_tables) + static_cast<int64_t>(un.seq) * a.max_blocks;

        for (int h = head0; h < hkv; h += hstep) {
            QSlice<QDT, KVDT, D> q[G];
            const char* qbase = static_cast<const char*>(a.q) +
                                (static_cast<int64_t>(un.row0) * a.q_stride + static_cast<int64_t>(h) * G * D +
                                 col * EPL) * QB;
#pragma unroll
            for (int g = 0; g < G; ++g) load_q<QDT, KVDT, D>(q[g], qbase + static_cast<int64_t>(g) * D * QB);
            const uint32_t head_off = static_cast<uint32_t>((h * D + col * EPL) * KVB);  // inside a token
            const uint32_t lane_off = row * row_bytes + head_off;

            float acc[G][EPL];
#pragma unroll
            for (int g = 0; g < G; ++g)
#pragma unroll
                for (int e = 0; e < EPL; ++e) acc[g][e] = 0.f;
            float m_run = -INFINITY;  // running max of this lane's head (the head's lanes agree)
            float l_run = 0.f;        // running sum of 2^(s - m_run) of this lane's head
            bool bad = false;

            const int step = TT * tp;
            for (int t0 = kb + sub * TT; t0 < ke; t0 += step) {
                Words<KW> kr[U], vr[U];
                if (t0 + TT <= ke) {
                    load_tile<KVDT, D, U, KW, UNIFORM_PAGE, true>(kr, vr, a, tbl, kc, vc, t0, ke, row, lane_off,
                                                                  head_off, tok_bytes, bad);
                } else {
                    load_tile<KVDT, D, U, KW, UNIFORM_PAGE, false>(kr, vr, a, tbl, kc, vc, t0, ke, row, lane_off,
                                                                   head_off, tok_bytes, bad);
                }
                process_tile<QDT, KVDT, D, G, U, KW, EPL>(kr, vr, q, acc, m_run, l_run, a.qk_scale,
                                                          t0 + my_tok < ke, col);
            }

            // per-head (max, sum) of this row, in every lane of the row
            float m[G], l[G];
            static_for<G>([&](auto g) {
                m[g] = row_bcast<g>(m_run);
                l[g] = row_bcast<g>(l_run);
            });

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
                    if (un.prow < 0) {
                        char* dst = static_cast<char*>(a.out) +
                                    (static_cast<int64_t>(un.row0) * hq_d + static_cast<int64_t>(hq_idx) * D + col * EPL) * QB;
#pragma unroll
                        for (int e = 0; e < EPL; ++e) o[e] *= a.v_scale;
                        store_out<QDT, EPL>(dst, o);
                    } else {
                        float* dst = a.partial_o + (static_cast<int64_t>(un.prow) * a.hq + hq_idx) * D + col * EPL;
#pragma unroll
                        for (int e = 0; e < EPL; e += 4)
                            *reinterpret_cast<float4*>(dst + e) = make_float4(o[e], o[e + 1], o[e + 2], o[e + 3]);
                        if (col == 0)
                            a.partial_lse[static_cast<int64_t>(un.prow) * a.hq + hq_idx] =
                                bad ? NAN : (l[g] > 0.f ? m[g] + __log2f(l[g]) : -INFINITY);
                    }
                }
            }
        }
    }
}

// Merge of the partial results of cut sequences.  One wave per (merge record,
// row, head): lane c reads part c's lse (log2 units), a wave max and sum give
// the part weights w_c = 2^(lse_c - M) / sum, then every lane accumulates its
// D/64 elements over the parts with independent loads.
constexpr int kMergeWaves = 4;

template <int QDT, int D>
__global__ __launch_bounds__(kMergeWaves * 64) void merge_kernel(const Merge* __restrict__ merges,
                                                                 const float* __restrict__ po,
                                                                 const float* __restrict__ pl,
                                                                 void* __restrict__ out, int hq, float v_scale) {
    constexpr int E = D / 64;  // elements per lane
    const Merge mg = merges[blockIdx.x];
    const int lane = threadIdx.x & 63;
    const int h = blockIdx.y * kMergeWaves + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    if (h >= hq) return;
    const int64_t hd = static_cast<int64_t>(hq) * D;
    for (int r = 0; r < mg.nrows; ++r) {
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

// Launch shape: 8-wave workgroups (one wave per kv head of the 8-head
// workloads), two per CU at <= 128 VGPRs.  Group 8 (eight q heads per lane),
// group 1 (sixteen tokens in flight per lane) and fp32 K/V need more
// registers and run one workgroup per CU.
constexpr int kDecodeWaves = 8;

template <int QDT, int KVDT, int D, int G>
int launch_decode_t(const AttnArgs& a, int num_queues, bool uniform, hipStream_t st) {
    constexpr int WPE = (G == 8 || G == 1 || KVDT == PKV_DTYPE_F32) ? 2 : 4;
    if (uniform)
        hipLaunchKernelGGL((decode_kernel<QDT, KVDT, D, G, kDecodeWaves, true, WPE>), dim3(num_queues),
                           dim3(kDecodeWaves * 64), 0, st, a);
    else
        hipLaunchKernelGGL((decode_kernel<QDT, KVDT, D, G, kDecodeWaves, false, WPE>), dim3(num_queues),
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
    const dim3 grid(num_merges, (a.hq + kMergeWaves - 1) / kMergeWaves);
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
