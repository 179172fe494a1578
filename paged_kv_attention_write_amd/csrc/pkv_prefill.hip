// Prefill chunks of a mixed step on the matrix cores (gfx950).
//
// A mixed step is two launches over one plan: the decode kernel walks the
// decode queues (the decode rows run the decode unit unchanged, never a
// gather) and this kernel walks the prefill queues.  ("nanoserve", packed
// batches and chunked prefill: a mixed step goes to the decode kernel for its
// one-row sequences and to a prefill kernel for its chunks.)
//
// A prefill unit is a block of rows of one chunk, one kv head and one key
// piece.  Its kPrefillQRows (row, q head) pairs are spread over the 8 waves,
// 16 per wave: pair x = 16 w + n is row x / G, q head h G + x % G, so the G
// heads that share K/V sit side by side.  Per tile of 32 keys the workgroup
// stages K and V row-major in LDS, then every wave computes, with
// v_mfma_f32_16x16x32_bf16,
//   S^T[key][pair] = K Q^T   (A = K from LDS, B = its q slice in registers)
//   O^T[d][pair]  += V^T P^T (A = V^T read from the row-major V tile with the
//                             transposing LDS load ds_read_b64_tr_b16,
//                             B = P straight from the registers that hold
//                             S^T, rounded to bf16)
// The transposed forms put one pair per lane column in both results: lane l
// holds pair l % 16 for keys / dimensions 4 (l / 16) + i, so the online
// softmax state of a pair lives in the lanes that accumulate its output and
// no data moves between the two products.  Row maxima and sums combine the
// four lanes of a pair (l, l^16, l^32, l^48).  Keys are masked bottom-right
// causally: row r of the chunk sits at position pos0 + r and sees keys up to
// it.  fp8 K/V are widened to bf16 (exactly) when staged.
//
// Pipeline per tile: the K/V loads of tiles t + 1 and t + 2 and the page
// ids of tiles t + 3 and t + 4 are in flight while tile t is computed from
// one LDS buffer; tile t + 1 is then staged into the other buffer, and one
// barrier closes the step.
#include <math.h>

#include "pkv_decode_unit.h"

namespace pkv {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef short i16x4_t __attribute__((ext_vector_type(4)));

constexpr int kPfWaves = 8;
constexpr int kPfPairsPerWave = 16;  // MFMA N
constexpr int kPfKeys = 32;          // keys per staged tile
constexpr int kPfPad = 16;           // bf16 elements of padding per LDS row
static_assert(kPfWaves * kPfPairsPerWave == kPrefillQRows, "one 16-pair slice per wave");

template <int D>
struct PrefillLds {
    uint16_t k[2][kPfKeys][D + kPfPad];
    uint16_t v[2][kPfKeys][D + kPfPad];
};

// Global bytes of one staged item (8 elements of one key).
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

// The staging role of a thread: key kk of the tile, elements 8 dg .. 8 dg + 7
// of it, for K and for V.  D = 64 leaves the upper half of the threads idle.
template <int D>
struct PfRole {
    static constexpr int GROUPS = D / 8;
    static constexpr int THREADS = kPfKeys * GROUPS;
    static_assert(THREADS <= kPfWaves * 64, "one item per thread");
    int kk, dg;
    bool active;
    __device__ PfRole() {
        const int t = static_cast<int>(threadIdx.x);
        active = t < THREADS;
        kk = t / GROUPS;
        dg = t % GROUPS;
    }
};

// Page id of the thread's key in the tile at t0, or -1 (past kend or the table).
__device__ __forceinline__ int32_t pf_page(const AttnArgs& a, const_ptr<int32_t> tbl, int t, int kend) {
    const int pidx = page_of(a, t);
    return (t < kend && pidx < a.max_blocks) ? tbl[pidx] : -1;
}

template <int KVDT, int D>
struct PfRegs {
    Words<PfItem<KVDT>::W> k, v;
    bool ok;
};

// Issue the K/V loads of the thread's key t (page id given).  Loads are
// never skipped: a key past kend or on a page outside the pool reads the
// first bytes of the pool instead (the pool holds at least one block), is
// staged as zeros, and a page outside the pool flags the unit.
template <int KVDT, int D>
__device__ __forceinline__ void pf_load(PfRegs<KVDT, D>& r, const AttnArgs& a, const PfRole<D>& role, int h,
                                        int t, int kend, int32_t page, bool& bad) {
    constexpr int KVB = dt_bytes(KVDT);
    constexpr int W = PfItem<KVDT>::W;
    const uint32_t nblocks = static_cast<uint32_t>(a.num_blocks < 0x7FFFFFFF ? a.num_blocks : 0x7FFFFFFF);
    const bool tv = role.active && t < kend;
    const bool ok = tv && static_cast<uint32_t>(page) < nblocks;  // a negative id wraps to >= 2^31
    bad |= tv && !ok;
    const int pidx = page_of(a, t);
    const int64_t slot = static_cast<int64_t>(page) * a.block_size + row_in_page(a, t, pidx);
    const int64_t off = ok ? ((slot * a.hkv + h) * D + role.dg * 8) * KVB : 0;
    r.k = load_words<W>(static_cast<const char*>(a.k_cache) + off);
    r.v = load_words<W>(static_cast<const char*>(a.v_cache) + off);
    r.ok = ok;
}

template <int KVDT, int D>
__device__ __forceinline__ void pf_stage(const PfRegs<KVDT, D>& r, const PfRole<D>& role, PrefillLds<D>& lds,
                                         int buf) {
    if (!role.active) return;
    Words<4> k = item_to_bf16<KVDT>(r.k), v = item_to_bf16<KVDT>(r.v);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        k.w[j] = r.ok ? k.w[j] : 0u;
        v.w[j] = r.ok ? v.w[j] : 0u;
    }
    store_words<4>(&lds.k[buf][role.kk][role.dg * 8], k);
    store_words<4>(&lds.v[buf][role.kk][role.dg * 8], v);
}

__device__ __forceinline__ bf16x8_t lds_bf16x8(const uint16_t* p) {
    return __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const uint4*>(p));
}

// Transposing 64-bit LDS read: within each 16-lane group, lane i receives
// element i % 4 of the 4-element chunk addressed by lane 4 j + i / 4, as its
// element j.
__device__ __forceinline__ uint2 lds_read_tr16(const uint16_t* p) {
    const i16x4_t r = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) i16x4_t*)(const_cast<uint16_t*>(p)));
    return __builtin_bit_cast(uint2, r);
}

// One tile of one wave: S^T for keys t0 + 16 kb2 + 4 g4 + i of pair n, the
// online softmax update, and O^T += V^T P^T.  qk = |scale * k_scale * log2 e|
// (a negative factor is carried by the sign of q, and qk >= 2^-100).  mask
// (uniform in the wave): the tile crosses the causal diagonal, the end of the
// key range or rows past the unit, so keys are tested one by one; otherwise
// every key of the tile is visible to every pair of the wave.  Per score the vector work is one fma into one v_exp_f32,
// a share of a max3, a packed bf16 conversion and a dot2 into the row sum.
template <int D, int NS = D / 32, int ND = D / 16>
__device__ __forceinline__ void pf_compute(const PrefillLds<D>& lds, int buf, int t0, int kend, int pos, bool row_ok,
                                           bool mask, int n, int g4, float qk, const bf16x8_t (&qb)[NS],
                                           f32x4_t (&acc)[ND], float& m_run, float& l_run) {
    float sv[8];  // raw q.k
#pragma unroll
    for (int kb2 = 0; kb2 < 2; ++kb2) {
        f32x4_t c = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < NS; ++s)
            c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(lds_bf16x8(&lds.k[buf][16 * kb2 + n][32 * s + 8 * g4]), qb[s],
                                                        c, 0, 0, 0);
#pragma unroll
        for (int i = 0; i < 4; ++i) sv[4 * kb2 + i] = c[i];
    }
    if (mask) {
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const int kp = t0 + 16 * (j >> 2) + 4 * g4 + (j & 3);
            sv[j] = (row_ok && kp < kend && kp <= pos) ? sv[j] : -INFINITY;
        }
    }
    float mr = fmaxf(fmaxf(fmaxf(sv[0], sv[1]), fmaxf(sv[2], sv[3])), fmaxf(fmaxf(sv[4], sv[5]), fmaxf(sv[6], sv[7])));
    mr = fmaxf(mr, __shfl_xor(mr, 16));
    mr = fmaxf(mr, __shfl_xor(mr, 32));
    const float mt = (mr == -INFINITY) ? -INFINITY : mr * qk;  // the tile's max in log2 units
    // lazy rescale, as in the decode unit: scores at most 2^8 above the
    // running maximum are taken against it
    const bool need = mt > m_run + 8.0f;
    if (__any(need)) {
        const float m_new = need ? mt : m_run;
        const float alpha = need ? exp2_fast(m_run - m_new) : 1.f;
        l_run *= alpha;
        m_run = m_new;
#pragma unroll
        for (int b = 0; b < ND; ++b) acc[b] *= alpha;
    }
    const float nmb = (m_run == -INFINITY) ? 0.f : -m_run;
    float p[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) p[j] = exp2_fast(fmaf(sv[j], qk, nmb));  // a masked key (-inf) gives 0
    bf16x8_t pb;
#pragma unroll
    for (int j = 0; j < 8; ++j) pb[j] = static_cast<__bf16>(p[j]);  // round to nearest even
    // the row sum adds the rounded weights that P V uses, two per dot2
    const bf16x2_t ones = {static_cast<__bf16>(1.0f), static_cast<__bf16>(1.0f)};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const bf16x2_t pp = {pb[2 * j], pb[2 * j + 1]};
        l_run = __builtin_amdgcn_fdot2_f32_bf16(pp, ones, l_run, false);
    }
    // V^T operand: lane group g4 takes keys 4 g4 + j (j < 4) and 16 + 4 g4 +
    // j - 4 (j >= 4), where the first product left their scores; lane 4 j + q
    // of the group points at V[key_j][16 b + 4 q]
    const int vkey = 4 * g4 + (n >> 2);
    const int vcol = 4 * (n & 3);
#pragma unroll
    for (int b = 0; b < ND; ++b) {
        const uint2 lo = lds_read_tr16(&lds.v[buf][vkey][16 * b + vcol]);
        const uint2 hi = lds_read_tr16(&lds.v[buf][16 + vkey][16 * b + vcol]);
        const bf16x8_t va = __builtin_bit_cast(bf16x8_t, make_uint4(lo.x, lo.y, hi.x, hi.y));
        acc[b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va, pb, acc[b], 0, 0, 0);
    }
}

// The prefill units of plan queue `queue` on the calling workgroup.
template <int KVDT, int D, int G>
__device__ __forceinline__ void prefill_queue(const AttnArgs& a, int queue, PrefillLds<D>& lds) {
    constexpr int QB = 2;       // bf16 queries
    constexpr int NS = D / 32;  // k steps of the first product
    constexpr int ND = D / 16;  // 16-row blocks of O^T

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int n = lane & 15;  // pair column of this lane
    const int g4 = lane >> 4;
    const PfRole<D> role;

    const const_ptr<Unit> units = as_const(a.units);
    const const_ptr<int32_t> qoff = as_const(a.queue_off);
    const int u_begin = qoff[queue];
    const int u_end = qoff[queue + 1];
    for (int ui = u_begin; ui < u_end; ++ui) {
        const Unit un = load_unit(units, ui);
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
        const int wave_first_pos = un.pos0 + wr0;
        // every pair of the wave is a row of the unit
        const bool wave_full = (wave * kPfPairsPerWave + kPfPairsPerWave - 1) / G < un.nrows;

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
                // a negative score factor is carried by the sign of q (exact)
                const uint32_t flip = a.qk_scale < 0.f ? 0x80008000u : 0u;
                qb[s] = __builtin_bit_cast(bf16x8_t, make_uint4(w.w[0] ^ flip, w.w[1] ^ flip, w.w[2] ^ flip,
                                                                w.w[3] ^ flip));
            }
        }
        // |factor|, at least 2^-100 so that -inf * qk stays -inf (a zero
        // factor then still gives exp2 of exactly 0 for every visible key)
        const float qk = fmaxf(fabsf(a.qk_scale), 0x1p-100f);

        f32x4_t acc[ND];
#pragma unroll
        for (int b = 0; b < ND; ++b) acc[b] = f32x4_t{0.f, 0.f, 0.f, 0.f};
        float m_run = -INFINITY;  // running max of this lane's pair (its four lanes agree)
        float l_run = 0.f;        // this lane's share of the running sum
        bool bad = false;

        // prologue: tile 0 staged; tiles 1 and 2 and the pages of tiles 3
        // and 4 in flight
        const int kb = un.kv_begin;
        const int kend_role = role.active ? kend : 0;  // idle staging threads look nothing up
        PfRegs<KVDT, D> ra, rb;
        __syncthreads();  // the LDS of the previous unit is free
        pf_load<KVDT, D>(ra, a, role, h, kb + role.kk, kend, pf_page(a, tbl, kb + role.kk, kend_role), bad);
        pf_stage<KVDT, D>(ra, role, lds, 0);
        pf_load<KVDT, D>(ra, a, role, h, kb + kPfKeys + role.kk, kend,
                         pf_page(a, tbl, kb + kPfKeys + role.kk, kend_role), bad);
        pf_load<KVDT, D>(rb, a, role, h, kb + 2 * kPfKeys + role.kk, kend,
                         pf_page(a, tbl, kb + 2 * kPfKeys + role.kk, kend_role), bad);
        int32_t pa = pf_page(a, tbl, kb + 3 * kPfKeys + role.kk, kend_role);
        int32_t pb = pf_page(a, tbl, kb + 4 * kPfKeys + role.kk, kend_role);
        __syncthreads();

        // Two phases per trip so that the two register sets take turns: the
        // phase that computes tile t from buffer t % 2 stages tile t + 1
        // (loaded two phases ago) into the other buffer and reloads its
        // register set with tile t + 3.
        auto phase = [&](int t0, int buf, PfRegs<KVDT, D>& rs, int32_t& pg) {
            if (wave_has_rows && t0 <= wave_last_pos) {
                const bool mask = !(wave_full && t0 + kPfKeys <= kend && t0 + kPfKeys - 1 <= wave_first_pos);
                pf_compute<D>(lds, buf, t0, kend, pos, row_ok, mask, n, g4, qk, qb, acc, m_run, l_run);
            }
            if (t0 + kPfKeys < kend) {
                pf_stage<KVDT, D>(rs, role, lds, buf ^ 1);
                const int t3 = t0 + 3 * kPfKeys + role.kk;
                pf_load<KVDT, D>(rs, a, role, h, t3, kend, pg, bad);
                pg = pf_page(a, tbl, t3 + 2 * kPfKeys, kend_role);
            }
            __syncthreads();
        };
        for (int t0 = kb; t0 < kend; t0 += 2 * kPfKeys) {
            phase(t0, 0, ra, pa);
            if (t0 + kPfKeys >= kend) break;
            phase(t0 + kPfKeys, 1, rb, pb);
        }
        bad = __syncthreads_or(bad) != 0;

        float l_tot = l_run + __shfl_xor(l_run, 16);
        l_tot += __shfl_xor(l_tot, 32);
        if (row_ok) {
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
                                         : make_float4(acc[b][0] * inv, acc[b][1] * inv, acc[b][2] * inv,
                                                       acc[b][3] * inv);
                    *reinterpret_cast<float4*>(dst + 16 * b) = o;
                }
                if (g4 == 0)
                    a.partial_lse[prow * a.hq + hq_idx] =
                        bad ? NAN : (l_tot > 0.f ? m_run + __log2f(l_tot) : -INFINITY);
            }
        }
    }
}

template <int KVDT, int D, int G>
__global__ __launch_bounds__(kPfWaves * 64) __attribute__((amdgpu_waves_per_eu(4)))
void prefill_kernel(AttnArgs a, int queue0) {
    __shared__ PrefillLds<D> lds;
    prefill_queue<KVDT, D, G>(a, queue0 + blockIdx.x, lds);
}

// Both halves of a mixed step in one launch: blocks below num_decode_queues
// walk the decode queues with the decode unit, the others the prefill queues,
// so that the bandwidth-bound decode rows and the matrix-core chunk tiles run
// side by side on every CU (one 8-wave workgroup of each fits at <= 128
// VGPRs).
template <int KVDT, int D, int G>
constexpr size_t mixed_lds_bytes() {
    return sizeof(DecodeLds<D, G, kPfWaves>) > sizeof(PrefillLds<D>) ? sizeof(DecodeLds<D, G, kPfWaves>)
                                                                      : sizeof(PrefillLds<D>);
}

template <int KVDT, int D, int G>
__global__ __launch_bounds__(kPfWaves * 64) __attribute__((amdgpu_waves_per_eu(4)))
void mixed_kernel(AttnArgs a, int num_decode_queues) {
    __shared__ __attribute__((aligned(16))) char smem[mixed_lds_bytes<KVDT, D, G>()];
    const int b = blockIdx.x;
    if (b < num_decode_queues) {
        const const_ptr<Unit> units = as_const(a.units);
        const const_ptr<int32_t> qoff = as_const(a.queue_off);
        const int u_end = qoff[b + 1];
        for (int ui = qoff[b]; ui < u_end; ++ui)
            decode_unit<PKV_DTYPE_BF16, KVDT, D, G, kPfWaves, true>(
                a, load_unit(units, ui), *reinterpret_cast<DecodeLds<D, G, kPfWaves>*>(smem));
    } else {
        prefill_queue<KVDT, D, G>(a, b, *reinterpret_cast<PrefillLds<D>*>(smem));
    }
}

template <int KVDT, int D, int G>
int launch_prefill_t(const AttnArgs& a, int num_queues, int queue0, hipStream_t st) {
    hipLaunchKernelGGL((prefill_kernel<KVDT, D, G>), dim3(num_queues), dim3(kPfWaves * 64), 0, st, a, queue0);
    return hipGetLastError() == hipSuccess ? PKV_OK : PKV_ERR_HIP;
}

template <int KVDT, int D>
int launch_prefill_g(const AttnArgs& a, int group, int num_queues, int queue0, hipStream_t st) {
    switch (group) {
        case 1: return launch_prefill_t<KVDT, D, 1>(a, num_queues, queue0, st);
        case 2: return launch_prefill_t<KVDT, D, 2>(a, num_queues, queue0, st);
        case 4: return launch_prefill_t<KVDT, D, 4>(a, num_queues, queue0, st);
        case 8: return launch_prefill_t<KVDT, D, 8>(a, num_queues, queue0, st);
        default: return PKV_ERR_UNSUPPORTED;
    }
}

template <int KVDT>
int launch_prefill_d(const AttnArgs& a, int d, int group, int num_queues, int queue0, hipStream_t st) {
    if (d == 64) return launch_prefill_g<KVDT, 64>(a, group, num_queues, queue0, st);
    if (d == 128) return launch_prefill_g<KVDT, 128>(a, group, num_queues, queue0, st);
    return PKV_ERR_UNSUPPORTED;
}

template <int KVDT>
int launch_mixed_d(const AttnArgs& a, int d, int group, int num_decode_queues, int num_prefill_queues,
                   hipStream_t st) {
    const dim3 grid(num_decode_queues + num_prefill_queues), block(kPfWaves * 64);
    if (d == 128 && group == 4)
        hipLaunchKernelGGL((mixed_kernel<KVDT, 128, 4>), grid, block, 0, st, a, num_decode_queues);
    else if (d == 128 && group == 2)
        hipLaunchKernelGGL((mixed_kernel<KVDT, 128, 2>), grid, block, 0, st, a, num_decode_queues);
    else if (d == 64 && group == 4)
        hipLaunchKernelGGL((mixed_kernel<KVDT, 64, 4>), grid, block, 0, st, a, num_decode_queues);
    else if (d == 64 && group == 2)
        hipLaunchKernelGGL((mixed_kernel<KVDT, 64, 2>), grid, block, 0, st, a, num_decode_queues);
    else
        return PKV_ERR_UNSUPPORTED;
    return hipGetLastError() == hipSuccess ? PKV_OK : PKV_ERR_HIP;
}

}  // namespace

bool mixed_one_launch(int q_dtype, int kv_dtype, int head_dim, int group, int block_size) {
    return q_dtype == PKV_DTYPE_BF16 && kv_dtype == PKV_DTYPE_BF16 && (head_dim == 64 || head_dim == 128) &&
           (group == 2 || group == 4) && block_size % kTileTokens == 0;
}

int launch_mixed(const AttnArgs& a, int head_dim, int group, int num_decode_queues, int num_prefill_queues,
                 void* stream) {
    return launch_mixed_d<PKV_DTYPE_BF16>(a, head_dim, group, num_decode_queues, num_prefill_queues,
                                          static_cast<hipStream_t>(stream));
}

bool prefill_supported(int q_dtype, int kv_dtype, int head_dim, int group) {
    return q_dtype == PKV_DTYPE_BF16 && (kv_dtype == PKV_DTYPE_BF16 || kv_dtype == PKV_DTYPE_FP8_E4M3) &&
           (head_dim == 64 || head_dim == 128) && (group == 1 || group == 2 || group == 4 || group == 8);
}

int launch_prefill(const AttnArgs& a, int q_dtype, int kv_dtype, int head_dim, int group, int num_queues,
                   int queue0, void* stream) {
    hipStream_t st = static_cast<hipStream_t>(stream);
    if (!prefill_supported(q_dtype, kv_dtype, head_dim, group)) return PKV_ERR_UNSUPPORTED;
    if (kv_dtype == PKV_DTYPE_BF16) return launch_prefill_d<PKV_DTYPE_BF16>(a, head_dim, group, num_queues, queue0, st);
    return launch_prefill_d<PKV_DTYPE_FP8_E4M3>(a, head_dim, group, num_queues, queue0, st);
}

}  // namespace pkv
