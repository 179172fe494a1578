// The decode unit: one query row of one sequence against a key range, every
// kv head, on one workgroup of NW waves.  Shared by the decode kernel and the
// mixed kernel (whose decode rows run exactly this code).
//
// What is computed: softmax(scale * q K^T) V over the keys of the unit, K/V
// read in place from the block pool through the sequence's block table with
// an online softmax ("nanoserve", Triton paged-attention decode bullet).
//
// Mapping onto CDNA4:
// * A wave owns one kv head of the unit (NW / H_kv waves share a head and
//   take alternate wave-tiles when H_kv < NW).
// * A wave reads 4 tokens per load instruction: lane (row r, col c) loads
//   elements [c*D/16, (c+1)*D/16) of token 4i + r, i.e. one coalesced
//   16-byte (bf16, D=128) slice per lane and a 256-byte row per 16 lanes.
//   The G = Hq/H_kv query heads of the group are held in registers and reuse
//   every K row once loaded.
// * The 16 (token, head) partial dot products of a lane row are reduced by a
//   butterfly that leaves one full score per lane (one exponential per
//   score); each row keeps its own online-softmax state over the tokens it
//   saw; the four rows (and the waves sharing a head) are merged once per
//   unit.
// * Scores are kept in log2 units (scale * log2 e folded into one factor)
//   so the exponentials are single v_exp_f32 instructions.
#pragma once

#include <math.h>

#include "pkv_attention.h"

namespace pkv {
namespace {

template <int QDT, int KVDT, int D, int G>
struct DecodeRegs {
    static constexpr int EPL = D / 16;                           // elements per lane
    static constexpr int KW = EPL * dt_bytes(KVDT) / 4;          // K/V words per lane
    static constexpr int QW = EPL * dt_bytes(QDT) / 4;           // q words per lane
    // bf16 q against bf16 or fp8 keys: q . k in bf16 pairs (an fp8 key is
    // exactly a bf16 value)
    static constexpr bool kDot2 = QDT == PKV_DTYPE_BF16 && (KVDT == PKV_DTYPE_BF16 || KVDT == PKV_DTYPE_FP8_E4M3);
    // P V as bf16 pairs over two tokens (one v_dot2_f32_bf16 per element,
    // head and token pair), the weights rounded to bf16 and the softmax sum
    // taken over the rounded weights (as the prefill tile rounds P for its
    // matrix product): half the vector instructions of fp32 weights times
    // widened values
    static constexpr bool kPvDot2 = kDot2;
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

// Key elements 2j and 2j + 1 of a lane's slice as a bf16 pair.  fp8 E4M3
// values (3 mantissa bits, magnitudes 2^-9 .. 448) are bf16 values exactly:
// converted to fp32, their low 16 bits are zero.
template <int KVDT, int KW>
__device__ __forceinline__ uint32_t key_pair(const Words<KW>& r, int j) {
    if constexpr (KVDT == PKV_DTYPE_BF16) {
        return r.w[j];
    } else {
        // two E4M3 codes to two bf16 values in one instruction (scale 1)
        const int w = static_cast<int>(r.w[j >> 1]);
        const bf16x2_t b = (j & 1) ? __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, true)
                                   : __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, false);
        return __builtin_bit_cast(uint32_t, b);
    }
}

// Element e of two tokens' slices as one bf16 pair (token a low, token b
// high), for e = 2k (lo) and e = 2k + 1 (hi): the V operand of a P V product
// over a token pair.
template <int KVDT, int KW, int NP>
__device__ __forceinline__ void token_pairs(uint32_t (&lo)[NP], uint32_t (&hi)[NP], const Words<KW>& a,
                                            const Words<KW>& b) {
    // slices as NP bf16 pairs of one token: elements (2k, 2k + 1)
    static_assert(NP == (KVDT == PKV_DTYPE_BF16 ? KW : 2 * KW), "bf16 pairs of a slice");
    uint32_t pa[NP], pb[NP];
#pragma unroll
    for (int k = 0; k < NP; ++k) {
        pa[k] = key_pair<KVDT, KW>(a, k);
        pb[k] = key_pair<KVDT, KW>(b, k);
    }
#pragma unroll
    for (int k = 0; k < NP; ++k) {
        lo[k] = __builtin_amdgcn_perm(pb[k], pa[k], 0x05040100u);  // (a[2k], b[2k])
        hi[k] = __builtin_amdgcn_perm(pb[k], pa[k], 0x07060302u);  // (a[2k + 1], b[2k + 1])
    }
}

// Loads of one wave-tile: U groups of 4 tokens (token t0 + 4u + row in lane
// row `row`).  With pages of a multiple of 16 tokens the page of every
// 16-token sub-tile is one scalar load and the group's base address is
// scalar (from `pages`, looked up by the caller); the per-lane part is a
// 32-bit byte offset.  FULL: every token of
// the tile is below ke.  Every load is issued, unconditionally, so that the
// wait before the products can count exactly the loads still in flight: a
// lane whose token is past the piece reads the unit's clamp token instead
// (`clamp_off`: the last key of the piece).  The caller masks the scores of
// those lanes to -inf, so their p is exactly 0 and the (finite) clamp values
// add nothing.  A token on a page outside the pool sets `bad` (its rows are
// written as NaN) and reads the pool start or the clamp token.
// How the decode unit finds the page of a key:
//   kPageTile   pages of a multiple of 16 tokens: one page id per 16-token
//               sub-tile of a wave-tile;
//   kPageGroup  pages of 4 or 8 tokens: one page id per group of 4 tokens
//               (one load instruction's tokens all lie in one page);
//   kPageOne    one-token pages: each lane reads its tokens' table entries
//               (vector loads) a wave-tile ahead of their use, and a token's
//               slot is its page;
//   kPageAny    any other page size: each lane reads its tokens' table
//               entries when the tile starts, and divides.
// Tiles and groups read the page ids of a wave-tile through scalar loads a
// tile ahead of their use.
constexpr int kPageAny = 0;
constexpr int kPageOne = 1;
constexpr int kPageGroup = 2;
constexpr int kPageTile = 3;

// Tokens per page id of a wave-tile, and page ids per wave-tile of U groups
// of 4 tokens.
template <int PK>
constexpr int kEntryTokens = PK == kPageOne ? 1 : (PK == kPageGroup ? 4 : 16);
template <int U, int PK>
constexpr int kTileEntries =
    (PK == kPageAny || PK == kPageOne) ? 1 : (4 * U >= kEntryTokens<PK> ? 4 * U / kEntryTokens<PK> : 1);

// Page ids of the wave-tile at t0 (-1 past ke or past the table): scalar
// loads, issued a tile ahead of their use.
template <int U, int PK>
__device__ __forceinline__ void tile_pages(int32_t (&pages)[(kTileEntries<U, PK>)], const AttnArgs& a,
                                           const SeqTable& tbl, int t0, int ke) {
#pragma unroll
    for (int s = 0; s < kTileEntries<U, PK>; ++s) {
        const int ts = t0 + kEntryTokens<PK> * s;
        const int pidx = page_of(a, ts);
        pages[s] = (ts < ke && pidx < tbl.n) ? tbl[pidx] : -1;
    }
}

// Per-token pages: the table entries of this lane's tokens t0 + 4u + row of
// the wave-tile at t0 (tokens at or past lim take the piece's last key),
// read unconditionally at a clamped index.
template <int U>
__device__ __forceinline__ void lane_pages(int32_t (&lp)[U], const AttnArgs& a, const SeqTable& tbl, int t0,
                                           int lim, int ke, int row) {
    const int last = page_of(a, ke - 1);
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const int t = t0 + 4 * u + row;
        const int pidx = t < lim ? page_of(a, t) : last;
        lp[u] = tbl.clamped(pidx);
    }
}

// Loads of one wave-tile: U groups of 4 tokens (token t0 + 4u + row in lane
// row `row`).  FULL: every token of the tile is below ke.  Every load is
// issued, unconditionally, so that the wait before the products can count
// exactly the loads still in flight: a lane whose token is past the piece
// reads the unit's clamp token instead (`clamp_off`: the last key of the
// piece).  The caller masks the scores of those lanes to -inf, so their p is
// exactly 0 and the (finite) clamp values add nothing.  A token on a page
// outside the pool sets `bad` (its rows are written as NaN) and reads the
// pool start or the clamp token.
//   kPageTile / kPageGroup: the tokens of an entry share a page, so the
//     entry's base address is scalar and the lane adds a 32-bit offset;
//   kPageOne: the lane's page is its row's entry; the slot is the page;
//   kPageAny: the lane's own table entries (lp) and 64-bit slots.
// WR (whole-tile pages): key tnew, the step's new token that this launch
// writes, is read from knew / vnew (the lane's piece of the caller's row)
// instead of the pool, and so is a masked lane's clamp token (key ke - 1)
// when it is that key; the tile holding tnew always takes the masked form.
template <int KVDT, int D, int U, int KW, int PK, bool FULL, bool WR = false>
__device__ __forceinline__ void load_tile(Words<KW> (&k)[U], Words<KW> (&v)[U], const AttnArgs& a,
                                          const int32_t (&pages)[(kTileEntries<U, PK>)], const int32_t (&lp)[U],
                                          const char* kc, const char* vc, int t0, int ke, int row, uint32_t lane_off,
                                          uint32_t head_off, int64_t tok_bytes, int64_t clamp_off, int tbl_n,
                                          bool& bad, const char* knew = nullptr, const char* vnew = nullptr,
                                          int tnew = -1) {
    static_assert(!WR || PK == kPageTile, "the new token is read in place on whole-tile pages");
    const int bs = a.block_size;
    // block ids are int32: a pool of more than 2^31 - 1 blocks is addressed up to that many
    const uint32_t nblocks = static_cast<uint32_t>(a.num_blocks < 0x7FFFFFFF ? a.num_blocks : 0x7FFFFFFF);
    if constexpr (PK == kPageTile || PK == kPageGroup) {
        constexpr int SUB = kTileEntries<U, PK>;
        constexpr int PER = U / SUB;  // 4-token groups per entry
#pragma unroll
        for (int s = 0; s < SUB; ++s) {
            const int ts = t0 + kEntryTokens<PK> * s;
            const int pidx = page_of(a, ts);
            const bool in = FULL || ts < ke;
            const uint32_t page = static_cast<uint32_t>(pages[s]);
            const bool pok = page < nblocks;  // a negative id wraps to >= 2^31
            if (in && !pok) bad = true;
            const int64_t slot0 =
                pok ? static_cast<int64_t>(static_cast<uint64_t>(page) * static_cast<uint32_t>(bs) +
                                           static_cast<uint32_t>(row_in_page(a, ts, pidx)))
                    : 0;
            const char* kb = kc + slot0 * tok_bytes;
            const char* vb = vc + slot0 * tok_bytes;
#pragma unroll
            for (int uu = 0; uu < PER; ++uu) {
                const int u = PER * s + uu;
                if constexpr (FULL) {
                    // a page outside the pool reads the pool start: its rows come out NaN anyway
                    k[u] = load_words_nt<KW>(kb + 4 * uu * tok_bytes + lane_off);
                    v[u] = load_words_nt<KW>(vb + 4 * uu * tok_bytes + lane_off);
                } else {
                    const bool ok = pok && t0 + 4 * u + row < ke;
                    const int64_t off = ok ? slot0 * tok_bytes + 4 * uu * tok_bytes + lane_off : clamp_off;
                    const char* kp = kc + off;
                    const char* vp = vc + off;
                    if constexpr (WR) {
                        if ((ok ? t0 + 4 * u + row : ke - 1) == tnew) {
                            kp = knew;
                            vp = vnew;
                        }
                    }
                    k[u] = load_words_nt<KW>(kp);
                    v[u] = load_words_nt<KW>(vp);
                }
            }
        }
    } else if constexpr (PK == kPageOne) {
        // one-token pages: the slot of token t0 + 4u + row is its page (lp)
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int t = t0 + 4 * u + row;
            const bool tv = FULL || t < ke;
            const uint32_t page = static_cast<uint32_t>(lp[u]);
            const bool ok = tv && t < tbl_n && page < nblocks;  // a negative id wraps to >= 2^31
            bad |= tv && !ok;
            const int64_t off = ok ? static_cast<int64_t>(page) * tok_bytes + head_off : clamp_off;
            k[u] = load_words_nt<KW>(kc + off);
            v[u] = load_words_nt<KW>(vc + off);
        }
    } else {
        // one page per token: lane row r takes the page of token t0 + 4u + r
        // from lp
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int t = t0 + 4 * u + row;
            const bool tv = FULL || t < ke;
            const int pidx = page_of(a, t);
            const uint32_t page = static_cast<uint32_t>(lp[u]);
            const bool ok = tv && pidx < tbl_n && page < nblocks;  // a negative id wraps to >= 2^31
            bad |= tv && !ok;
            const uint64_t slot = static_cast<uint64_t>(page) * static_cast<uint32_t>(bs) +
                                  static_cast<uint32_t>(row_in_page(a, t, pidx));
            const int64_t off = ok ? static_cast<int64_t>(slot) * tok_bytes + head_off : clamp_off;
            k[u] = load_words_nt<KW>(kc + off);
            v[u] = load_words_nt<KW>(vc + off);
        }
    }
}

// Byte offset (inside a pool) of the clamp token of a piece ending at ke:
// key ke - 1 of the sequence, at the lane's head offset, or the head offset
// alone when that key's page is outside the pool.
__device__ __forceinline__ int64_t clamp_offset(const AttnArgs& a, const SeqTable& tbl, int ke,
                                                uint32_t head_off, int64_t tok_bytes) {
    const int bs = a.block_size;
    const uint32_t nblocks = static_cast<uint32_t>(a.num_blocks < 0x7FFFFFFF ? a.num_blocks : 0x7FFFFFFF);
    const int t = ke - 1;
    const int pidx = page_of(a, t);
    const uint32_t page = static_cast<uint32_t>(pidx < tbl.n ? tbl[pidx] : -1);
    if (page >= nblocks) return head_off;
    return static_cast<int64_t>(static_cast<uint64_t>(page) * static_cast<uint32_t>(bs) +
                                static_cast<uint32_t>(row_in_page(a, t, pidx))) * tok_bytes + head_off;
}

// Scores in log2 units above the running maximum by at most this much are
// accumulated against the stale maximum; the accumulator is rescaled only
// when a tile's maximum climbs further, so p <= 2^8 and nothing overflows.
constexpr float kRescaleThreshold = 8.0f;

// One wave-tile of the online softmax: scores of the 4U tokens x G heads,
// lazy rescale, P V accumulate.  CAP: the scores pass through the logit
// soft-cap (cap, cap_k in log2 units, see soft_cap_log2) before the mask.
// my_valid: this lane's token is one the row sees.
template <int QDT, int KVDT, int D, int G, int U, int KW, int EPL, bool CAP>
__device__ __forceinline__ void process_tile(const Words<KW> (&k)[U], const Words<KW> (&v)[U],
                                             const QSlice<QDT, KVDT, D> (&q)[G], float (&acc)[G][EPL],
                                             float& m_run, float& l_run, float qk_scale, float cap, float cap_k,
                                             bool my_valid) {
    using R = DecodeRegs<QDT, KVDT, D, G>;
    f32x16_t part;  // partial q.k of this lane's slice, index u * G + g
#pragma unroll
    for (int u = 0; u < U; ++u) {
        if constexpr (R::kDot2) {
            uint32_t kp[EPL / 2];
#pragma unroll
            for (int j = 0; j < EPL / 2; ++j) kp[j] = key_pair<KVDT, KW>(k[u], j);
#pragma unroll
            for (int g = 0; g < G; ++g) {
                float d = 0.f;
#pragma unroll
                for (int j = 0; j < EPL / 2; ++j)
                    d = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, q[g].w[j]),
                                                        __builtin_bit_cast(bf16x2_t, kp[j]), d, false);
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
    if constexpr (CAP) sc = soft_cap_log2(sc, cap, cap_k);
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
    if constexpr (R::kPvDot2) {
        // lane col c holds the weight of token 4 (c / G) + row and head c % G;
        // lane c + G holds the same head's weight of the next token.  Each
        // lane packs the two as bf16 (round to nearest even); the pair of
        // tokens 2j, 2j + 1 and head g sits in lane 2 j G + g.  The row sum
        // adds the rounded weights, so the output is a convex combination of
        // V rows under the weights P V uses.
        const float pn = dpp_f32<kDppRowRor + (16 - G)>(p);  // lane c + G (mod 16)
        const uint32_t pk = __builtin_bit_cast(uint32_t, __builtin_convertvector((float2_t){p, pn}, bf16x2_t));
        l_run += row_group_sum<G>(__uint_as_float(pk << 16));
        static_for<U / 2>([&](auto jc) {
            constexpr int j = decltype(jc)::value;
            uint32_t vlo[EPL / 2], vhi[EPL / 2];
            token_pairs<KVDT, KW, EPL / 2>(vlo, vhi, v[2 * j], v[2 * j + 1]);
            static_for<G>([&](auto g) {
                const bf16x2_t pb = __builtin_bit_cast(
                    bf16x2_t, __builtin_amdgcn_mov_dpp(static_cast<int>(pk), kDppRowNewBcast + 2 * j * G + g, 0xF,
                                                       0xF, true));
#pragma unroll
                for (int k = 0; k < EPL / 2; ++k) {
                    acc[g][2 * k] = __builtin_amdgcn_fdot2_f32_bf16(pb, __builtin_bit_cast(bf16x2_t, vlo[k]),
                                                                   acc[g][2 * k], false);
                    acc[g][2 * k + 1] = __builtin_amdgcn_fdot2_f32_bf16(pb, __builtin_bit_cast(bf16x2_t, vhi[k]),
                                                                       acc[g][2 * k + 1], false);
                }
            });
        });
    } else {
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
}

// LDS of the decode unit: the per-wave results that are merged across the
// waves sharing a kv head.
template <int D, int G, int NW>
struct DecodeLds {
    float acc[NW][G][D];
    float ml[NW][G][2];
    int bad[NW];
};

// One run of decode work on the calling workgroup: one unit's query row
// against a range of its keys, for the kv head(s) of each wave.  `open` sets
// up a unit for kv head h of this wave (q slice, empty softmax state),
// `tiles` accumulates keys [ta, tb) of the unit (ta a multiple of 16 past
// kv_begin), `flush` combines the wave's four rows and the waves sharing the
// head and writes the result: the output row (`direct`) or a normalised
// partial with its log-sum-exp at partial row `prow`.  Every wave of the
// workgroup makes the same calls (flush contains barriers when waves share a
// head).
template <int QDT, int KVDT, int D, int G, int NW, int PK>
struct DecodeRun {
    // page ids through scalar loads a tile ahead (else per-lane table reads)
    static constexpr bool UNIFORM_PAGE = PK == kPageTile || PK == kPageGroup;
    using R = DecodeRegs<QDT, KVDT, D, G>;
    static constexpr int EPL = R::EPL;
    static constexpr int KW = R::KW;
    static constexpr int QB = dt_bytes(QDT);
    static constexpr int KVB = dt_bytes(KVDT);
    static constexpr int U = 16 / G;  // tokens per lane per wave-tile
    static constexpr int TT = 4 * U;  // tokens per wave-tile

    // lane geometry
    int lane, wave, row, col, my_tok;
    int tp, sub, head0, hstep;  // waves per kv head, this wave's place among them, first head, head stride
    int64_t tok_bytes;
    // the unit
    Unit un;
    int n, kb, ke, lo, h;  // lo: first key the row sees (its window)
    // the step's new token, read from the caller's row (tnew < 0: none)
    const char* knew_lane;
    const char* vnew_lane;
    int tnew;
    bool stale;            // the device's lengths or row offsets differ from the plan's
    SeqTable tbl;
    uint32_t head_off, lane_off;
    int64_t clamp_off;
    // softmax state of this wave's head
    QSlice<QDT, KVDT, D> q[G];
    float acc[G][EPL];
    float m_run, l_run;
    bool bad;

    __device__ __forceinline__ explicit DecodeRun(const AttnArgs& a) {
        lane = threadIdx.x & 63;
        wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
        row = lane >> 4;
        col = lane & 15;
        my_tok = 4 * (col / G) + row;  // token offset in the tile of this lane's score
        const int hkv = a.hkv;
        tp = (hkv <= NW && NW % hkv == 0) ? NW / hkv : 1;
        sub = wave % tp;
        head0 = wave / tp;
        hstep = NW / tp;
        tok_bytes = static_cast<int64_t>(hkv) * D * KVB;  // one token, all kv heads
    }

    // The key range comes from the plan alone (a decode row sits at position
    // n - 1), so the first loads need not wait for a length read; the
    // device length (and, in a packed batch, the row offsets) are read
    // alongside and checked at the flush: a sequence whose length or rows
    // differ from the plan's (a stale plan) gets NaN rows.
    __device__ __forceinline__ void open(const AttnArgs& a, const Unit& u, int head) {
        un = u;
        h = head;
        n = u.pos0 + 1;
        stale = unit_is_stale(a, u);
        kb = u.kv_begin;
        ke = min(u.kv_end, n);
        lo = a.window > 0 ? max(0, n - a.window) : 0;
        tbl = seq_table(a, u.seq);
        const char* qbase = static_cast<const char*>(a.q) +
                            (static_cast<int64_t>(u.row0) * a.q_stride + static_cast<int64_t>(h) * G * D +
                             col * EPL) * QB;
#pragma unroll
        for (int g = 0; g < G; ++g) load_q<QDT, KVDT, D>(q[g], qbase + static_cast<int64_t>(g) * D * QB);
        head_off = static_cast<uint32_t>((h * D + col * EPL) * KVB);  // inside a token
        lane_off = row * static_cast<uint32_t>(tok_bytes) + head_off;
        clamp_off = kb < ke ? clamp_offset(a, tbl, ke, head_off, tok_bytes) : head_off;
#pragma unroll
        for (int g = 0; g < G; ++g)
#pragma unroll
            for (int e = 0; e < EPL; ++e) acc[g][e] = 0.f;
        m_run = -INFINITY;  // running max of this lane's head (the head's lanes agree)
        l_run = 0.f;        // running sum of 2^(s - m_run) of this lane's head
        bad = false;
        tnew = -1;
    }

    // Key n - 1 of the open unit (this step's new token, which the launch
    // writes) is read from the caller's k_new / v_new row.
    __device__ __forceinline__ void take_new_token(const AttnArgs& a) {
        const int64_t src = static_cast<int64_t>(un.row0) * a.new_stride * KVB;
        knew_lane = static_cast<const char*>(a.k_new) + src + head_off;
        vnew_lane = static_cast<const char*>(a.v_new) + src + head_off;
        tnew = n - 1;
    }

    // Keys [ta, tb) of the open unit (tb <= ke).  Tokens past tb are masked:
    // they may belong to another workgroup's range.
    template <bool WR = false>
    __device__ __forceinline__ void tiles(const AttnArgs& a, int ta, int tb) {
        const char* __restrict__ kc = static_cast<const char*>(a.k_cache);
        const char* __restrict__ vc = static_cast<const char*>(a.v_cache);
        const int step = TT * tp;
        // Whole-tile pages: the page ids of the wave's next tile are loaded
        // while this tile is computed, so the next tile's K/V loads need not
        // wait for a table read.
        int32_t pages[(kTileEntries<U, PK>)];
        int32_t lp[U];  // per-token pages: this lane's table entries
        if constexpr (UNIFORM_PAGE) tile_pages<U, PK>(pages, a, tbl, ta + sub * TT, tb);
        if constexpr (PK == kPageOne) lane_pages<U>(lp, a, tbl, ta + sub * TT, tb, ke, row);
        const uint32_t vspan = static_cast<uint32_t>(max(tb - lo, 0));  // keys lo .. tb - 1 are valid
        // the loop is built twice, with and without the logit soft-cap, so
        // that the plain call's loop carries no test of it
        auto loop = [&](auto cap_on) {
        for (int t0 = ta + sub * TT; t0 < tb; t0 += step) {
            Words<KW> kr[U], vr[U];
            if constexpr (PK == kPageAny) lane_pages<U>(lp, a, tbl, t0, tb, ke, row);
            if (t0 + TT <= tb && !(WR && tnew >= 0 && t0 + TT > tnew)) {
                load_tile<KVDT, D, U, KW, PK, true>(kr, vr, a, pages, lp, kc, vc, t0, tb, row, lane_off, head_off,
                                                    tok_bytes, clamp_off, tbl.n, bad);
            } else {
                load_tile<KVDT, D, U, KW, PK, false, WR>(kr, vr, a, pages, lp, kc, vc, t0, tb, row, lane_off,
                                                         head_off, tok_bytes, clamp_off, tbl.n, bad, knew_lane,
                                                         vnew_lane, tnew);
            }
            if constexpr (UNIFORM_PAGE) {
                if (t0 + step < tb) tile_pages<U, PK>(pages, a, tbl, t0 + step, tb);
            }
            if constexpr (PK == kPageOne) {
                // the next wave-tile's entries, while this one is computed
                if (t0 + step < tb) lane_pages<U>(lp, a, tbl, t0 + step, tb, ke, row);
            }
            // lo <= t0 + my_tok < tb as one unsigned compare
            const bool valid = static_cast<uint32_t>(t0 - lo + my_tok) < vspan;
            process_tile<QDT, KVDT, D, G, U, KW, EPL, decltype(cap_on)::value>(kr, vr, q, acc, m_run, l_run,
                                                                               a.qk_scale, a.soft_cap, a.soft_cap_k,
                                                                               valid);
        }
        };
        if (a.soft_cap > 0.f) {
            loop(std::true_type{});
        } else {
            loop(std::false_type{});
        }
    }

    __device__ __forceinline__ void flush(const AttnArgs& a, DecodeLds<D, G, NW>& lds, bool direct, int prow) {
        // per-head (max, sum) of this row, in every lane of the row
        float m[G], l[G];
        static_for<G>([&](auto g) {
            m[g] = row_bcast<g>(m_run);
            l[g] = row_bcast<g>(l_run);
        });

        // merge the four rows of the wave
        bool bd = __any(bad) || stale;
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
                    for (int e = 0; e < EPL; ++e) lds.acc[wave][g][col * EPL + e] = acc[g][e];
            }
            if (lane == 0) {
#pragma unroll
                for (int g = 0; g < G; ++g) {
                    lds.ml[wave][g][0] = m[g];
                    lds.ml[wave][g][1] = l[g];
                }
                lds.bad[wave] = bd ? 1 : 0;
            }
            __syncthreads();
            if (sub == 0) {
#pragma unroll
                for (int g = 0; g < G; ++g) {
                    float M = -INFINITY;
                    for (int w = 0; w < tp; ++w) M = fmaxf(M, lds.ml[wave + w][g][0]);
                    const float Ms = (M == -INFINITY) ? 0.f : M;
                    float lt = 0.f;
                    float at[EPL];
#pragma unroll
                    for (int e = 0; e < EPL; ++e) at[e] = 0.f;
                    for (int w = 0; w < tp; ++w) {
                        const float f = exp2_fast(lds.ml[wave + w][g][0] - Ms);
                        lt += lds.ml[wave + w][g][1] * f;
#pragma unroll
                        for (int e = 0; e < EPL; ++e) at[e] = fmaf(lds.acc[wave + w][g][col * EPL + e], f, at[e]);
                    }
                    m[g] = M;
                    l[g] = lt;
#pragma unroll
                    for (int e = 0; e < EPL; ++e) acc[g][e] = at[e];
                }
                for (int w = 1; w < tp; ++w) bd |= lds.bad[wave + w] != 0;
            }
        }

        if (sub == 0 && row == 0) {
            const int64_t hq_d = static_cast<int64_t>(a.hq) * D;
#pragma unroll
            for (int g = 0; g < G; ++g) {
                const int hq_idx = h * G + g;
                const float inv = l[g] > 0.f ? 1.f / l[g] : 0.f;
                float o[EPL];
#pragma unroll
                for (int e = 0; e < EPL; ++e) o[e] = bd ? NAN : acc[g][e] * inv;
                if (direct) {
                    char* dst = static_cast<char*>(a.out) +
                                (static_cast<int64_t>(un.row0) * hq_d + static_cast<int64_t>(hq_idx) * D + col * EPL) * QB;
#pragma unroll
                    for (int e = 0; e < EPL; ++e) o[e] *= a.v_scale;
                    store_out<QDT, EPL>(dst, o);
                } else {
                    float* dst = a.partial_o + (static_cast<int64_t>(prow) * a.hq + hq_idx) * D + col * EPL;
#pragma unroll
                    for (int e = 0; e < EPL; e += 4)
                        *reinterpret_cast<float4*>(dst + e) = make_float4(o[e], o[e + 1], o[e + 2], o[e + 3]);
                    if (col == 0)
                        a.partial_lse[static_cast<int64_t>(prow) * a.hq + hq_idx] =
                            bd ? NAN : (l[g] > 0.f ? m[g] + __log2f(l[g]) : -INFINITY);
                }
            }
        }
    }
};

// Whether a decode unit's result is the output row: it was not cut into
// pieces, so the plan gave it no partial row.  (A whole unit need not start
// at key 0: under a sliding window it starts at its first visible tile.)
__device__ __forceinline__ bool unit_is_whole(const Unit& u) { return u.prow < 0; }

// A decode step's new token (key n - 1 of the unit's sequence, every kv
// head, K and V) written into the pool by the workgroup whose unit holds that
// key ("nanoserve", "One engine step": each layer writes this step's K/V,
// then attends).  That unit reads the key from the caller's row rather than
// from the pool, and no other workgroup of the launch reads it, so the
// stores need no ordering against any load of the launch: as the unit starts,
// `load` checks the slot and `fetch` reads the token's 16-byte pieces (at
// most two per thread) into registers, so that they have arrived when
// `store` writes them once the unit is done.  A slot_mapping entry < 0 writes nothing (the key is read from the pool as it
// is); an entry other than the key's slot, a key on a page outside the pool
// or a stale plan writes nothing either and marks the row wrong (reported
// NaN).
template <int KVDT, int D, int NW>
struct TokenWrite {
    static constexpr int KVB = dt_bytes(KVDT);
    int64_t slot;
    bool go, wrong;

    __device__ __forceinline__ void load(const AttnArgs& a, const Unit& un) {
        const int n = un.pos0 + 1;
        slot = as_const(a.slot_mapping)[un.row0];
        const SeqTable tbl = seq_table(a, un.seq);
        const int pidx = page_of(a, n - 1);
        const int32_t page = tbl.clamped(pidx);
        const bool in_pool = pidx < tbl.n && page >= 0 && page < a.num_blocks;
        const int64_t key_slot = static_cast<int64_t>(page) * a.block_size + row_in_page(a, n - 1, pidx);
        wrong = slot >= 0 && (!in_pool || slot != key_slot || unit_is_stale(a, un));
        go = slot >= 0 && !wrong;
    }

    uint4 w[2];

    __device__ __forceinline__ void fetch(const AttnArgs& a, const Unit& un) {
        const int chunks = a.hkv * D * KVB / 16;  // 16-byte pieces of one token's K (or V)
        const int64_t src_row = static_cast<int64_t>(un.row0) * a.new_stride * KVB;
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const int c = static_cast<int>(threadIdx.x) + i * NW * 64;
            w[i] = uint4{0u, 0u, 0u, 0u};
            if (c < 2 * chunks) {
                const bool v = c >= chunks;
                const int64_t piece = static_cast<int64_t>(v ? c - chunks : c) * 16;
                w[i] = *reinterpret_cast<const uint4*>(static_cast<const char*>(v ? a.v_new : a.k_new) + src_row +
                                                       piece);
            }
        }
    }

    __device__ __forceinline__ void store(const AttnArgs& a, const Unit& un) const {
        if (!go) return;
        const int chunks = a.hkv * D * KVB / 16;
        const int64_t row_bytes = static_cast<int64_t>(a.hkv) * D * KVB;
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const int c = static_cast<int>(threadIdx.x) + i * NW * 64;
            if (c < 2 * chunks) {
                const bool v = c >= chunks;
                const int64_t piece = static_cast<int64_t>(v ? c - chunks : c) * 16;
                char* const dst = const_cast<char*>(static_cast<const char*>(v ? a.v_cache : a.k_cache));
                *reinterpret_cast<uint4*>(dst + slot * row_bytes + piece) = w[i];
            }
        }
    }
};

// One decode unit, all of it, on the calling workgroup: every kv head, whole
// units to the output row, pieces to their partial row.  WR: the unit that
// holds its sequence's last key also writes the step's new token, reading
// that key from the caller's row.
template <int QDT, int KVDT, int D, int G, int NW, int PK, bool WR = false>
__device__ __forceinline__ void decode_unit(const AttnArgs& a, const Unit& un, DecodeLds<D, G, NW>& lds) {
    DecodeRun<QDT, KVDT, D, G, NW, PK> run(a);
    const bool direct = unit_is_whole(un);
    if constexpr (WR) {
        const bool writes = un.kv_end == un.pos0 + 1;
        TokenWrite<KVDT, D, NW> tw;
        tw.wrong = false;
        tw.go = false;
        if (writes) {
            tw.load(a, un);
            tw.fetch(a, un);
        }
        for (int h = run.head0; h < a.hkv; h += run.hstep) {
            run.open(a, un, h);
            run.stale |= tw.wrong;
            if (tw.go) run.take_new_token(a);
            run.template tiles<true>(a, run.kb, run.ke);
            run.flush(a, lds, direct, un.prow);
        }
        tw.store(a, un);
    } else {
        for (int h = run.head0; h < a.hkv; h += run.hstep) {
            run.open(a, un, h);
            run.tiles(a, run.kb, run.ke);
            run.flush(a, lds, direct, un.prow);
        }
    }
}

}  // namespace
}  // namespace pkv
