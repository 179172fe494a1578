// Prefill chunks of a mixed step on the matrix cores (gfx950).
//
// A mixed step walks one plan with two kinds of workgroup: decode workgroups
// walk the decode queues (the decode rows run the decode unit unchanged,
// never a gather) and prefill workgroups the prefill queues.  For bf16 K/V
// on pages of whole 16-token tiles (groups 2 and 4) both run in one launch,
// mixed_kernel, side by side on every compute unit; other cases launch the
// decode kernel and prefill_kernel one after the other.  ("nanoserve", packed
// batches and chunked prefill: a mixed step sends its one-row sequences to
// the decode kernel and its chunks to a prefill path.)
//
// Steps whose chunks are all a few rows (at most 16 (row, q head) pairs per
// kv head: a speculative verify step) are planned as decode rows are and run
// the few-row kernel instead (below).  Chunks alone (no decode row) run the
// prefill kernel; for bf16 K/V at D = 128 on whole-tile pages its units of at
// least 64 pairs take the wide form, 4 waves of 32 pairs.
//
// A prefill unit is a block of rows of one chunk, one kv head and one key
// piece.  Its kPrefillQRows (row, q head) pairs are spread over the 8 waves,
// 16 per wave (or the 4 waves of the wide form, 32 per wave): pair
// x = 16 w + n is row x / G, q head h G + x % G, so the G heads that share
// K/V sit side by side.  Per tile of 32 keys the workgroup
// stages K and V in LDS, then every wave computes, with
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
// Two staging paths feed the same tile code: a ring of four LDS stages
// filled by direct-to-LDS loads (bf16 K/V, D = 128, pages of a power of two
// >= 16 tokens) and two padded LDS buffers filled from registers (every other
// case).  Both keep the loads of later tiles in flight while tile t is
// computed and close each step with one barrier.  The transposing V reads
// are written out in asm with their wait (see v_operands).
#include <math.h>

#include "pkv_decode_unit.h"

namespace pkv {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));

constexpr int kPfWaves = 8;           // waves of a workgroup of the mixed kernel (16 pairs each)
constexpr int kPfWideWaves = 4;       // waves of a wide prefill workgroup (32 pairs each)
constexpr int kPfPairsPerBlock = 16;  // MFMA N
constexpr int kPfKeys = 32;           // keys per staged tile
constexpr int kPfPad = 16;            // bf16 elements of padding per LDS row

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

// Table entry of the page of key t, read unconditionally at an index clamped
// into the sequence's row: every thread issues the same
// loads in the same order, so the waits for them count in order and none is
// taken right after its load.  pf_load decides whether the entry is valid.
__device__ __forceinline__ int32_t pf_page(const AttnArgs& a, const SeqTable& tbl, int t) {
    return tbl.clamped(page_of(a, t));
}

template <int KVDT, int D>
struct PfRegs {
    Words<PfItem<KVDT>::W> k, v;
    bool ok;
};

// Issue the K/V loads of the thread's key t (its table entry given).  Loads are
// never skipped: a key past kend or on a page outside the pool reads the
// first bytes of the pool instead (the pool holds at least one block), is
// staged as zeros, and a page outside the pool flags the unit.
template <int KVDT, int D>
__device__ __forceinline__ void pf_load(PfRegs<KVDT, D>& r, const AttnArgs& a, const PfRole<D>& role, int h,
                                        int t, int kend, int32_t page, int tbl_n, bool& bad) {
    constexpr int KVB = dt_bytes(KVDT);
    constexpr int W = PfItem<KVDT>::W;
    const uint32_t nblocks = static_cast<uint32_t>(a.num_blocks < 0x7FFFFFFF ? a.num_blocks : 0x7FFFFFFF);
    const int pidx = page_of(a, t);
    const bool tv = role.active && t < kend;
    // a key past the table, or a negative id (wraps to >= 2^31), is invalid
    const bool ok = tv && pidx < tbl_n && static_cast<uint32_t>(page) < nblocks;
    bad |= tv && !ok;
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

// Maximum that propagates NaN (IEEE 754-2019 maximum; v_maximum3_f32 on
// gfx950, which needs no quieting of its inputs).
__device__ __forceinline__ float vmax(float x, float y) { return __builtin_elementwise_maximum(x, y); }

__device__ __forceinline__ bf16x8_t lds_bf16x8(const uint16_t* p) {
    return __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const uint4*>(p));
}

// Transposing 64-bit LDS reads (ds_read_b64_tr_b16: within each 16-lane
// group, lane i receives element i % 4 of the 4-element chunk addressed by
// lane 4 j + i / 4, as its element j) of the V^T operand blocks B0 ..
// B0 + NB - 1 of a tile view, two per block (keys 0-15 and 16-31), issued in
// one asm statement that also waits for them.  Written by hand because the
// compiler's wait insertion takes every ds_read_b64_tr_b16 it emits itself
// for a possible reader of any direct-to-LDS load still in flight and waits
// for all of them (vmcnt(0)), which would drain the loads of the next tiles
// at every tile; the loads a tile needs are waited for explicitly before it
// is read.
template <class Tile, int B0, int NB>
__device__ __forceinline__ void v_operands(const uint16_t* vl, bf16x8_t* va) {
    static_assert(NB == 2 || NB == 4, "two or four blocks per statement");
    const uint32_t addr = static_cast<uint32_t>(
        reinterpret_cast<uintptr_t>((const __attribute__((address_space(3))) uint16_t*)vl));
    constexpr int lo0 = 2 * Tile::v_off(0, B0), hi0 = 2 * Tile::v_off(1, B0);
    constexpr int lo1 = 2 * Tile::v_off(0, B0 + 1), hi1 = 2 * Tile::v_off(1, B0 + 1);
    u32x2_t r[2 * NB];
    if constexpr (NB == 2) {
        __asm__ volatile(
            "ds_read_b64_tr_b16 %0, %4 offset:%5\n\t"
            "ds_read_b64_tr_b16 %1, %4 offset:%6\n\t"
            "ds_read_b64_tr_b16 %2, %4 offset:%7\n\t"
            "ds_read_b64_tr_b16 %3, %4 offset:%8\n\t"
            "s_waitcnt lgkmcnt(0)"
            : "=&v"(r[0]), "=&v"(r[1]), "=&v"(r[2]), "=&v"(r[3])
            : "v"(addr), "n"(lo0), "n"(hi0), "n"(lo1), "n"(hi1)
            : "memory");
    } else {
        constexpr int lo2 = 2 * Tile::v_off(0, B0 + 2), hi2 = 2 * Tile::v_off(1, B0 + 2);
        constexpr int lo3 = 2 * Tile::v_off(0, B0 + 3), hi3 = 2 * Tile::v_off(1, B0 + 3);
        __asm__ volatile(
            "ds_read_b64_tr_b16 %0, %8 offset:%9\n\t"
            "ds_read_b64_tr_b16 %1, %8 offset:%10\n\t"
            "ds_read_b64_tr_b16 %2, %8 offset:%11\n\t"
            "ds_read_b64_tr_b16 %3, %8 offset:%12\n\t"
            "ds_read_b64_tr_b16 %4, %8 offset:%13\n\t"
            "ds_read_b64_tr_b16 %5, %8 offset:%14\n\t"
            "ds_read_b64_tr_b16 %6, %8 offset:%15\n\t"
            "ds_read_b64_tr_b16 %7, %8 offset:%16\n\t"
            "s_waitcnt lgkmcnt(0)"
            : "=&v"(r[0]), "=&v"(r[1]), "=&v"(r[2]), "=&v"(r[3]), "=&v"(r[4]), "=&v"(r[5]), "=&v"(r[6]),
              "=&v"(r[7])
            : "v"(addr), "n"(lo0), "n"(hi0), "n"(lo1), "n"(hi1), "n"(lo2), "n"(hi2), "n"(lo3), "n"(hi3)
            : "memory");
    }
#pragma unroll
    for (int b = 0; b < NB; ++b)
        va[B0 + b] = __builtin_bit_cast(bf16x8_t, u32x4_t{r[2 * b].x, r[2 * b].y, r[2 * b + 1].x, r[2 * b + 1].y});
}

// LDS views of one staged tile; rows are addressed as (16-row block, row in
// block).  The register-staged path keeps row-major rows padded by kPfPad
// elements.  A ring stage of the direct-to-LDS path (D = 128) is 16 slots of
// kRingSlotElems elements (1 KiB + 32 bytes): slot 8 f + i holds, as four
// 256-byte rows j = 0..3, the K rows of keys 16 f + i and 16 f + i + 8 and
// then the V rows of the same two keys, the 16-byte chunk c of row j stored
// at c ^ (j & 1).  The padding and the swap make the 16 rows of a K operand
// read and each 32-lane half of a transposing V read fall in distinct banks,
// and every read of a lane sits at a constant offset from one address.
//
// A view gives a lane's operand addresses as one per-lane pointer plus
// compile-time offsets: k_lane(n, g4) + k_off(kb2, s) is the K operand of
// pair column n, lane group g4, key block kb2 and k step s (keys 16 kb2 + n,
// elements 32 s + 8 g4 .. + 7), which k_operand reads; v_lane(n, g4) +
// v_off(hi, b) the 4-element piece of the V^T operand (key 16 hi + 4 g4 +
// n / 4, elements 16 b + 4 (n % 4) .. + 3).
template <int D>
struct PaddedTile {
    const uint16_t* k;
    const uint16_t* v;
    static constexpr int kRow = D + kPfPad;
    __device__ const uint16_t* k_lane(int n, int g4) const { return k + n * kRow + 8 * g4; }
    static constexpr int k_off(int kb2, int s) { return 16 * kb2 * kRow + 32 * s; }
    __device__ bf16x8_t k_operand(int n, int g4, int kb2, int s) const {
        return lds_bf16x8(k_lane(n, g4) + k_off(kb2, s));
    }
    __device__ const uint16_t* v_lane(int n, int g4) const { return v + (4 * g4 + (n >> 2)) * kRow + 4 * (n & 3); }
    static constexpr int v_off(int hi, int b) { return 16 * hi * kRow + 16 * b; }
};

constexpr int kRingSlotElems = 528;
constexpr int kRingStageElems = 16 * kRingSlotElems;  // K and V of one tile

struct RingTile {
    const uint16_t* st;
    // key r < 16 of a half, row j = r / 8 (+ 2 for V) of slot r % 8
    __device__ const uint16_t* k_lane(int n, int g4) const {
        const int jr = n >> 3;
        return st + (n & 7) * kRingSlotElems + jr * 128 + 8 * (g4 ^ jr);
    }
    static constexpr int k_off(int kb2, int s) { return 8 * kRingSlotElems * kb2 + 32 * s; }
    __device__ bf16x8_t k_operand(int n, int g4, int kb2, int s) const {
        return lds_bf16x8(k_lane(n, g4) + k_off(kb2, s));
    }
    __device__ const uint16_t* v_lane(int n, int g4) const {
        const int key = 4 * g4 + (n >> 2);
        const int jr = key >> 3;
        return st + (key & 7) * kRingSlotElems + (2 + jr) * 128 + 8 * (((n >> 1) & 1) ^ jr) + 4 * (n & 1);
    }
    static constexpr int v_off(int hi, int b) { return 8 * kRingSlotElems * hi + 16 * b; }
};

// One tile of one wave: S^T for keys t0 + 16 kb2 + 4 g4 + i of the wave's
// pair blocks (pair n of each), the online softmax update, and O^T += V^T P^T.
// A wave holds PB blocks of 16 pairs: each K and V operand read from LDS
// feeds PB products, so LDS bytes per product fall as 1 / PB.
// qk = |scale * k_scale * log2 e| (a negative factor is carried by the sign
// of q, and qk >= 2^-100).  mask (uniform in the wave): the tile crosses the
// causal diagonal, the end of the key range, a row's window start (a key is
// visible while pos - key < win) or rows past the unit, so keys are tested
// one by one; otherwise every key of the tile is visible to every pair of
// the wave.  cap > 0 (uniform): the scores pass through the logit soft-cap
// first.  Per score the vector work is one fma into one v_exp_f32, a share
// of a max tree, a packed bf16 conversion and a dot2 into the row sum.  The
// first VH blocks of the V operand are read before the softmax so that the
// reads overlap it.
// The first product of a tile: the raw q.k of the wave's pairs (sv[pb][j]:
// key t0 + 16 (j / 4) + 4 g4 + j % 4 of pair n of block pb).
template <int D, int PB, class Tile>
__device__ __forceinline__ void pf_scores(const Tile& T, int n, int g4, const bf16x8_t (&qb)[PB][D / 32],
                                          float (&sv)[PB][8]) {
    constexpr int NS = D / 32;
#pragma unroll
    for (int kb2 = 0; kb2 < 2; ++kb2) {
        f32x4_t c[PB];
#pragma unroll
        for (int pb = 0; pb < PB; ++pb) c[pb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < NS; ++s) {
            const bf16x8_t kop = T.k_operand(n, g4, kb2, s);
#pragma unroll
            for (int pb = 0; pb < PB; ++pb)
                c[pb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kop, qb[pb][s], c[pb], 0, 0, 0);
        }
#pragma unroll
        for (int pb = 0; pb < PB; ++pb)
#pragma unroll
            for (int i = 0; i < 4; ++i) sv[pb][4 * kb2 + i] = c[pb][i];
    }
}

// The rest of a tile from its raw scores: soft-cap, mask, online softmax and
// O^T += V^T P^T.
template <int D, int PB, int VH, class Tile>
__device__ __forceinline__ void pf_update(const Tile& T, float (&sv)[PB][8], int t0, int kend,
                                          const int (&pos)[PB], int win, const bool (&row_ok)[PB], bool mask, int n,
                                          int g4, float qk, float cap, float cap_k, f32x4_t (&acc)[PB][D / 16],
                                          float (&m_run)[PB], float (&l_run)[PB]) {
    constexpr int ND = D / 16;
    const uint16_t* const vl = T.v_lane(n, g4);
    if (cap > 0.f) {  // capped scores are already in log2 units
#pragma unroll
        for (int pb = 0; pb < PB; ++pb)
#pragma unroll
            for (int j = 0; j < 8; ++j) sv[pb][j] = soft_cap_log2(sv[pb][j] * qk, cap, cap_k);
        qk = 1.f;
    }
    if (mask) {
#pragma unroll
        for (int pb = 0; pb < PB; ++pb)
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const int kp = t0 + 16 * (j >> 2) + 4 * g4 + (j & 3);
                sv[pb][j] = (row_ok[pb] && kp < kend && kp <= pos[pb] && pos[pb] - kp < win) ? sv[pb][j] : -INFINITY;
            }
    }
    // V^T operand: lane group g4 takes keys 4 g4 + j (j < 4) and 16 + 4 g4 +
    // j - 4 (j >= 4), where the first product left their scores; lane 4 j + q
    // of the group points at V[key_j][16 b + 4 q].
    static_assert(VH == ND / 2, "half of the V operand blocks before the softmax, half after");
    bf16x8_t va[ND];
    v_operands<Tile, 0, VH>(vl, va);
    bf16x8_t pbv[PB];
#pragma unroll
    for (int pb = 0; pb < PB; ++pb) {
        // Lazy rescale, as in the decode unit: scores at most 2^8 above the
        // running maximum are taken against it.  The running maximum is
        // shared by the four lanes of a pair, so while no lane's own tile
        // maximum passes it by more than 8 (log2) nothing is exchanged;
        // otherwise the pair's maximum is formed across its lanes and the
        // pair rescales.
        const float* s8 = sv[pb];
        // NaN-propagating maxima (v_maximum3_f32) take the products' raw
        // outputs as they are, where fmaxf would first quiet each of them; a
        // NaN score comes only from non-finite K or q, whose row is NaN
        // either way.  qk > 0, so -inf stays -inf when scaled.
        const float ml =
            vmax(vmax(vmax(s8[0], s8[1]), vmax(s8[2], s8[3])), vmax(vmax(s8[4], s8[5]), vmax(s8[6], s8[7])));
        const float mtl = ml * qk;  // this lane's tile maximum in log2 units
        if (__any(mtl > m_run[pb] + 8.0f)) {
            float mr = vmax(ml, __shfl_xor(ml, 16));
            mr = vmax(mr, __shfl_xor(mr, 32));
            const float mt = mr * qk;  // the pair's tile maximum
            const bool need = mt > m_run[pb] + 8.0f;
            const float m_new = need ? mt : m_run[pb];
            const float alpha = need ? exp2_fast(m_run[pb] - m_new) : 1.f;
            l_run[pb] *= alpha;
            m_run[pb] = m_new;
#pragma unroll
            for (int b = 0; b < ND; ++b) acc[pb][b] *= alpha;
        }
        const float nmb = (m_run[pb] == -INFINITY) ? 0.f : -m_run[pb];
        float p[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) p[j] = exp2_fast(fmaf(s8[j], qk, nmb));  // a masked key (-inf) gives 0
#pragma unroll
        for (int j = 0; j < 8; ++j) pbv[pb][j] = static_cast<__bf16>(p[j]);  // round to nearest even
        // the row sum adds the rounded weights that P V uses, two per dot2
        const bf16x2_t ones = {static_cast<__bf16>(1.0f), static_cast<__bf16>(1.0f)};
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const bf16x2_t pp = {pbv[pb][2 * j], pbv[pb][2 * j + 1]};
            l_run[pb] = __builtin_amdgcn_fdot2_f32_bf16(pp, ones, l_run[pb], false);
        }
    }
    // the first half's products go out before the second half is read, so
    // that its reads overlap them
#pragma unroll
    for (int b = 0; b < VH; ++b)
#pragma unroll
        for (int pb = 0; pb < PB; ++pb)
            acc[pb][b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va[b], pbv[pb], acc[pb][b], 0, 0, 0);
    v_operands<Tile, VH, ND - VH>(vl, va);
#pragma unroll
    for (int b = VH; b < ND; ++b)
#pragma unroll
        for (int pb = 0; pb < PB; ++pb)
            acc[pb][b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va[b], pbv[pb], acc[pb][b], 0, 0, 0);
}

template <int D, int PB, int VH, class Tile>
__device__ __forceinline__ void pf_compute(const Tile& T, int t0, int kend, const int (&pos)[PB], int win,
                                           const bool (&row_ok)[PB], bool mask, int n, int g4, float qk, float cap,
                                           float cap_k, const bf16x8_t (&qb)[PB][D / 32], f32x4_t (&acc)[PB][D / 16],
                                           float (&m_run)[PB], float (&l_run)[PB]) {
    float sv[PB][8];
    pf_scores<D, PB>(T, n, g4, qb, sv);
    pf_update<D, PB, VH>(T, sv, t0, kend, pos, win, row_ok, mask, n, g4, qk, cap, cap_k, acc, m_run, l_run);
}

// One wave's share of a prefill unit: its PB blocks of 16 (row, q head)
// pairs, their q slices, the running softmax state and the O^T accumulator,
// and the unit's key range.  The unit's kPrefillQRows pairs are spread over
// NWV waves, 16 PB per wave: pair x = 16 PB w + 16 pb + n.  open() reads the
// unit and the q slices; close() writes the output (uncut unit) or the
// normalised partial and its LSE (cut unit) once the workgroup has agreed on
// `bad`.
template <int D, int G, int NWV, int PB>
struct PfWave {
    static constexpr int NS = D / 32;  // k steps of the first product
    static constexpr int ND = D / 16;  // 16-row blocks of O^T
    static constexpr int PPW = kPfPairsPerBlock * PB;  // pairs per wave
    static_assert(NWV * PPW == kPrefillQRows, "the waves cover the unit's pairs");
    int n, g4, h, kb, kend;
    int r[PB], hq_idx[PB], pos[PB];
    bool row_ok[PB];
    int win;  // window: keys pos - win < j <= pos (INT32_MAX: no window)
    bool wave_has_rows, wave_full;
    int wave_first_pos, wave_last_pos;
    SeqTable tbl;
    bf16x8_t qb[PB][NS];
    float qk;
    f32x4_t acc[PB][ND];
    float m_run[PB], l_run[PB];
    bool bad;

    __device__ __forceinline__ void open(const AttnArgs& a, const Unit& un, int wave, int lane, int kv_head) {
        constexpr int QB = 2;  // bf16 queries
        n = lane & 15;         // pair column of this lane
        g4 = lane >> 4;
        h = kv_head;
        // rows of this wave: positions pos0 + wr0 .. pos0 + wr1
        const int wr0 = (wave * PPW) / G;
        const int wr1 = min(un.nrows - 1, (wave * PPW + PPW - 1) / G);
        wave_has_rows = wr0 < un.nrows;
        wave_last_pos = un.pos0 + wr1;
        wave_first_pos = un.pos0 + wr0;
        // every pair of the wave is a row of the unit
        wave_full = (wave * PPW + PPW - 1) / G < un.nrows;

        kb = un.kv_begin;
        kend = min(un.kv_end, un.pos0 + un.nrows);  // no row sees past its position
        // a stale plan (lengths or row offsets of the sequence other than the
        // plan's) makes every row of the unit NaN, as in the decode unit
        bad = unit_is_stale(a, un);
        win = a.window > 0 ? a.window : INT32_MAX;
        tbl = seq_table(a, un.seq);
        // a negative score factor is carried by the sign of q (exact)
        const uint32_t flip = a.qk_scale < 0.f ? 0x80008000u : 0u;
        const char* qrow0 = static_cast<const char*>(a.q) + static_cast<int64_t>(un.row0) * a.q_stride * QB;
#pragma unroll
        for (int pb = 0; pb < PB; ++pb) {
            const int x = wave * PPW + kPfPairsPerBlock * pb + n;
            r[pb] = x / G;  // row of the chunk block
            hq_idx[pb] = h * G + x % G;
            row_ok[pb] = r[pb] < un.nrows;
            pos[pb] = un.pos0 + r[pb];
            // q slice of this lane's pair: elements 32 s + 8 g4 .. + 7
            const char* qrow = static_cast<const char*>(a.q) +
                               (static_cast<int64_t>(un.row0 + r[pb]) * a.q_stride +
                                static_cast<int64_t>(hq_idx[pb]) * D) * QB;
#pragma unroll
            for (int s = 0; s < NS; ++s) {
                // pairs past the unit's rows read the unit's first row (no
                // branch around the load) and take zeros
                Words<4> w = load_words<4>((row_ok[pb] ? qrow : qrow0) + (32 * s + 8 * g4) * QB);
                const uint32_t fl = row_ok[pb] ? flip : 0u;
                const uint32_t keep = row_ok[pb] ? 0xFFFFFFFFu : 0u;
                qb[pb][s] = __builtin_bit_cast(bf16x8_t, make_uint4((w.w[0] ^ fl) & keep, (w.w[1] ^ fl) & keep,
                                                                    (w.w[2] ^ fl) & keep, (w.w[3] ^ fl) & keep));
            }
#pragma unroll
            for (int b = 0; b < ND; ++b) acc[pb][b] = f32x4_t{0.f, 0.f, 0.f, 0.f};
            m_run[pb] = -INFINITY;  // running max of this lane's pair (its four lanes agree)
            l_run[pb] = 0.f;        // this lane's share of the running sum
        }
        // |factor|, at least 2^-100 so that -inf * qk stays -inf (a zero
        // factor then still gives exp2 of exactly 0 for every visible key)
        qk = fmaxf(fabsf(a.qk_scale), 0x1p-100f);
    }

    // Tiles wholly past the wave's last row, or wholly before the first
    // row's window, hold no key any pair of the wave sees.
    __device__ __forceinline__ bool computes(int t0) const {
        return wave_has_rows && t0 <= wave_last_pos && wave_first_pos - (t0 + kPfKeys - 1) < win;
    }
    __device__ __forceinline__ bool masked(int t0) const {
        return !(wave_full && t0 + kPfKeys <= kend && t0 + kPfKeys - 1 <= wave_first_pos &&
                 wave_last_pos - t0 < win);
    }
    template <int VH, class Tile>
    __device__ __forceinline__ void tile(const AttnArgs& a, const Tile& T, int t0) {
        if (computes(t0))
            pf_compute<D, PB, VH>(T, t0, kend, pos, win, row_ok, masked(t0), n, g4, qk, a.soft_cap, a.soft_cap_k,
                                  qb, acc, m_run, l_run);
    }

    __device__ __forceinline__ void close(const AttnArgs& a, const Unit& un) {
#pragma unroll
        for (int pb = 0; pb < PB; ++pb) {
            float l_tot = l_run[pb] + __shfl_xor(l_run[pb], 16);
            l_tot += __shfl_xor(l_tot, 32);
            if (!row_ok[pb]) continue;
            const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
            if (un.prow < 0) {
                uint16_t* dst = static_cast<uint16_t*>(a.out) +
                                (static_cast<int64_t>(un.row0 + r[pb]) * a.hq + hq_idx[pb]) * D + 4 * g4;
                const float sc = inv * a.v_scale;
#pragma unroll
                for (int b = 0; b < ND; ++b) {
                    float o[4];
#pragma unroll
                    for (int i = 0; i < 4; ++i) o[i] = bad ? NAN : acc[pb][b][i] * sc;
                    store_out<PKV_DTYPE_BF16, 4>(reinterpret_cast<char*>(dst + 16 * b), o);
                }
            } else {
                const int64_t prow = static_cast<int64_t>(un.prow) + r[pb];
                float* dst = a.partial_o + (prow * a.hq + hq_idx[pb]) * D + 4 * g4;
#pragma unroll
                for (int b = 0; b < ND; ++b) {
                    const float4 o = bad ? make_float4(NAN, NAN, NAN, NAN)
                                         : make_float4(acc[pb][b][0] * inv, acc[pb][b][1] * inv,
                                                       acc[pb][b][2] * inv, acc[pb][b][3] * inv);
                    *reinterpret_cast<float4*>(dst + 16 * b) = o;
                }
                if (g4 == 0)
                    a.partial_lse[prow * a.hq + hq_idx[pb]] =
                        bad ? NAN : (l_tot > 0.f ? m_run[pb] + __log2f(l_tot) : -INFINITY);
            }
        }
    }
};

// One kv head h of unit `un` on the calling workgroup, K/V staged through
// registers into two padded LDS buffers (any page size, bf16 or fp8 K/V,
// D = 64 or 128).
template <int KVDT, int D, int G>
__device__ __forceinline__ void prefill_unit(const AttnArgs& a, const Unit& un, int h, int wave, int lane,
                                             const PfRole<D>& role, PrefillLds<D>& lds) {
    PfWave<D, G, kPfWaves, 1> W;
    W.open(a, un, wave, lane, h);
    const int kb = W.kb, kend = W.kend;
    const SeqTable tbl = W.tbl;

    // prologue: tile 0 staged; tiles 1 and 2 and the pages of tiles 3
    // and 4 in flight
    PfRegs<KVDT, D> ra, rb;
    __syncthreads();  // the LDS of the previous unit is free
    pf_load<KVDT, D>(ra, a, role, h, kb + role.kk, kend, pf_page(a, tbl, kb + role.kk), tbl.n, W.bad);
    pf_stage<KVDT, D>(ra, role, lds, 0);
    pf_load<KVDT, D>(ra, a, role, h, kb + kPfKeys + role.kk, kend, pf_page(a, tbl, kb + kPfKeys + role.kk),
                     tbl.n, W.bad);
    pf_load<KVDT, D>(rb, a, role, h, kb + 2 * kPfKeys + role.kk, kend,
                     pf_page(a, tbl, kb + 2 * kPfKeys + role.kk), tbl.n, W.bad);
    int32_t pa = pf_page(a, tbl, kb + 3 * kPfKeys + role.kk);
    int32_t pb = pf_page(a, tbl, kb + 4 * kPfKeys + role.kk);
    __syncthreads();

    // Two phases per trip so that the two register sets take turns: the
    // phase that computes tile t from buffer t % 2 stages tile t + 1
    // (loaded two phases ago) into the other buffer and reloads its
    // register set with tile t + 3.
    auto phase = [&](int t0, int buf, PfRegs<KVDT, D>& rs, int32_t& pg) {
        W.template tile<D / 32>(a, PaddedTile<D>{&lds.k[buf][0][0], &lds.v[buf][0][0]}, t0);
        // unconditional, also past the last tile: the other buffer is
        // free (every wave passed the previous barrier) and every address
        // stays in bounds, so the loads keep one fixed order and their
        // waits count in order
        pf_stage<KVDT, D>(rs, role, lds, buf ^ 1);
        const int t3 = t0 + 3 * kPfKeys + role.kk;
        pf_load<KVDT, D>(rs, a, role, h, t3, kend, pg, tbl.n, W.bad);
        pg = pf_page(a, tbl, t3 + 2 * kPfKeys);
        __syncthreads();
    };
    for (int t0 = kb; t0 < kend; t0 += 2 * kPfKeys) {
        phase(t0, 0, ra, pa);
        if (t0 + kPfKeys >= kend) break;
        phase(t0 + kPfKeys, 1, rb, pb);
    }
    W.bad = __syncthreads_or(W.bad) != 0;
    W.close(a, un);
}

// The units of plan queue `queue` on the calling workgroup through the
// register-staged tile.  A prefill unit holds one kv head; a unit of a
// few-row step (ALL_HEADS: on a decode queue) holds every kv head, taken
// here one after the other.
template <int KVDT, int D, int G, bool ALL_HEADS = false>
__device__ __forceinline__ void prefill_queue(const AttnArgs& a, int queue, PrefillLds<D>& lds) {
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const PfRole<D> role;

    const const_ptr<Unit> units = as_const(a.units);
    const const_ptr<int32_t> qoff = as_const(a.queue_off);
    const int u_begin = qoff[queue];
    const int u_end = qoff[queue + 1];
    for (int ui = u_begin; ui < u_end; ++ui) {
        const Unit un = load_unit(units, ui);
        if constexpr (ALL_HEADS) {
            for (int h = 0; h < a.hkv; ++h) prefill_unit<KVDT, D, G>(a, un, h, wave, lane, role, lds);
        } else {
            prefill_unit<KVDT, D, G>(a, un, un.kind - kUnitPrefill, wave, lane, role, lds);
        }
    }
}

// ---------------------------------------------------------------------------
// Direct-to-LDS path (bf16 K/V, D = 128, block_size a power of two >= 16).
//
// A ring of kRingStages LDS stages, each one 32-key tile of K and V in the
// slot layout above.  Per tile, wave w fills slots w and 8 + w with
// global_load_lds_dwordx4, which writes LDS without passing through
// registers: lane l loads the 16 bytes that the layout puts at position l of
// the slot (16 lanes read one 256-byte row of K or V).  Tile t + 3 is loaded
// while tile t is computed.  Each step waits (vmcnt) until the wave's own
// loads of the current tile have landed and then meets the others at a
// barrier, after which every slot is visible.  The page-table entries come
// through scalar loads two tiles ahead of their use, so vmcnt counts only the
// tile loads.  Each 16-key half of a tile lies in one page (tiles start at
// multiples of 16 keys and pages hold a power of two >= 16 of them), so a
// slot needs one entry and a tile two.
// ---------------------------------------------------------------------------
constexpr int kRingStages = 4;

typedef __attribute__((address_space(3))) void lds_void_t;

// Cache policy field of a direct-to-LDS load: the default one (the ring's
// tiles, whose keys the other row blocks of a chunk read again), or
// non-temporal (the nt bit on gfx950), as the decode unit's K/V loads are
// (the few-row kernel's tiles, read once).
constexpr int kLdsLoadDefault = 0;
constexpr int kLdsLoadNt = 2;

// s_waitcnt vmcnt(N) (expcnt and lgkmcnt left alone; gfx9 encoding)
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}
// s_waitcnt lgkmcnt(0)
__device__ __forceinline__ void wait_lgkmcnt0() { __builtin_amdgcn_s_waitcnt(0xC07F); }

// Workgroup barrier without a memory fence (the waits before it are
// explicit); the empty asm statements keep the compiler from moving memory
// accesses across it.
__device__ __forceinline__ void ring_barrier() {
    __asm__ volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    __asm__ volatile("" ::: "memory");
}

template <int G, int NWV>
__device__ __forceinline__ void prefill_queue_ring(const AttnArgs& a, int queue, uint16_t* s0, uint16_t* s1,
                                                   uint16_t* s2, uint16_t* s3) {
    constexpr int D = 128;
    constexpr int SE = 8 / NWV;  // slots per 16-key half that a wave fills: wave + NWV e, e < SE
    static_assert(SE * NWV == 8, "the waves share the 8 slots of a half");
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const uint32_t nblocks = static_cast<uint32_t>(a.num_blocks < 0x7FFFFFFF ? a.num_blocks : 0x7FFFFFFF);
    const int shift = a.block_shift;
    // this lane's load into slot wave + NWV e: slot row j = lane / 16, a K
    // row (j < 2) or a V row of key wave + NWV e + 8 (j % 2) of a half (rows
    // of the pool are hkv * 256 bytes apart), logical chunk
    // (lane % 16) ^ (j % 2)
    const int j = lane >> 4;
    const char* const lane_src = static_cast<const char*>(j < 2 ? a.k_cache : a.v_cache) +
                                 static_cast<uint32_t>(wave + 8 * (j & 1)) * static_cast<uint32_t>(a.hkv) * (D * 2) +
                                 static_cast<uint32_t>(((lane & 15) ^ (j & 1)) * 16);
    const uint32_t slot_src_step = static_cast<uint32_t>(NWV) * static_cast<uint32_t>(a.hkv) * (D * 2);
    const const_ptr<Unit> units = as_const(a.units);
    const const_ptr<int32_t> qoff = as_const(a.queue_off);
    const int u_begin = qoff[queue];
    const int u_end = qoff[queue + 1];
    for (int ui = u_begin; ui < u_end; ++ui) {
        const Unit un = load_unit(units, ui);
        PfWave<D, G, NWV, 8 / NWV> W;
        W.open(a, un, wave, lane, un.kind - kUnitPrefill);
        const int kb = W.kb, kend = W.kend, h = W.h;
        const SeqTable tbl = W.tbl;
        const int ntiles = kend > kb ? (kend - kb + kPfKeys - 1) / kPfKeys : 0;
        const int glast = kend > kb ? ((kend - 1) & ~15) : kb;  // start of the unit's last 16 keys
        // bytes of a pool row (one key, every kv head) and of a page; this
        // unit's kv head within a row
        const uint32_t row_bytes = static_cast<uint32_t>(a.hkv) * (D * 2);
        const uint64_t page_bytes = static_cast<uint64_t>(row_bytes) << shift;
        const char* const head_src = lane_src + static_cast<uint32_t>(h) * (D * 2);

        // a half of 16 keys starting at t0 + 16 f, clamped to the last half
        // (so that a half past kend reads keys that exist), and its
        // page-table entry (index clamped into the row; validity is decided
        // at the load)
        auto half = [&](int t0, int f) { return min(t0 + 16 * f, glast); };
        auto entry = [&](int t0, int f) { return tbl.clamped(half(t0, f) >> shift); };
        struct Entries {
            int32_t e0, e1;
        };
        auto entries = [&](int t0) { return Entries{entry(t0, 0), entry(t0, 1)}; };
        auto issue = [&](uint16_t* st, int t0, Entries e) {
#pragma unroll
            for (int f = 0; f < 2; ++f) {
                const int g = half(t0, f);
                const int32_t ef = f ? e.e1 : e.e0;
                const int pidx = g >> shift;
                const bool ok = pidx < tbl.n && static_cast<uint32_t>(ef) < nblocks;
                W.bad |= t0 + 16 * f < kend && !ok;
                const uint64_t in_page = static_cast<uint64_t>(static_cast<uint32_t>(g - (pidx << shift))) * row_bytes;
                const char* const src = head_src + static_cast<uint64_t>(static_cast<uint32_t>(ok ? ef : 0)) * page_bytes +
                                        in_page;
#pragma unroll
                for (int e = 0; e < SE; ++e)
                    __builtin_amdgcn_global_load_lds(src + e * slot_src_step,
                                                     (lds_void_t*)(st + (8 * f + wave + NWV * e) * kRingSlotElems),
                                                     16, 0, kLdsLoadDefault);
            }
        };

        Entries e[kRingStages];  // page entries of the tiles in flight, slot = tile % 4
        ring_barrier();          // every wave is done with the previous unit's stages
        e[0] = entries(kb);
        e[1] = entries(kb + kPfKeys);
        e[2] = entries(kb + 2 * kPfKeys);
        if (0 < ntiles) issue(s0, kb, e[0]);
        if (1 < ntiles) issue(s1, kb + kPfKeys, e[1]);
        if (2 < ntiles) issue(s2, kb + 2 * kPfKeys, e[2]);
        e[3] = entries(kb + 3 * kPfKeys);
        e[0] = entries(kb + 4 * kPfKeys);

        // this wave's loads of tile tt are in once at most those of the
        // `later` tiles issued after it are still in flight; keys at or
        // past kend were read from inside their page (or from the last
        // group): their V rows are zeroed so that a zero weight never meets
        // a non-finite value
        auto land = [&](int tt, uint16_t* st, int later) {
            const int t0 = kb + tt * kPfKeys;
            if (later >= 2)
                wait_vmcnt<4 * SE>();
            else if (later == 1)
                wait_vmcnt<2 * SE>();
            else
                wait_vmcnt<0>();
            if (t0 + kPfKeys > kend) {
                if (j >= 2) {
#pragma unroll
                    for (int f = 0; f < 2; ++f)
#pragma unroll
                        for (int e = 0; e < SE; ++e)
                            if (t0 + 16 * f + wave + NWV * e + 8 * (j & 1) >= kend)
                                *reinterpret_cast<uint4*>(st + (8 * f + wave + NWV * e) * kRingSlotElems + lane * 8) =
                                    make_uint4(0, 0, 0, 0);
                }
                wait_lgkmcnt0();
            }
        };
        // tile tt from stage cur; tile tt + 3 into stage nxt with entry
        // use_e; the entry of tile tt + 5 into load_e
        auto phase = [&](int tt, uint16_t* cur, uint16_t* nxt, Entries use_e, Entries& load_e) {
            const int t0 = kb + tt * kPfKeys;
            // the (up to two) later tiles already issued may stay in flight
            land(tt, cur, min(2, ntiles - 1 - tt));
            ring_barrier();
            if (tt + 3 < ntiles) issue(nxt, t0 + 3 * kPfKeys, use_e);
            load_e = entries(t0 + 5 * kPfKeys);
            W.template tile<D / 32>(a, RingTile{cur}, t0);
        };
        for (int tt = 0; tt < ntiles; tt += kRingStages) {
            phase(tt, s0, s3, e[3], e[1]);
            if (tt + 1 >= ntiles) break;
            phase(tt + 1, s1, s0, e[0], e[2]);
            if (tt + 2 >= ntiles) break;
            phase(tt + 2, s2, s1, e[1], e[3]);
            if (tt + 3 >= ntiles) break;
            phase(tt + 3, s3, s2, e[2], e[0]);
        }
        W.bad = __syncthreads_or(W.bad) != 0;
        W.close(a, un);
    }
}

// LDS of the direct-to-LDS path: four stage arrays of their own (so that the
// compiler sees which stage a read touches); the decode workgroups of a mixed
// launch use the first one.
template <int D, int G>
constexpr int ring_stage0_elems() {
    return sizeof(DecodeLds<D, G, kPfWaves>) / 2 > kRingStageElems ? (sizeof(DecodeLds<D, G, kPfWaves>) + 1) / 2
                                                                   : kRingStageElems;
}

template <int KVDT, int D, int G, bool RING>
__global__ __launch_bounds__(kPfWaves * 64) __attribute__((amdgpu_waves_per_eu(4)))
void prefill_kernel(AttnArgs a, int queue0) {
    if constexpr (RING) {
        __shared__ __attribute__((aligned(16))) uint16_t s0[kRingStageElems], s1[kRingStageElems],
            s2[kRingStageElems], s3[kRingStageElems];
        prefill_queue_ring<G, kPfWaves>(a, queue0 + blockIdx.x, s0, s1, s2, s3);
    } else {
        __shared__ PrefillLds<D> lds;
        prefill_queue<KVDT, D, G>(a, queue0 + blockIdx.x, lds);
    }
}

// Chunk units of many rows alone (no decode workgroup shares the launch): 4
// waves of 32 pairs each.  Every K and V operand read from LDS feeds two
// products, half the LDS bytes per product of the 8-wave form, and the
// 256-register budget holds the two pair blocks' accumulators and q slices;
// two workgroups (two waves per SIMD, 2 x 66 KiB of ring) share a CU.  Units
// of a few rows (fewer than 64 pairs) would leave a wave's second block
// empty and keep the 8-wave form.
template <int G>
__global__ __launch_bounds__(kPfWideWaves * 64) __attribute__((amdgpu_waves_per_eu(2)))
void prefill_wide_kernel(AttnArgs a, int queue0) {
    __shared__ __attribute__((aligned(16))) uint16_t s0[kRingStageElems], s1[kRingStageElems], s2[kRingStageElems],
        s3[kRingStageElems];
    prefill_queue_ring<G, kPfWideWaves>(a, queue0 + blockIdx.x, s0, s1, s2, s3);
}

// ---------------------------------------------------------------------------
// Few-row steps (a speculative verify step: a handful of new rows per
// sequence).  Such a step is planned as decode rows are: each sequence's key
// range is cut into pieces over the decode queues, and a unit holds all the
// sequence's rows (at most 16 (row, q head) pairs per kv head, one MFMA pair
// block) and every kv head.  One 8-wave workgroup per queue; wave w takes kv
// heads w, w + 8, ... of each unit, so that the workgroup streams whole key
// rows of the pool as the decode kernel does.  A wave walks the unit's
// 32-key tiles on its own, with no barrier, through an LDS tile of its own in
// the ring layout (each load instruction two whole 256-byte rows of K and
// two of V), reading the operands back as the ring path does.  bf16 rows go
// straight to the LDS tile (direct-to-LDS, non-temporal), and the next
// tile's loads go out once the tile's products have read it, so that no
// load is in flight while the wave reads LDS.  fp8 codes go to registers
// and are widened to bf16 as they are written to the tile; there the next
// tile's loads go out before the products, which overlap them.  One tile is
// in flight per wave (two measured slower: the read rate of the pool falls
// with more bytes in flight per CU, as for the decode kernel).  D = 128,
// pages of a power of two >= 16 tokens (each 16-key half of a tile lies in
// one page).
// ---------------------------------------------------------------------------
constexpr int kFrWaves = 8;

// Registers of one tile in flight: the lane's piece of each of the 16 slots
// of the ring layout (row lane / 16 of slot 8 f + i: the K row (rows 0 and
// 1) or V row (rows 2 and 3) of key 16 f + i + 8 (row % 2), stored chunk
// lane % 16): 16 bytes of bf16, or the 8 fp8 codes that widen to them.
template <int KVDT>
struct FrRegs {
    using piece_t = std::conditional_t<KVDT == PKV_DTYPE_FP8_E4M3, u32x2_t, u32x4_t>;
    piece_t x[16];
};

// A slot piece as 8 bf16 values (fp8 E4M3 codes widen exactly: low and high
// code pairs of each word).
__device__ __forceinline__ u32x4_t fr_bf16(const u32x4_t& x) { return x; }
__device__ __forceinline__ u32x4_t fr_bf16(const u32x2_t& x) {
    auto lo = [](uint32_t d) {
        return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(static_cast<int>(d), 1.0f, false));
    };
    auto hi = [](uint32_t d) {
        return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(static_cast<int>(d), 1.0f, true));
    };
    return u32x4_t{lo(x.x), hi(x.x), lo(x.y), hi(x.y)};
}

// Unit `un`, kv head h, on the calling wave alone; st is the wave's tile.
template <int KVDT, int G>
__device__ __forceinline__ void fewrow_head(const AttnArgs& a, const Unit& un, int h, uint16_t* st, int lane) {
    constexpr int D = 128;
    constexpr int RB = D * dt_bytes(KVDT);  // bytes of one key's row of one kv head
    constexpr int PIECE = RB / 16;          // bytes of a lane's piece of a row
    using Regs = FrRegs<KVDT>;
    const int j = lane >> 4;   // slot row of this lane
    const uint32_t nblocks = static_cast<uint32_t>(a.num_blocks < 0x7FFFFFFF ? a.num_blocks : 0x7FFFFFFF);
    const int shift = a.block_shift;
    const uint32_t row_bytes = static_cast<uint32_t>(a.hkv) * RB;  // pool row of one key
    const uint64_t page_bytes = static_cast<uint64_t>(row_bytes) << a.block_shift;
    // this lane's source in slot i of a half: key i + 8 (j % 2) of the half,
    // K (j < 2) or V, logical chunk (lane % 16) ^ (j % 2)
    const char* const src = static_cast<const char*>(j < 2 ? a.k_cache : a.v_cache) + (8 * (j & 1)) * row_bytes +
                            static_cast<uint32_t>(((lane & 15) ^ (j & 1)) * PIECE);
    const char* const head_src = src + static_cast<uint32_t>(h) * RB;  // this kv head within a pool row

    // the unit's pairs as "wave 0" of a layout of one pair block per wave
    PfWave<D, G, kPfWaves, 1> W;
    W.open(a, un, 0, lane, h);
    const int kb = W.kb, kend = W.kend;
    const SeqTable tbl = W.tbl;
    const int ntiles = kend > kb ? (kend - kb + kPfKeys - 1) / kPfKeys : 0;
    const int glast = kend > kb ? ((kend - 1) & ~15) : kb;  // start of the unit's last 16 keys

    if constexpr (KVDT == PKV_DTYPE_BF16) {
        // bf16: tile i straight into the wave's LDS tile, per half f of 16
        // keys (clamped to the unit's last half, so that every address lies
        // in a page of the sequence or in the pool's first page) its
        // page-table entry and one direct-to-LDS load per slot.  Only the
        // wave reads its tile, so a vmcnt wait publishes it; the next tile's
        // loads go out once the tile's products have read it.
        auto issue = [&](int i) {
            const int t0 = kb + kPfKeys * i;
#pragma unroll
            for (int f = 0; f < 2; ++f) {
                const int g = min(t0 + 16 * f, glast);
                const int pidx = g >> shift;
                const int32_t e = tbl.clamped(pidx);
                const bool ok = pidx < tbl.n && static_cast<uint32_t>(e) < nblocks;
                W.bad |= t0 + 16 * f < kend && !ok;
                const int64_t row0 = static_cast<int64_t>(ok ? e : 0) * a.block_size + (g - (pidx << shift));
                const char* const base = src + (row0 * a.hkv + h) * RB;
#pragma unroll
                for (int i8 = 0; i8 < 8; ++i8)
                    __builtin_amdgcn_global_load_lds(base + i8 * row_bytes,
                                                     (lds_void_t*)(st + (8 * f + i8) * kRingSlotElems), 16, 0,
                                                     kLdsLoadNt);
            }
        };
        if (ntiles > 0) issue(0);
        for (int c = 0; c < ntiles; ++c) {
            const int t0 = kb + kPfKeys * c;
            wait_vmcnt<0>();
            // V rows of keys at or past kend were read from inside their
            // page (or from the last half): zeros, so that a zero weight
            // never meets a non-finite value
            if (t0 + kPfKeys > kend) {
                if (j >= 2) {
#pragma unroll
                    for (int s16 = 0; s16 < 16; ++s16)
                        if (t0 + 16 * (s16 >> 3) + (s16 & 7) + 8 * (j & 1) >= kend)
                            *reinterpret_cast<u32x4_t*>(st + s16 * kRingSlotElems + lane * 8) =
                                u32x4_t{0u, 0u, 0u, 0u};
                }
                wait_lgkmcnt0();
            }
            W.template tile<D / 32>(a, RingTile{st}, t0);
            __asm__ volatile("" ::: "memory");  // the tile's reads stay before the loads that overwrite it
            if (c + 1 < ntiles) issue(c + 1);
        }
    } else {
        // fp8 codes: tile i into registers r, widened to bf16 as they are
        // written to the LDS tile.  Per half f of 16 keys (clamped as above)
        // its page-table entry and one load per slot.  Past the unit's last
        // tile (the loop issues one tile ahead whether or not there is one,
        // so that the compiler counts the loads in flight exactly at every
        // wait) they read the first rows of the pool (a few KiB, cached) and
        // are never used.
        auto issue = [&](int i, Regs& r) {
            const int t0 = kb + kPfKeys * i;
            const bool live = i < ntiles;
#pragma unroll
            for (int f = 0; f < 2; ++f) {
                const int g = min(t0 + 16 * f, glast);
                const int pidx = g >> shift;
                const int32_t e = tbl.clamped(pidx);
                const bool ok = pidx < tbl.n && static_cast<uint32_t>(e) < nblocks;
                W.bad |= t0 + 16 * f < kend && !ok;
                // the page id times the page's bytes plus the row's offset
                const char* const base =
                    live ? head_src + static_cast<uint64_t>(static_cast<uint32_t>(ok ? e : 0)) * page_bytes +
                               static_cast<uint64_t>(static_cast<uint32_t>(g - (pidx << shift))) * row_bytes
                         : head_src;
#pragma unroll
                for (int i8 = 0; i8 < 8; ++i8)
                    r.x[8 * f + i8] = __builtin_nontemporal_load(
                        reinterpret_cast<const typename Regs::piece_t*>(base + i8 * row_bytes));
            }
        };
        // tile c into the wave's LDS tile, V rows of keys at or past kend
        // as zeros (the previous tile's reads of the LDS tile have
        // completed: they are waited for where they are issued)
        auto stage = [&](int c, const Regs& r) {
            const int t0 = kb + kPfKeys * c;
            if (t0 + kPfKeys <= kend) {  // every key of the tile is in the unit (uniform)
#pragma unroll
                for (int s16 = 0; s16 < 16; ++s16)
                    *reinterpret_cast<u32x4_t*>(st + s16 * kRingSlotElems + lane * 8) = fr_bf16(r.x[s16]);
                return;
            }
#pragma unroll
            for (int s16 = 0; s16 < 16; ++s16) {
                const bool zero = j >= 2 && t0 + 16 * (s16 >> 3) + (s16 & 7) + 8 * (j & 1) >= kend;
                *reinterpret_cast<u32x4_t*>(st + s16 * kRingSlotElems + lane * 8) =
                    zero ? u32x4_t{0u, 0u, 0u, 0u} : fr_bf16(r.x[s16]);
            }
        };
        // one register set: a tile's registers are free once it is in LDS;
        // the next tile's loads go out before the tile's products, whose
        // widening then overlaps them
        Regs r;
        issue(0, r);
        for (int c = 0; c < ntiles; ++c) {
            stage(c, r);
            issue(c + 1, r);
            W.template tile<D / 32>(a, RingTile{st}, kb + kPfKeys * c);
        }
    }
    W.close(a, un);
}

// Few-row steps on the caches, head dims and pages the few-row kernel does
// not serve: the register-staged prefill tile over the decode queues.
template <int KVDT, int D, int G>
__global__ __launch_bounds__(kPfWaves * 64) __attribute__((amdgpu_waves_per_eu(2)))
void fewrow_reg_kernel(AttnArgs a) {
    __shared__ PrefillLds<D> lds;
    prefill_queue<KVDT, D, G, true>(a, blockIdx.x, lds);
}

template <int KVDT, int G>
__global__ __launch_bounds__(kFrWaves * 64) __attribute__((amdgpu_waves_per_eu(2)))
void fewrow_kernel(AttnArgs a) {
    __shared__ __attribute__((aligned(16))) uint16_t lds[kFrWaves * kRingStageElems];
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    uint16_t* const st = lds + wave * kRingStageElems;
    const const_ptr<Unit> units = as_const(a.units);
    const const_ptr<int32_t> qoff = as_const(a.queue_off);
    const int u_end = qoff[blockIdx.x + 1];
    for (int ui = qoff[blockIdx.x]; ui < u_end; ++ui) {
        const Unit un = load_unit(units, ui);
        for (int h = wave; h < a.hkv; h += kFrWaves) fewrow_head<KVDT, G>(a, un, h, st, lane);
    }
}

// Both halves of a mixed step in one launch: blocks below num_decode_queues
// walk the decode queues with the decode unit, the others the prefill queues,
// so that the bandwidth-bound decode rows and the matrix-core chunk tiles run
// side by side on every CU (two 8-wave workgroups fit at <= 128 VGPRs).
template <int KVDT, int D, int G>
constexpr size_t mixed_lds_bytes() {
    return sizeof(DecodeLds<D, G, kPfWaves>) > sizeof(PrefillLds<D>) ? sizeof(DecodeLds<D, G, kPfWaves>)
                                                                      : sizeof(PrefillLds<D>);
}

template <int D, int G>
__device__ __forceinline__ void mixed_decode_queue(const AttnArgs& a, int b, DecodeLds<D, G, kPfWaves>& lds) {
    const const_ptr<Unit> units = as_const(a.units);
    const const_ptr<int32_t> qoff = as_const(a.queue_off);
    const int u_end = qoff[b + 1];
    for (int ui = qoff[b]; ui < u_end; ++ui)
        decode_unit<PKV_DTYPE_BF16, PKV_DTYPE_BF16, D, G, kPfWaves, kPageTile>(a, load_unit(units, ui), lds);
}

template <int KVDT, int D, int G, bool RING>
__global__ __launch_bounds__(kPfWaves * 64) __attribute__((amdgpu_waves_per_eu(4)))
void mixed_kernel(AttnArgs a, int num_decode_queues, int tail_queue0) {
    static_assert(KVDT == PKV_DTYPE_BF16, "one launch for bf16 K/V");
    const int b = blockIdx.x;
    // a decode workgroup's tail: prefill queue tail_queue0 + b, once every
    // wave is done with the decode units' LDS
    if constexpr (RING) {
        __shared__ __attribute__((aligned(16))) uint16_t s0[ring_stage0_elems<D, G>()], s1[kRingStageElems],
            s2[kRingStageElems], s3[kRingStageElems];
        if (b < num_decode_queues) {
            mixed_decode_queue<D, G>(a, b, *reinterpret_cast<DecodeLds<D, G, kPfWaves>*>(s0));
            if (tail_queue0 < 0) return;
            __syncthreads();
            prefill_queue_ring<G, kPfWaves>(a, tail_queue0 + b, s0, s1, s2, s3);
        } else {
            prefill_queue_ring<G, kPfWaves>(a, b, s0, s1, s2, s3);
        }
    } else {
        __shared__ __attribute__((aligned(16))) char smem[mixed_lds_bytes<KVDT, D, G>()];
        if (b < num_decode_queues) {
            mixed_decode_queue<D, G>(a, b, *reinterpret_cast<DecodeLds<D, G, kPfWaves>*>(smem));
            if (tail_queue0 < 0) return;
            __syncthreads();
            prefill_queue<KVDT, D, G>(a, tail_queue0 + b, *reinterpret_cast<PrefillLds<D>*>(smem));
        } else {
            prefill_queue<KVDT, D, G>(a, b, *reinterpret_cast<PrefillLds<D>*>(smem));
        }
    }
}

// The direct-to-LDS path serves bf16 K/V at D = 128 on power-of-two pages of
// at least 16 tokens.
template <int KVDT, int D>
constexpr bool ring_capable() {
    return KVDT == PKV_DTYPE_BF16 && D == 128;
}
__host__ inline bool ring_pages(const AttnArgs& a) { return a.block_shift >= 4; }

template <int KVDT, int D, int G>
int launch_prefill_t(const AttnArgs& a, int max_pairs, int num_queues, int queue0, hipStream_t st) {
    // the longest chunk's units hold at least 64 (row, q head) pairs: wide
    // tiles
    const bool wide = max_pairs >= kPrefillQRows / 2;
    if constexpr (ring_capable<KVDT, D>()) {
        if (ring_pages(a) && wide)
            hipLaunchKernelGGL((prefill_wide_kernel<G>), dim3(num_queues), dim3(kPfWideWaves * 64), 0, st, a,
                               queue0);
        else if (ring_pages(a))
            hipLaunchKernelGGL((prefill_kernel<KVDT, D, G, true>), dim3(num_queues), dim3(kPfWaves * 64), 0, st, a,
                               queue0);
        else
            hipLaunchKernelGGL((prefill_kernel<KVDT, D, G, false>), dim3(num_queues), dim3(kPfWaves * 64), 0, st,
                               a, queue0);
    } else {
        hipLaunchKernelGGL((prefill_kernel<KVDT, D, G, false>), dim3(num_queues), dim3(kPfWaves * 64), 0, st, a,
                           queue0);
    }
    return hipGetLastError() == hipSuccess ? PKV_OK : PKV_ERR_HIP;
}

template <int KVDT, int D>
int launch_prefill_g(const AttnArgs& a, int group, int max_pairs, int num_queues, int queue0, hipStream_t st) {
    switch (group) {
        case 1: return launch_prefill_t<KVDT, D, 1>(a, max_pairs, num_queues, queue0, st);
        case 2: return launch_prefill_t<KVDT, D, 2>(a, max_pairs, num_queues, queue0, st);
        case 4: return launch_prefill_t<KVDT, D, 4>(a, max_pairs, num_queues, queue0, st);
        case 8: return launch_prefill_t<KVDT, D, 8>(a, max_pairs, num_queues, queue0, st);
        default: return PKV_ERR_UNSUPPORTED;
    }
}

template <int KVDT>
int launch_prefill_d(const AttnArgs& a, int d, int group, int max_pairs, int num_queues, int queue0,
                     hipStream_t st) {
    if (d == 64) return launch_prefill_g<KVDT, 64>(a, group, max_pairs, num_queues, queue0, st);
    if (d == 128) return launch_prefill_g<KVDT, 128>(a, group, max_pairs, num_queues, queue0, st);
    return PKV_ERR_UNSUPPORTED;
}

template <int KVDT>
int launch_mixed_d(const AttnArgs& a, int d, int group, int num_decode_queues, int num_prefill_queues,
                   int tail_queue0, hipStream_t st) {
    const dim3 grid(num_decode_queues + num_prefill_queues), block(kPfWaves * 64);
    const bool ring = ring_pages(a);
    if (d == 128 && group == 4 && ring)
        hipLaunchKernelGGL((mixed_kernel<KVDT, 128, 4, true>), grid, block, 0, st, a, num_decode_queues,
                           tail_queue0);
    else if (d == 128 && group == 4)
        hipLaunchKernelGGL((mixed_kernel<KVDT, 128, 4, false>), grid, block, 0, st, a, num_decode_queues,
                           tail_queue0);
    else if (d == 128 && group == 2 && ring)
        hipLaunchKernelGGL((mixed_kernel<KVDT, 128, 2, true>), grid, block, 0, st, a, num_decode_queues,
                           tail_queue0);
    else if (d == 128 && group == 2)
        hipLaunchKernelGGL((mixed_kernel<KVDT, 128, 2, false>), grid, block, 0, st, a, num_decode_queues,
                           tail_queue0);
    else if (d == 64 && group == 4)
        hipLaunchKernelGGL((mixed_kernel<KVDT, 64, 4, false>), grid, block, 0, st, a, num_decode_queues,
                           tail_queue0);
    else if (d == 64 && group == 2)
        hipLaunchKernelGGL((mixed_kernel<KVDT, 64, 2, false>), grid, block, 0, st, a, num_decode_queues,
                           tail_queue0);
    else
        return PKV_ERR_UNSUPPORTED;
    return hipGetLastError() == hipSuccess ? PKV_OK : PKV_ERR_HIP;
}

}  // namespace

bool fewrow_capable(int q_dtype, int kv_dtype, int head_dim, int block_size) {
    return q_dtype == PKV_DTYPE_BF16 && (kv_dtype == PKV_DTYPE_BF16 || kv_dtype == PKV_DTYPE_FP8_E4M3) &&
           head_dim == 128 && block_size >= kTileTokens && (block_size & (block_size - 1)) == 0;
}

int launch_fewrow(const AttnArgs& a, int q_dtype, int kv_dtype, int head_dim, int group, int num_queues,
                  void* stream) {
    hipStream_t st = static_cast<hipStream_t>(stream);
    if (!prefill_supported(q_dtype, kv_dtype, head_dim, group)) return PKV_ERR_UNSUPPORTED;
    const dim3 grid(num_queues);
    if (fewrow_capable(q_dtype, kv_dtype, head_dim, a.block_size)) {
        auto fr = [&](auto kvdt) -> int {
            constexpr int KVDT = decltype(kvdt)::value;
            switch (group) {
                case 1: hipLaunchKernelGGL((fewrow_kernel<KVDT, 1>), grid, dim3(kFrWaves * 64), 0, st, a); break;
                case 2: hipLaunchKernelGGL((fewrow_kernel<KVDT, 2>), grid, dim3(kFrWaves * 64), 0, st, a); break;
                case 4: hipLaunchKernelGGL((fewrow_kernel<KVDT, 4>), grid, dim3(kFrWaves * 64), 0, st, a); break;
                case 8: hipLaunchKernelGGL((fewrow_kernel<KVDT, 8>), grid, dim3(kFrWaves * 64), 0, st, a); break;
                default: return PKV_ERR_UNSUPPORTED;
            }
            return hipGetLastError() == hipSuccess ? PKV_OK : PKV_ERR_HIP;
        };
        if (kv_dtype == PKV_DTYPE_BF16) return fr(std::integral_constant<int, PKV_DTYPE_BF16>{});
        return fr(std::integral_constant<int, PKV_DTYPE_FP8_E4M3>{});
    }
    // other caches, head dims and pages: the register-staged prefill tile
    // over the decode queues, one kv head of a unit after the other
    auto reg = [&](auto kvdt, auto d) -> int {
        constexpr int KVDT = decltype(kvdt)::value, D = decltype(d)::value;
        switch (group) {
            case 1: hipLaunchKernelGGL((fewrow_reg_kernel<KVDT, D, 1>), grid, dim3(kPfWaves * 64), 0, st, a); break;
            case 2: hipLaunchKernelGGL((fewrow_reg_kernel<KVDT, D, 2>), grid, dim3(kPfWaves * 64), 0, st, a); break;
            case 4: hipLaunchKernelGGL((fewrow_reg_kernel<KVDT, D, 4>), grid, dim3(kPfWaves * 64), 0, st, a); break;
            case 8: hipLaunchKernelGGL((fewrow_reg_kernel<KVDT, D, 8>), grid, dim3(kPfWaves * 64), 0, st, a); break;
            default: return PKV_ERR_UNSUPPORTED;
        }
        return hipGetLastError() == hipSuccess ? PKV_OK : PKV_ERR_HIP;
    };
    using BF = std::integral_constant<int, PKV_DTYPE_BF16>;
    using F8 = std::integral_constant<int, PKV_DTYPE_FP8_E4M3>;
    using D64 = std::integral_constant<int, 64>;
    using D128 = std::integral_constant<int, 128>;
    if (kv_dtype == PKV_DTYPE_BF16) return head_dim == 64 ? reg(BF{}, D64{}) : reg(BF{}, D128{});
    return head_dim == 64 ? reg(F8{}, D64{}) : reg(F8{}, D128{});
}

bool mixed_one_launch(int q_dtype, int kv_dtype, int head_dim, int group, int block_size) {
    return q_dtype == PKV_DTYPE_BF16 && kv_dtype == PKV_DTYPE_BF16 && (head_dim == 64 || head_dim == 128) &&
           (group == 2 || group == 4) && block_size % kTileTokens == 0;
}

int launch_mixed(const AttnArgs& a, int head_dim, int group, int num_decode_queues, int num_prefill_queues,
                 int tail_queue0, void* stream) {
    return launch_mixed_d<PKV_DTYPE_BF16>(a, head_dim, group, num_decode_queues, num_prefill_queues, tail_queue0,
                                          static_cast<hipStream_t>(stream));
}

bool prefill_supported(int q_dtype, int kv_dtype, int head_dim, int group) {
    return q_dtype == PKV_DTYPE_BF16 && (kv_dtype == PKV_DTYPE_BF16 || kv_dtype == PKV_DTYPE_FP8_E4M3) &&
           (head_dim == 64 || head_dim == 128) && (group == 1 || group == 2 || group == 4 || group == 8);
}

int launch_prefill(const AttnArgs& a, int q_dtype, int kv_dtype, int head_dim, int group, int max_q_len,
                   int num_queues, int queue0, void* stream) {
    hipStream_t st = static_cast<hipStream_t>(stream);
    if (!prefill_supported(q_dtype, kv_dtype, head_dim, group)) return PKV_ERR_UNSUPPORTED;
    // (row, q head) pairs of the largest unit
    const int max_pairs = static_cast<int>(std::min<int64_t>(static_cast<int64_t>(max_q_len) * group, kPrefillQRows));
    if (kv_dtype == PKV_DTYPE_BF16)
        return launch_prefill_d<PKV_DTYPE_BF16>(a, head_dim, group, max_pairs, num_queues, queue0, st);
    return launch_prefill_d<PKV_DTYPE_FP8_E4M3>(a, head_dim, group, max_pairs, num_queues, queue0, st);
}

}  // namespace pkv
