// Arguments and launchers of the attention kernels (decode, mixed, merge).
#pragma once

#include "pkv_device.h"
#include "pkv_internal.h"

namespace pkv {

constexpr int dt_bytes(int dt) { return dt == PKV_DTYPE_F32 ? 4 : (dt == PKV_DTYPE_BF16 ? 2 : 1); }

struct AttnArgs {
    void* out;                    // [T][hq][D], q's dtype, contiguous
    const void* q;                // [T][hq][D] with token stride q_stride
    int64_t q_stride;             // elements
    const void* k_cache;          // [num_blocks][block_size][hkv][D]
    const void* v_cache;
    const int32_t* block_tables;  // [B][max_blocks], or the CSR entries kv_indices
    int32_t max_blocks;
    const int32_t* kv_indptr;     // [B + 1] CSR row offsets into block_tables, or null (dense rows)
    const int32_t* context_lens;  // [B]
    const int32_t* cu_seqlens;    // [B + 1] packed row offsets (mixed calls), or null (decode: row s is sequence s)
    int32_t hq;
    int32_t hkv;
    int64_t num_blocks;
    int32_t block_size;
    int32_t block_shift;          // log2(block_size) when a power of two, else -1
    float qk_scale;               // scale * k_scale * log2(e): scores in log2 units
    float v_scale;                // applied to the final output
    float soft_cap;               // logit soft-cap in log2 units (cap * log2 e), 0: off
    float soft_cap_k;             // 2 log2(e) / soft_cap: tanh(s / cap) = 1 - 2 / (2^(s * soft_cap_k) + 1)
    int32_t window;               // keys visible to a row at position p: p - window < j <= p; 0: all
    const Unit* units;
    const int32_t* queue_off;
    float* partial_o;             // [rows][hq][D]
    float* partial_lse;           // [rows][hq], log2 units
    // A decode step's new tokens written by the decode launch itself (null:
    // no write): row s of k_new / v_new ([B][hkv][D], the cache's dtype,
    // token stride new_stride elements) into slot slot_mapping[s].
    const int32_t* slot_mapping;
    const void* k_new;
    const void* v_new;
    int64_t new_stride;
};

// A score s in log2 units under the logit soft-cap c (log2 units too):
// c * tanh(s / c), with tanh(x) = 1 - 2 / (e^(2x) + 1) and e^(2x) =
// 2^(s * 2 / c) since s and c carry the same factor log2 e.  Saturates to
// +-c for large |s| (2^x overflows to inf or underflows to 0).
__device__ __forceinline__ float soft_cap_log2(float s, float cap, float cap_k) {
    const float e = exp2_fast(s * cap_k);
    return cap * (1.f - 2.f * __builtin_amdgcn_rcpf(e + 1.f));
}

// Index in the block table of the page holding token t, and t's row in it
// (shifts for a power-of-two page size, else a division).
__device__ __forceinline__ int page_of(const AttnArgs& a, int t) {
    return a.block_shift >= 0 ? t >> a.block_shift : t / a.block_size;
}
__device__ __forceinline__ int row_in_page(const AttnArgs& a, int t, int pidx) { return t - pidx * a.block_size; }

// The page-table row of one sequence: its entries and their number.  Dense
// tables give every sequence max_blocks entries; a CSR table ("How Easy Is It
// to Start Serving LLMs?", Phase 4 §1: kv_indptr / kv_indices) gives sequence
// s the entries kv_indptr[s] .. kv_indptr[s+1] - 1.  An empty CSR row points
// at kv_indptr[0] (so that a clamped read stays in bounds) with n = 0, which
// makes every page of it invalid.
struct SeqTable {
    const_ptr<int32_t> p;
    int32_t n;
    // entry i clamped into the row (read unconditionally; the caller checks i < n)
    __device__ __forceinline__ int32_t clamped(int i) const { return p[max(0, min(i, n - 1))]; }
    __device__ __forceinline__ int32_t operator[](int i) const { return p[i]; }
};

__device__ __forceinline__ SeqTable seq_table(const AttnArgs& a, int seq) {
    if (a.kv_indptr != nullptr) {
        const const_ptr<int32_t> ip = as_const(a.kv_indptr);
        const int32_t b = ip[seq];
        const int32_t n = ip[seq + 1] - b;
        return n > 0 ? SeqTable{as_const(a.block_tables) + b, n} : SeqTable{ip, 0};
    }
    return SeqTable{as_const(a.block_tables) + static_cast<int64_t>(seq) * a.max_blocks, a.max_blocks};
}

// Whether the device-side lengths and row offsets of a unit's sequence
// disagree with what the plan was made from (a stale plan, or cu_seqlens
// that are not the prefix sums of the plan's q_lens).  The unit's rows r =
// 0 .. nrows-1 sit at packed rows row0 + r and positions pos0 + r: with the
// device's n keys and L = cu[s+1] - cu[s] rows, row row0 + r is row row0 +
// r - cu[s] of the sequence and sits at n - L + row0 + r - cu[s].  Decode
// calls (no cu_seqlens) have row s = sequence s and one row each.
__device__ __forceinline__ bool unit_is_stale(const AttnArgs& a, const Unit& u) {
    const int32_t n = as_const(a.context_lens)[u.seq];
    if (a.cu_seqlens == nullptr) return n != u.pos0 + 1;
    const const_ptr<int32_t> cu = as_const(a.cu_seqlens);
    const int32_t c0 = cu[u.seq], c1 = cu[u.seq + 1];
    const int32_t r0 = u.row0 - c0;  // the unit's first row within the sequence
    return r0 < 0 || r0 + u.nrows > c1 - c0 || u.pos0 != n - (c1 - c0) + r0;
}

__device__ __forceinline__ Unit load_unit(const_ptr<Unit> units, int i) {
    const const_ptr<int32_t> w = reinterpret_cast<const_ptr<int32_t>>(units + i);
    return Unit{w[0], w[1], w[2], w[3], w[4], w[5], w[6], w[7]};
}

// Store EPL fp32 values as the output dtype (bf16: round to nearest even).
template <int QDT, int EPL>
__device__ __forceinline__ void store_out(char* dst, const float (&o)[EPL]) {
    if constexpr (QDT == PKV_DTYPE_F32) {
        Words<EPL> w;
#pragma unroll
        for (int e = 0; e < EPL; ++e) w.w[e] = __float_as_uint(o[e]);
        store_words<EPL>(dst, w);
    } else {
        Words<EPL / 2> w;
#pragma unroll
        for (int j = 0; j < EPL / 2; ++j) w.w[j] = f32_to_bf16_rne(o[2 * j]) | (f32_to_bf16_rne(o[2 * j + 1]) << 16);
        store_words<EPL / 2>(dst, w);
    }
}

int launch_decode(const AttnArgs& a, int q_dtype, int kv_dtype, int head_dim, int group, int num_queues,
                  void* stream);
// The decode kernel that also writes the step's new tokens (bf16 q and K/V,
// pages of whole 16-token tiles; a.slot_mapping set).
int launch_decode_write(const AttnArgs& a, int head_dim, int group, int num_queues, void* stream);
// Prefill chunks: the prefill queues queue0 .. queue0 + num_queues - 1 of
// the plan; max_q_len (the plan's longest chunk) picks the tile width.
bool prefill_supported(int q_dtype, int kv_dtype, int head_dim, int group);
int launch_prefill(const AttnArgs& a, int q_dtype, int kv_dtype, int head_dim, int group, int max_q_len,
                   int num_queues, int queue0, void* stream);
// A few-row step (every unit on the decode queues, holding a sequence's few
// rows and every kv head): the few-row kernel (bf16 q, bf16 or fp8 K/V,
// D = 128, pages of a power of two >= 16 tokens: fewrow_capable), or the
// register-staged prefill tile where that kernel does not serve the cache.
// The few-row kernel also runs decode calls on fp8 caches.
bool fewrow_capable(int q_dtype, int kv_dtype, int head_dim, int block_size);
int launch_fewrow(const AttnArgs& a, int q_dtype, int kv_dtype, int head_dim, int group, int num_queues,
                  void* stream);
// Decode rows and chunks of a mixed step in one launch (bf16 K/V on pages of
// whole tiles, groups 2 and 4, where one workgroup of each fits a CU):
// num_prefill_queues prefill workgroups beside the decode ones, and decode
// workgroup q then runs prefill queue tail_queue0 + q (tail_queue0 < 0: no
// tails).
bool mixed_one_launch(int q_dtype, int kv_dtype, int head_dim, int group, int block_size);
int launch_mixed(const AttnArgs& a, int head_dim, int group, int num_decode_queues, int num_prefill_queues,
                 int tail_queue0, void* stream);
// max_rows: the most rows of any merge record (1 for a decode-only plan).
int launch_merge(const AttnArgs& a, const pkv_plan* plan, const void* workspace, int max_rows, int q_dtype,
                 int head_dim, void* stream);
int launch_kv_write(const void* k_new, const void* v_new, int32_t new_dtype, int64_t stride_elems,
                    const int32_t* slots, int64_t T, void* kc, void* vc, int32_t cache_dtype, int64_t num_slots,
                    int32_t hd, float ks, float vs, void* stream);

}  // namespace pkv
