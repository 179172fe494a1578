// C ABI: argument checks, the plan upload and kernel launches.  Every check
// runs on the host before anything is launched; a failing check returns a
// negative status and leaves device memory untouched.
#include <algorithm>
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>

#include "pkv_attention.h"
#include "pkv_internal.h"

namespace {

using namespace pkv;

constexpr float kLog2e = 1.4426950408889634f;
// Persistent decode workgroups per compute unit.  One workgroup per CU
// streams fastest for bf16 on whole-tile pages (measured against two and
// more); the kernels that need more waves in flight (page sizes that are not
// a multiple of 16, fp8) use 16-wave workgroups instead, and the prefill
// launch takes two queues per decode queue.
constexpr int kQueuesPerCU = 1;

bool dtype_ok(int32_t dt) { return dt == PKV_DTYPE_F32 || dt == PKV_DTYPE_BF16 || dt == PKV_DTYPE_FP8_E4M3; }

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

bool attn_pair_ok(int32_t q_dtype, int32_t kv_dtype) {
    return (q_dtype == PKV_DTYPE_F32 && kv_dtype == PKV_DTYPE_F32) ||
           (q_dtype == PKV_DTYPE_BF16 && kv_dtype == PKV_DTYPE_BF16) ||
           (q_dtype == PKV_DTYPE_BF16 && kv_dtype == PKV_DTYPE_FP8_E4M3);
}

// Checks shared by decode and mixed.  `rows` = query rows in q/out.
int check_attention(void* out, const void* q, int32_t q_dtype, int64_t q_token_stride, const void* k_cache,
                    const void* v_cache, int32_t kv_dtype, const int32_t* block_tables, int32_t max_blocks,
                    const int32_t* context_lens, int32_t num_seqs, int32_t rows, int32_t hq, int32_t hkv,
                    int32_t d, int64_t num_blocks, int32_t block_size, float scale, float k_scale,
                    float v_scale, const pkv_plan* plan, void* workspace, size_t workspace_bytes) {
    if (!dtype_ok(q_dtype) || !dtype_ok(kv_dtype) || q_dtype == PKV_DTYPE_FP8_E4M3) return PKV_ERR_DTYPE;
    if (plan == nullptr) return PKV_ERR_NULL;
    if (num_seqs < 0 || rows < 0 || hq < 1 || hkv < 1 || hq % hkv != 0 || block_size < 1 || num_blocks < 1 ||
        max_blocks < 1)
        return PKV_ERR_SHAPE;
    if (d != 64 && d != 128) return PKV_ERR_UNSUPPORTED;
    const int32_t group = hq / hkv;
    if (group != 1 && group != 2 && group != 4 && group != 8) return PKV_ERR_UNSUPPORTED;
    if (!attn_pair_ok(q_dtype, kv_dtype)) return PKV_ERR_UNSUPPORTED;
    if (q_token_stride < static_cast<int64_t>(hq) * d) return PKV_ERR_SHAPE;
    if (!std::isfinite(scale)) return PKV_ERR_SHAPE;
    if (kv_dtype == PKV_DTYPE_FP8_E4M3 &&
        (!std::isfinite(k_scale) || !std::isfinite(v_scale) || k_scale <= 0.f || v_scale <= 0.f))
        return PKV_ERR_SHAPE;
    if (plan->magic != PKV_PLAN_MAGIC || plan->num_seqs != num_seqs || plan->num_tokens != rows ||
        plan->num_q_heads != hq || plan->num_kv_heads != hkv || plan->head_dim != d ||
        plan->num_wide_merges < 0 || plan->num_block_merges < 0 ||
        plan->num_wide_merges + plan->num_block_merges > plan->num_merges ||
        plan->num_wide_merges > plan->max_row_merges || plan->num_block_merges > plan->max_block_merges ||
        plan->num_merges - plan->num_block_merges > plan->max_row_merges || plan->window_left < 0 ||
        plan->num_tail_queues < 0 || plan->num_tail_queues > plan->num_prefill_queues ||
        (plan->num_tail_queues != 0 && plan->num_tail_queues != plan->num_queues) ||
        !(plan->logits_soft_cap >= 0.f) || !std::isfinite(plan->logits_soft_cap))
        return PKV_ERR_PLAN;
    if (rows == 0) return PKV_OK;
    if (out == nullptr || q == nullptr || k_cache == nullptr || v_cache == nullptr || block_tables == nullptr ||
        context_lens == nullptr || workspace == nullptr)
        return PKV_ERR_NULL;
    if (workspace_bytes < static_cast<size_t>(plan->workspace_bytes)) return PKV_ERR_WORKSPACE;
    // vector loads: every lane reads D/16 contiguous elements
    const size_t qb = static_cast<size_t>(dt_bytes(q_dtype));
    const size_t lane_q = static_cast<size_t>(d / 16) * qb;
    const size_t lane_kv = static_cast<size_t>(d / 16) * static_cast<size_t>(dt_bytes(kv_dtype));
    const size_t qa = lane_q >= 16 ? 16 : lane_q;
    const size_t kva = lane_kv >= 16 ? 16 : lane_kv;
    if (!aligned(q, qa) || (static_cast<size_t>(q_token_stride) * qb) % qa != 0 || !aligned(out, qa) ||
        !aligned(k_cache, kva) || !aligned(v_cache, kva) || !aligned(workspace, kAlign))
        return PKV_ERR_SHAPE;
    return PKV_OK;
}

AttnArgs make_args(void* out, const void* q, int64_t q_token_stride, const void* k_cache, const void* v_cache,
                   int32_t kv_dtype, const int32_t* block_tables, int32_t max_blocks, const int32_t* context_lens,
                   int32_t hq, int32_t hkv, int64_t num_blocks, int32_t block_size, float scale, float k_scale,
                   float v_scale, const pkv_plan* plan, void* workspace) {
    char* ws = static_cast<char*>(workspace);
    const bool fp8 = kv_dtype == PKV_DTYPE_FP8_E4M3;
    AttnArgs a;
    a.out = out;
    a.q = q;
    a.q_stride = q_token_stride;
    a.k_cache = k_cache;
    a.v_cache = v_cache;
    a.block_tables = block_tables;
    a.max_blocks = max_blocks;
    a.kv_indptr = nullptr;
    a.context_lens = context_lens;
    a.cu_seqlens = nullptr;
    a.hq = hq;
    a.hkv = hkv;
    a.num_blocks = num_blocks;
    a.block_size = block_size;
    a.block_shift = (block_size & (block_size - 1)) == 0 ? __builtin_ctz(static_cast<uint32_t>(block_size)) : -1;
    a.qk_scale = scale * (fp8 ? k_scale : 1.f) * kLog2e;
    a.v_scale = fp8 ? v_scale : 1.f;
    // the soft-cap in the scores' log2 units, and the exponent factor of
    // tanh(s / c) = 1 - 2 / (e^(2 s / c) + 1) for such scores
    a.soft_cap = plan->logits_soft_cap > 0.f ? plan->logits_soft_cap * kLog2e : 0.f;
    a.soft_cap_k = plan->logits_soft_cap > 0.f ? 2.f / plan->logits_soft_cap : 0.f;
    a.window = plan->window_left;
    a.units = reinterpret_cast<const Unit*>(ws + plan->off_units);
    a.queue_off = reinterpret_cast<const int32_t*>(ws + plan->off_queues);
    a.partial_o = reinterpret_cast<float*>(ws + plan->off_partial_o);
    a.partial_lse = reinterpret_cast<float*>(ws + plan->off_partial_lse);
    a.slot_mapping = nullptr;
    a.k_new = nullptr;
    a.v_new = nullptr;
    a.new_stride = 0;
    return a;
}

// Timing hook of pkv_set_split_event: recorded on a call's stream between
// its attention kernel and its merge kernel.  A record that fails is skipped
// (and its error cleared, so that the merge launch's check does not see it):
// the call's work is launched either way.
hipEvent_t g_split_event = nullptr;

int mark_split(void* stream) {
    if (g_split_event != nullptr && hipEventRecord(g_split_event, static_cast<hipStream_t>(stream)) != hipSuccess)
        (void)hipGetLastError();
    return PKV_OK;
}

}  // namespace

extern "C" {

int pkv_set_split_event(void* event) {
    g_split_event = static_cast<hipEvent_t>(event);
    return PKV_OK;
}

const char* paged_attn_strerror(int status) {
    switch (status) {
        case PKV_OK: return "ok";
        case PKV_ERR_NULL: return "a required pointer is NULL";
        case PKV_ERR_SHAPE: return "inconsistent sizes, strides, lengths or alignment";
        case PKV_ERR_DTYPE: return "unknown dtype code";
        case PKV_ERR_UNSUPPORTED: return "unsupported head_dim, group size or dtype pair";
        case PKV_ERR_WORKSPACE: return "workspace or host staging buffer too small";
        case PKV_ERR_PLAN: return "plan missing, stale or made for other shapes";
        case PKV_ERR_HIP: return "HIP runtime error or kernel launch failure";
        default: return "unknown status";
    }
}

int pkv_abi_version(void) { return PKV_ABI_VERSION; }

}  // extern "C"

// Checks of paged_kv_write, also made by the decode call that writes.
static int check_write(const void* k_new, const void* v_new, int32_t new_dtype, int64_t new_token_stride,
                       const int32_t* slot_mapping, int64_t num_tokens, const void* k_cache, const void* v_cache,
                       int32_t cache_dtype, int64_t num_blocks, int32_t block_size, int32_t num_kv_heads,
                       int32_t head_dim, float k_scale, float v_scale) {
    if (!dtype_ok(new_dtype) || !dtype_ok(cache_dtype) || new_dtype == PKV_DTYPE_FP8_E4M3) return PKV_ERR_DTYPE;
    const bool pair = (new_dtype == cache_dtype) || (new_dtype == PKV_DTYPE_F32 && cache_dtype == PKV_DTYPE_BF16) ||
                      cache_dtype == PKV_DTYPE_FP8_E4M3;
    if (!pair) return PKV_ERR_UNSUPPORTED;
    if (num_tokens < 0 || num_blocks < 1 || block_size < 1 || num_kv_heads < 1 || head_dim < 8 ||
        head_dim % 8 != 0 || static_cast<int64_t>(num_kv_heads) * head_dim > 65536)
        return PKV_ERR_SHAPE;
    const int64_t hd = static_cast<int64_t>(num_kv_heads) * head_dim;
    if (new_token_stride < hd || new_token_stride % 8 != 0) return PKV_ERR_SHAPE;
    if (cache_dtype == PKV_DTYPE_FP8_E4M3 &&
        (!std::isfinite(k_scale) || !std::isfinite(v_scale) || k_scale <= 0.f || v_scale <= 0.f))
        return PKV_ERR_SHAPE;
    if (num_tokens == 0) return PKV_OK;
    if (!k_new || !v_new || !slot_mapping || !k_cache || !v_cache) return PKV_ERR_NULL;
    const size_t in_align = 16;
    const size_t out_align = cache_dtype == PKV_DTYPE_FP8_E4M3 ? 8 : 16;
    if (!aligned(k_new, in_align) || !aligned(v_new, in_align) || !aligned(k_cache, out_align) ||
        !aligned(v_cache, out_align))
        return PKV_ERR_SHAPE;
    if (num_blocks > INT64_MAX / block_size) return PKV_ERR_SHAPE;
    return PKV_OK;
}

extern "C" {

int paged_kv_write(const void* k_new, const void* v_new, int32_t new_dtype, int64_t new_token_stride,
                   const int32_t* slot_mapping, int64_t num_tokens, void* k_cache, void* v_cache,
                   int32_t cache_dtype, int64_t num_blocks, int32_t block_size, int32_t num_kv_heads,
                   int32_t head_dim, float k_scale, float v_scale, void* stream) {
    const int st = check_write(k_new, v_new, new_dtype, new_token_stride, slot_mapping, num_tokens, k_cache, v_cache,
                               cache_dtype, num_blocks, block_size, num_kv_heads, head_dim, k_scale, v_scale);
    if (st != PKV_OK || num_tokens == 0) return st;
    const int64_t hd = static_cast<int64_t>(num_kv_heads) * head_dim;
    return launch_kv_write(k_new, v_new, new_dtype, new_token_stride, slot_mapping, num_tokens, k_cache, v_cache,
                           cache_dtype, num_blocks * block_size, static_cast<int32_t>(hd), k_scale, v_scale,
                           stream);
}

int paged_attn_default_queues(int32_t* num_queues) {
    if (num_queues == nullptr) return PKV_ERR_NULL;
    int dev = 0;
    int cus = 0;
    if (hipGetDevice(&dev) != hipSuccess) return PKV_ERR_HIP;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus < 1)
        return PKV_ERR_HIP;
    *num_queues = cus * kQueuesPerCU;
    return PKV_OK;
}

int paged_attn_workspace_size(int32_t max_seqs, int32_t max_tokens, int32_t num_q_heads, int32_t head_dim,
                              int32_t num_queues, size_t* workspace_bytes, size_t* host_bytes) {
    if (workspace_bytes == nullptr && host_bytes == nullptr) return PKV_ERR_NULL;
    if (max_seqs < 0 || max_tokens < 0 || num_q_heads < 1 || head_dim < 1) return PKV_ERR_SHAPE;
    if (num_queues <= 0) {
        const int st = paged_attn_default_queues(&num_queues);
        if (st != PKV_OK) return st;
    }
    plan_bounds(max_seqs, max_tokens, num_q_heads, head_dim, num_queues, workspace_bytes, host_bytes);
    return PKV_OK;
}

int paged_attn_plan_host(const int32_t* context_lens_host, const int32_t* q_lens_host, int32_t num_seqs,
                         int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim, int32_t num_queues,
                         void* host_image, size_t host_bytes, pkv_plan* plan) {
    return plan_host(context_lens_host, q_lens_host, num_seqs, num_q_heads, num_kv_heads, head_dim, num_queues,
                     host_image, host_bytes, plan);
}

int paged_attn_plan_variant(const int32_t* context_lens_host, const int32_t* q_lens_host, int32_t num_seqs,
                            int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim, int32_t num_queues,
                            float logits_soft_cap, int32_t window_left, int32_t max_seqs, int32_t max_tokens,
                            void* host_staging, size_t host_staging_bytes, void* workspace, size_t workspace_bytes,
                            pkv_plan* plan, void* stream) {
    if (plan == nullptr) return PKV_ERR_NULL;
    if (workspace == nullptr) {  // host only
        return plan_host(context_lens_host, q_lens_host, num_seqs, num_q_heads, num_kv_heads, head_dim, num_queues,
                         host_staging, host_staging_bytes, plan, max_seqs >= 0 ? max_seqs : -1,
                         max_seqs >= 0 ? max_tokens : -1, logits_soft_cap, window_left);
    }
    if (host_staging == nullptr) return PKV_ERR_NULL;
    if (max_seqs >= 0 && max_tokens < 0) return PKV_ERR_SHAPE;
    if (num_queues <= 0) {
        const int st = paged_attn_default_queues(&num_queues);
        if (st != PKV_OK) return st;
    }
    int st = plan_host(context_lens_host, q_lens_host, num_seqs, num_q_heads, num_kv_heads, head_dim, num_queues,
                       host_staging, host_staging_bytes, plan, max_seqs >= 0 ? max_seqs : -1,
                       max_seqs >= 0 ? max_tokens : -1, logits_soft_cap, window_left);
    if (st != PKV_OK) return st;
    if (workspace_bytes < static_cast<size_t>(plan->workspace_bytes) || !aligned(workspace, kAlign)) {
        plan->magic = 0;
        return PKV_ERR_WORKSPACE;
    }
    if (hipMemcpyAsync(workspace, host_staging, static_cast<size_t>(plan->image_bytes), hipMemcpyHostToDevice,
                       static_cast<hipStream_t>(stream)) != hipSuccess) {
        plan->magic = 0;
        return PKV_ERR_HIP;
    }
    return PKV_OK;
}

int paged_attn_plan(const int32_t* context_lens_host, const int32_t* q_lens_host, int32_t num_seqs,
                    int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim, int32_t num_queues,
                    void* host_staging, size_t host_staging_bytes, void* workspace, size_t workspace_bytes,
                    pkv_plan* plan, void* stream) {
    if (plan == nullptr || host_staging == nullptr || workspace == nullptr) return PKV_ERR_NULL;
    return paged_attn_plan_variant(context_lens_host, q_lens_host, num_seqs, num_q_heads, num_kv_heads, head_dim,
                                   num_queues, 0.f, 0, -1, -1, host_staging, host_staging_bytes, workspace,
                                   workspace_bytes, plan, stream);
}

int paged_attn_plan_capacity(const int32_t* context_lens_host, const int32_t* q_lens_host, int32_t num_seqs,
                             int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim, int32_t num_queues,
                             int32_t max_seqs, int32_t max_tokens, void* host_staging, size_t host_staging_bytes,
                             void* workspace, size_t workspace_bytes, pkv_plan* plan, void* stream) {
    if (plan == nullptr || host_staging == nullptr || workspace == nullptr) return PKV_ERR_NULL;
    if (max_seqs < 0 || max_tokens < 0) return PKV_ERR_SHAPE;
    return paged_attn_plan_variant(context_lens_host, q_lens_host, num_seqs, num_q_heads, num_kv_heads, head_dim,
                                   num_queues, 0.f, 0, max_seqs, max_tokens, host_staging, host_staging_bytes,
                                   workspace, workspace_bytes, plan, stream);
}

}  // extern "C"

// Decode over dense rows (kv_indptr null) or CSR rows (block_tables holds
// kv_indices, max_blocks_per_seq is unused).
static int decode_impl(void* out, const void* q, int32_t q_dtype, int64_t q_token_stride, const void* k_cache,
                       const void* v_cache, int32_t kv_dtype, const int32_t* block_tables,
                       int32_t max_blocks_per_seq, const int32_t* kv_indptr, const int32_t* context_lens,
                       int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                       int64_t num_blocks, int32_t block_size, float scale, float k_scale, float v_scale,
                       const pkv_plan* plan, void* workspace, size_t workspace_bytes, void* stream,
                       const AttnArgs* write = nullptr) {
    int st = check_attention(out, q, q_dtype, q_token_stride, k_cache, v_cache, kv_dtype, block_tables,
                             max_blocks_per_seq, context_lens, num_seqs, num_seqs, num_q_heads, num_kv_heads,
                             head_dim, num_blocks, block_size, scale, k_scale, v_scale, plan, workspace,
                             workspace_bytes);
    if (st != PKV_OK) return st;
    if (plan->max_q_len > 1) return PKV_ERR_PLAN;
    if (num_seqs == 0) return PKV_OK;
    AttnArgs a = make_args(out, q, q_token_stride, k_cache, v_cache, kv_dtype, block_tables, max_blocks_per_seq,
                           context_lens, num_q_heads, num_kv_heads, num_blocks, block_size, scale, k_scale, v_scale,
                           plan, workspace);
    a.kv_indptr = kv_indptr;
    if (write != nullptr) {
        a.slot_mapping = write->slot_mapping;
        a.k_new = write->k_new;
        a.v_new = write->v_new;
        a.new_stride = write->new_stride;
        st = launch_decode_write(a, head_dim, num_q_heads / num_kv_heads, plan->num_queues, stream);
        if (st == PKV_OK) st = mark_split(stream);
        if (st != PKV_OK) return st;
        return launch_merge(a, plan, workspace, 1, q_dtype, head_dim, stream);
    }
    const int group = num_q_heads / num_kv_heads;
    // fp8 caches: the few-row kernel (products on the matrix cores, the
    // widening done once as a tile is staged) instead of the vector decode
    // unit, whose widening and dot products bound it
    if (kv_dtype == PKV_DTYPE_FP8_E4M3 && fewrow_capable(q_dtype, kv_dtype, head_dim, block_size) &&
        prefill_supported(q_dtype, kv_dtype, head_dim, group))
        st = launch_fewrow(a, q_dtype, kv_dtype, head_dim, group, plan->num_queues, stream);
    else
        st = launch_decode(a, q_dtype, kv_dtype, head_dim, group, plan->num_queues, stream);
    if (st == PKV_OK) st = mark_split(stream);
    if (st != PKV_OK) return st;
    return launch_merge(a, plan, workspace, 1, q_dtype, head_dim, stream);
}

extern "C" {

int paged_attn_decode(void* out, const void* q, int32_t q_dtype, int64_t q_token_stride, const void* k_cache,
                      const void* v_cache, int32_t kv_dtype, const int32_t* block_tables,
                      int32_t max_blocks_per_seq, const int32_t* context_lens, int32_t num_seqs,
                      int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim, int64_t num_blocks,
                      int32_t block_size, float scale, float k_scale, float v_scale, const pkv_plan* plan,
                      void* workspace, size_t workspace_bytes, void* stream) {
    if (block_tables == nullptr && num_seqs > 0) return PKV_ERR_NULL;
    return decode_impl(out, q, q_dtype, q_token_stride, k_cache, v_cache, kv_dtype, block_tables, max_blocks_per_seq,
                       nullptr, context_lens, num_seqs, num_q_heads, num_kv_heads, head_dim, num_blocks, block_size,
                       scale, k_scale, v_scale, plan, workspace, workspace_bytes, stream);
}

int paged_attn_decode_write(void* out, const void* q, int32_t q_dtype, int64_t q_token_stride, const void* k_new,
                            const void* v_new, int32_t new_dtype, int64_t new_token_stride,
                            const int32_t* slot_mapping, void* k_cache, void* v_cache, int32_t kv_dtype,
                            const int32_t* block_tables, int32_t max_blocks_per_seq, const int32_t* context_lens,
                            int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                            int64_t num_blocks, int32_t block_size, float scale, float k_scale, float v_scale,
                            const pkv_plan* plan, void* workspace, size_t workspace_bytes, void* stream) {
    if (block_tables == nullptr && num_seqs > 0) return PKV_ERR_NULL;
    // every check of both calls before anything is launched
    int st = check_write(k_new, v_new, new_dtype, new_token_stride, slot_mapping, num_seqs, k_cache, v_cache,
                         kv_dtype, num_blocks, block_size, num_kv_heads, head_dim, k_scale, v_scale);
    if (st != PKV_OK) return st;
    st = check_attention(out, q, q_dtype, q_token_stride, k_cache, v_cache, kv_dtype, block_tables,
                         max_blocks_per_seq, context_lens, num_seqs, num_seqs, num_q_heads, num_kv_heads, head_dim,
                         num_blocks, block_size, scale, k_scale, v_scale, plan, workspace, workspace_bytes);
    if (st != PKV_OK) return st;
    if (plan->max_q_len > 1) return PKV_ERR_PLAN;
    if (num_seqs == 0) return PKV_OK;
    // one launch for bf16 tokens into a bf16 cache on pages of whole tiles
    // (copied as they are, in 16-byte pieces); otherwise the write kernel and
    // then the decode call
    const size_t eb = static_cast<size_t>(dt_bytes(kv_dtype));
    // (a thread of the 512 copies at most two 16-byte pieces of a token)
    const bool one = q_dtype == PKV_DTYPE_BF16 && kv_dtype == PKV_DTYPE_BF16 && new_dtype == PKV_DTYPE_BF16 &&
                     block_size % kTileTokens == 0 && num_kv_heads * head_dim <= 4096 &&
                     aligned(k_new, 16) && aligned(v_new, 16) &&
                     (static_cast<size_t>(new_token_stride) * eb) % 16 == 0 &&
                     (static_cast<size_t>(num_kv_heads) * static_cast<size_t>(head_dim) * eb) % 16 == 0;
    if (!one) {
        st = paged_kv_write(k_new, v_new, new_dtype, new_token_stride, slot_mapping, num_seqs, k_cache, v_cache,
                            kv_dtype, num_blocks, block_size, num_kv_heads, head_dim, k_scale, v_scale, stream);
        if (st != PKV_OK) return st;
        return decode_impl(out, q, q_dtype, q_token_stride, k_cache, v_cache, kv_dtype, block_tables,
                           max_blocks_per_seq, nullptr, context_lens, num_seqs, num_q_heads, num_kv_heads, head_dim,
                           num_blocks, block_size, scale, k_scale, v_scale, plan, workspace, workspace_bytes, stream);
    }
    AttnArgs w{};
    w.slot_mapping = slot_mapping;
    w.k_new = k_new;
    w.v_new = v_new;
    w.new_stride = new_token_stride;
    return decode_impl(out, q, q_dtype, q_token_stride, k_cache, v_cache, kv_dtype, block_tables, max_blocks_per_seq,
                       nullptr, context_lens, num_seqs, num_q_heads, num_kv_heads, head_dim, num_blocks, block_size,
                       scale, k_scale, v_scale, plan, workspace, workspace_bytes, stream, &w);
}

int paged_attn_decode_noalloc(void* out, const void* q, int32_t q_dtype, int64_t q_token_stride,
                              const void* k_cache, const void* v_cache, int32_t kv_dtype,
                              const int32_t* block_tables, int32_t max_blocks_per_seq, const int32_t* context_lens,
                              int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                              int64_t num_blocks, int32_t block_size, float scale, float k_scale, float v_scale,
                              const pkv_plan* plan, const void* plan_image_host, void* stream) {
    if (plan == nullptr) return PKV_ERR_NULL;
    // the plan must fit the scratch array; checked before any HIP call
    if (plan->magic != PKV_PLAN_MAGIC) return PKV_ERR_PLAN;
    if (plan->workspace_bytes < 0 || static_cast<size_t>(plan->workspace_bytes) > kNoallocScratchBytes)
        return PKV_ERR_WORKSPACE;
    if (block_tables == nullptr && num_seqs > 0) return PKV_ERR_NULL;
    if (num_seqs > 0 && plan->image_bytes > 0 && plan_image_host == nullptr) return PKV_ERR_NULL;
    // every check of the attention call before any HIP call; the scratch
    // array stands in as the workspace (non-null, aligned, of its size)
    int st = check_attention(out, q, q_dtype, q_token_stride, k_cache, v_cache, kv_dtype, block_tables,
                             max_blocks_per_seq, context_lens, num_seqs, num_seqs, num_q_heads, num_kv_heads,
                             head_dim, num_blocks, block_size, scale, k_scale, v_scale, plan,
                             reinterpret_cast<void*>(kAlign), kNoallocScratchBytes);
    if (st != PKV_OK || num_seqs == 0) return st;
    if (plan->max_q_len > 1) return PKV_ERR_PLAN;
    void* ws = nullptr;
    st = noalloc_scratch(&ws);
    if (st != PKV_OK) return st;
    if (hipMemcpyAsync(ws, plan_image_host, static_cast<size_t>(plan->image_bytes), hipMemcpyHostToDevice,
                       static_cast<hipStream_t>(stream)) != hipSuccess)
        return PKV_ERR_HIP;
    return decode_impl(out, q, q_dtype, q_token_stride, k_cache, v_cache, kv_dtype, block_tables, max_blocks_per_seq,
                       nullptr, context_lens, num_seqs, num_q_heads, num_kv_heads, head_dim, num_blocks, block_size,
                       scale, k_scale, v_scale, plan, ws, kNoallocScratchBytes, stream);
}

int paged_attn_decode_csr(void* out, const void* q, int32_t q_dtype, int64_t q_token_stride, const void* k_cache,
                          const void* v_cache, int32_t kv_dtype, const int32_t* kv_indptr,
                          const int32_t* kv_indices, const int32_t* context_lens, int32_t num_seqs,
                          int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim, int64_t num_blocks,
                          int32_t block_size, float scale, float k_scale, float v_scale, const pkv_plan* plan,
                          void* workspace, size_t workspace_bytes, void* stream) {
    if (num_seqs > 0 && (kv_indptr == nullptr || kv_indices == nullptr)) return PKV_ERR_NULL;
    return decode_impl(out, q, q_dtype, q_token_stride, k_cache, v_cache, kv_dtype, kv_indices, 1, kv_indptr,
                       context_lens, num_seqs, num_q_heads, num_kv_heads, head_dim, num_blocks, block_size, scale,
                       k_scale, v_scale, plan, workspace, workspace_bytes, stream);
}

}  // extern "C"

// Most rows of any merge record: decode merges have one, prefill merges a row block.
static int merge_rows(const pkv_plan* plan, int group) {
    if (plan->max_q_len <= 1) return 1;
    return std::max(1, std::min(plan->max_q_len, std::max(1, kPrefillQRows / group)));
}

static int mixed_impl(void* out, const void* q, int32_t q_dtype, int64_t q_token_stride, const void* k_cache,
                      const void* v_cache, int32_t kv_dtype, const int32_t* block_tables,
                      int32_t max_blocks_per_seq, const int32_t* kv_indptr, const int32_t* cu_seqlens,
                      const int32_t* context_lens, int32_t num_seqs, int32_t num_tokens, int32_t num_q_heads,
                      int32_t num_kv_heads, int32_t head_dim, int64_t num_blocks, int32_t block_size, float scale,
                      float k_scale, float v_scale, const pkv_plan* plan, void* workspace, size_t workspace_bytes,
                      void* stream) {
    int st = check_attention(out, q, q_dtype, q_token_stride, k_cache, v_cache, kv_dtype, block_tables,
                             max_blocks_per_seq, context_lens, num_seqs, num_tokens, num_q_heads, num_kv_heads,
                             head_dim, num_blocks, block_size, scale, k_scale, v_scale, plan, workspace,
                             workspace_bytes);
    if (st != PKV_OK) return st;
    if (num_tokens == 0) return PKV_OK;
    if (cu_seqlens == nullptr) return PKV_ERR_NULL;
    AttnArgs a = make_args(out, q, q_token_stride, k_cache, v_cache, kv_dtype, block_tables, max_blocks_per_seq,
                           context_lens, num_q_heads, num_kv_heads, num_blocks, block_size, scale, k_scale, v_scale,
                           plan, workspace);
    a.kv_indptr = kv_indptr;
    a.cu_seqlens = cu_seqlens;
    const int group = num_q_heads / num_kv_heads;
    const bool chunks = plan->num_prefill_units > 0;
    // a few-row step: the sequences' rows sit in decode-queue units
    const bool few = !chunks && plan->max_q_len > 1;
    if ((chunks || few) && !prefill_supported(q_dtype, kv_dtype, head_dim, group)) return PKV_ERR_UNSUPPORTED;
    // the prefill and few-row tiles load 8 elements of a key at a time
    const size_t item = 8 * static_cast<size_t>(dt_bytes(kv_dtype));
    if ((chunks || few) && (!aligned(k_cache, item) || !aligned(v_cache, item))) return PKV_ERR_SHAPE;
    const bool decode_rows = plan->num_units > plan->num_prefill_units;
    if (few) {
        st = launch_fewrow(a, q_dtype, kv_dtype, head_dim, group, plan->num_queues, stream);
        if (st == PKV_OK) st = mark_split(stream);
        if (st != PKV_OK) return st;
        return launch_merge(a, plan, workspace, merge_rows(plan, group), q_dtype, head_dim, stream);
    }
    // decode rows and chunks side by side in one launch, each decode
    // workgroup then running its tail queue; chunks alone take the prefill
    // kernel, whose wide form needs no room for a decode workgroup on the CU.
    // In two launches the tails are prefill workgroups like the others.
    if (chunks && decode_rows && mixed_one_launch(q_dtype, kv_dtype, head_dim, group, block_size)) {
        const int main_queues = plan->num_prefill_queues - plan->num_tail_queues;
        st = launch_mixed(a, head_dim, group, plan->num_queues, main_queues,
                          plan->num_tail_queues > 0 ? plan->num_queues + main_queues : -1, stream);
        if (st == PKV_OK) st = mark_split(stream);
        if (st != PKV_OK) return st;
        return launch_merge(a, plan, workspace, merge_rows(plan, group), q_dtype, head_dim, stream);
    }
    if (decode_rows) {
        st = launch_decode(a, q_dtype, kv_dtype, head_dim, group, plan->num_queues, stream);
        if (st != PKV_OK) return st;
    }
    if (chunks) {
        st = launch_prefill(a, q_dtype, kv_dtype, head_dim, group, plan->max_q_len, plan->num_prefill_queues,
                            plan->num_queues, stream);
        if (st != PKV_OK) return st;
    }
    st = mark_split(stream);
    if (st != PKV_OK) return st;
    return launch_merge(a, plan, workspace, merge_rows(plan, group), q_dtype, head_dim, stream);
}

extern "C" {

int paged_attn_mixed(void* out, const void* q, int32_t q_dtype, int64_t q_token_stride, const void* k_cache,
                     const void* v_cache, int32_t kv_dtype, const int32_t* block_tables,
                     int32_t max_blocks_per_seq, const int32_t* cu_seqlens, const int32_t* context_lens,
                     int32_t num_seqs, int32_t num_tokens, int32_t num_q_heads, int32_t num_kv_heads,
                     int32_t head_dim, int64_t num_blocks, int32_t block_size, float scale, float k_scale,
                     float v_scale, const pkv_plan* plan, void* workspace, size_t workspace_bytes,
                     void* stream) {
    if (block_tables == nullptr && num_tokens > 0) return PKV_ERR_NULL;
    return mixed_impl(out, q, q_dtype, q_token_stride, k_cache, v_cache, kv_dtype, block_tables, max_blocks_per_seq,
                      nullptr, cu_seqlens, context_lens, num_seqs, num_tokens, num_q_heads, num_kv_heads, head_dim,
                      num_blocks, block_size, scale, k_scale, v_scale, plan, workspace, workspace_bytes, stream);
}

int paged_attn_mixed_csr(void* out, const void* q, int32_t q_dtype, int64_t q_token_stride, const void* k_cache,
                         const void* v_cache, int32_t kv_dtype, const int32_t* kv_indptr, const int32_t* kv_indices,
                         const int32_t* cu_seqlens, const int32_t* context_lens, int32_t num_seqs,
                         int32_t num_tokens, int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                         int64_t num_blocks, int32_t block_size, float scale, float k_scale, float v_scale,
                         const pkv_plan* plan, void* workspace, size_t workspace_bytes, void* stream) {
    if (num_tokens > 0 && (kv_indptr == nullptr || kv_indices == nullptr)) return PKV_ERR_NULL;
    return mixed_impl(out, q, q_dtype, q_token_stride, k_cache, v_cache, kv_dtype, kv_indices, 1, kv_indptr,
                      cu_seqlens, context_lens, num_seqs, num_tokens, num_q_heads, num_kv_heads, head_dim, num_blocks,
                      block_size, scale, k_scale, v_scale, plan, workspace, workspace_bytes, stream);
}

}  // extern "C"
