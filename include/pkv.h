/*
 * pkv.h - C ABI of a paged-KV attention library for AMD MI355X (gfx950).
 *
 * Three operations of an LLM serving step, over a KV cache held as a pool of
 * fixed-size blocks:
 *
 *   paged_kv_write     this step's new K/V rows go to the physical slots a
 *                      per-token slot list names;
 *   paged_attn_decode  one query row per sequence attends over its whole
 *                      context, read in place through a per-sequence block
 *                      table with an online softmax, long contexts split
 *                      into pieces that a merge joins back together;
 *   paged_attn_mixed   the same over a packed batch in which some sequences
 *                      bring a chunk of several new rows (chunked prefill)
 *                      and the rest one row each (decode).
 *
 * Sources (the pages this library follows):
 *   "nanoserve" (README): the paged KV cache and per-request block table; the
 *     packed [T] token batch; the engine step, where each layer stores the
 *     new tokens' K/V by slot before its attention reads the whole context
 *     through the block table; the paged decode kernel with a running
 *     softmax; the split of a mixed step into decode rows and prefill
 *     chunks.
 *   "How to design an LLM serving system (a vLLM deep dive)", section
 *     "PagedAttention": block table, slot_mapping, default block size 16;
 *     "Two phases and the KV cache": kv bytes per token.
 *   "How Easy Is It to Start Serving LLMs?", Phase 4 §1 (the block-sparse
 *     page table: a request reads the pool at the page ids its row lists,
 *     shared prompt pages are listed by several requests) and §3 (load
 *     balancing: a host-side plan once per step splits long requests into
 *     pieces and packs them evenly onto the processors, every layer reuses
 *     it from a fixed device buffer, and a merge joins the pieces).
 *
 * Conventions for every entry point:
 *   - All pointers are device pointers unless the name ends in _host.  The
 *     caller owns every buffer; no call allocates or frees memory.
 *   - Calls are asynchronous on `stream` (a hipStream_t passed as void*;
 *     NULL is the null stream).  The returned status covers host-side
 *     argument checks and launch errors only; it is returned before any
 *     device work runs and nothing is launched when it is not PKV_OK.
 *   - Index arrays are int32; address arithmetic is 64-bit.
 *   - Layouts (row-major, innermost last):
 *       k_cache, v_cache  [num_blocks][block_size][num_kv_heads][head_dim]
 *       block_tables      [num_seqs][max_blocks_per_seq]
 *       q, out            [num_tokens][num_q_heads][head_dim]; consecutive
 *                         tokens of q are q_token_stride elements apart
 *       k_new, v_new      [num_tokens][num_kv_heads][head_dim]; consecutive
 *                         tokens new_token_stride elements apart
 *   - Query head h reads kv head h / (num_q_heads / num_kv_heads).
 *   - context_lens[s] counts the keys of sequence s after this step's write.
 *     A chunk of L rows over n keys is aligned at the bottom right: its row i
 *     sits at position n - L + i and sees keys 0 .. n - L + i.
 *   - Device-side contents are trusted except where stated: a block id
 *     outside [0, num_blocks) is never dereferenced; the rows of a sequence
 *     whose table holds one come out as NaN.  Every unit of work takes its
 *     key range and rows from the plan; a sequence whose context_lens entry
 *     (or, in a packed batch, whose cu_seqlens entries) differ from what the
 *     plan was made from (a stale plan) gets NaN in the rows the plan gives
 *     it.
 *   - Calls that share a workspace must be ordered on one stream.
 */
#ifndef PKV_H_
#define PKV_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define PKV_ABI_VERSION 6

/* Status codes. */
#define PKV_OK 0
#define PKV_ERR_NULL (-1)        /* a required pointer is NULL */
#define PKV_ERR_SHAPE (-2)       /* inconsistent sizes (heads, lengths, strides) */
#define PKV_ERR_DTYPE (-3)       /* unknown dtype code */
#define PKV_ERR_UNSUPPORTED (-4) /* valid but not built: head_dim, group size, dtype pair */
#define PKV_ERR_WORKSPACE (-5)   /* workspace or host staging buffer too small */
#define PKV_ERR_PLAN (-6)        /* plan missing, stale or made for other shapes */
#define PKV_ERR_HIP (-7)         /* a HIP runtime call or kernel launch failed */

/* Storage dtypes. */
#define PKV_DTYPE_F32 0      /* IEEE binary32 */
#define PKV_DTYPE_BF16 1     /* bfloat16 */
#define PKV_DTYPE_FP8_E4M3 2 /* OCP FP8 E4M3 (bias 7, max 448, no inf), one fp32 scale per tensor */

/*
 * Split-KV plan: a host-side description of work the planner placed in a
 * workspace.  Filled by paged_attn_plan / paged_attn_plan_host; treat as
 * opaque.  It stays valid for every call that uses the same workspace, the
 * same lengths and the same head shape (e.g. all layers of one step).
 */
typedef struct pkv_plan {
    int32_t magic;            /* PKV_PLAN_MAGIC once filled */
    int32_t num_seqs;
    int32_t num_tokens;       /* sum of the query rows */
    int32_t num_q_heads;
    int32_t num_kv_heads;
    int32_t head_dim;
    int32_t num_queues;       /* workgroups of the decode launch */
    int32_t num_units;        /* pieces of work (decode and prefill) */
    int32_t num_merges;       /* groups of rows whose pieces are merged */
    int32_t num_partial_rows; /* rows of partial results in the workspace */
    int32_t target_tiles;     /* ideal work per queue, in 16-token tiles */
    int32_t max_q_len;
    int32_t num_prefill_queues; /* workgroups of the prefill launch (0: no chunk rows); with
                                   num_tail_queues, the last of them are tails */
    int32_t num_prefill_units;  /* of num_units; they sit after the decode units */
    int32_t num_wide_merges;  /* merge records listed first: one row each whose pieces are
                                 many (merged by several waves per q head) */
    int32_t num_block_merges; /* records listed next: blocks of chunk rows; the one-row
                                 records with few pieces follow */
    int32_t max_row_merges;   /* most one-row records any plan with these q_lens can have
                                 (the rows with q_len 1) */
    int32_t max_block_merges; /* most row-block records any plan with these q_lens can have;
                                 these two size the merge launch of a call made while its
                                 stream is being captured */
    int32_t window_left;      /* sliding window: a row at position p sees keys p - window_left < j <= p
                                 (0: every key up to p) */
    float logits_soft_cap;    /* scores pass through c * tanh(s / c) before the softmax (0: off) */
    int32_t num_tail_queues;  /* a step with decode rows and chunks: one per decode queue, the
                                 last prefill queues; in the one-launch mixed step decode
                                 workgroup q runs tail q after its decode units (0: none) */
    int64_t off_units;        /* byte offsets inside the workspace */
    int64_t off_queues;
    int64_t off_merges;
    int64_t off_partial_o;
    int64_t off_partial_lse;
    int64_t image_bytes;      /* bytes the host image holds (copied to offset 0) */
    int64_t workspace_bytes;  /* bytes of workspace the plan uses */
} pkv_plan;

#define PKV_PLAN_MAGIC 0x504b5635 /* "PKV5" */

/* Text of a status code; never NULL. */
const char* paged_attn_strerror(int status);

/* PKV_ABI_VERSION of the built library. */
int pkv_abi_version(void);

/*
 * pkv_set_split_event - a timing hook (a measurement aid; no page defines
 * it).  While `event` (a hipEvent_t passed as void*, created by the caller)
 * is not NULL, every attention call (paged_attn_decode,
 * paged_attn_decode_write, paged_attn_mixed, their _csr forms and
 * paged_attn_decode_noalloc) records it on its stream after launching its
 * attention kernel(s) and before launching its merge kernel, so that the
 * attention kernel's time can be read beside the whole call's.  The setting
 * is process-wide and unsynchronised: set it from the thread that makes the
 * calls, and keep it NULL while a stream is being captured.  A record that
 * fails is skipped; the call's work is launched either way.  Returns PKV_OK.
 */
int pkv_set_split_event(void* event);

/*
 * paged_kv_write - write this step's K/V rows into the block pool by slot.
 *
 * For every token t with 0 <= slot_mapping[t] < num_blocks * block_size:
 *     k_cache viewed as [num_blocks * block_size][num_kv_heads][head_dim]
 *     row slot_mapping[t] = convert(k_new row t), and likewise for V.
 * Other slots are not touched; slot < 0 (and a slot past the pool) skips the
 * token.  convert() is a bit copy when new_dtype == cache_dtype, round to
 * nearest even for F32 -> BF16, and for a FP8_E4M3 cache the code nearest
 * to fl32(x / scale) with ties to even, saturating at +-448, NaN -> 0x7F
 * (k_scale for K, v_scale for V).  Two tokens naming one slot is a caller
 * error.
 * ("nanoserve", "One engine step", steps 2-3; "How to design an LLM serving
 * system", "PagedAttention": slot_mapping tells the kernel where each new
 * token's K/V goes.)
 *
 *   k_new, v_new       device, new_dtype, [num_tokens][num_kv_heads][head_dim]
 *   new_dtype          F32 or BF16
 *   new_token_stride   elements between tokens of k_new and v_new
 *                      (>= num_kv_heads * head_dim)
 *   slot_mapping       device int32 [num_tokens]
 *   k_cache, v_cache   device, cache_dtype, the pool
 *   cache_dtype        F32 (from F32), BF16 (from F32 or BF16), FP8_E4M3
 *   head_dim           multiple of 8, num_kv_heads * head_dim <= 65536
 *   k_scale, v_scale   > 0 and finite; used by the FP8 cache only
 * Returns PKV_OK or an error code; num_tokens == 0 launches nothing.
 */
int paged_kv_write(const void* k_new, const void* v_new, int32_t new_dtype, int64_t new_token_stride,
                   const int32_t* slot_mapping, int64_t num_tokens, void* k_cache, void* v_cache,
                   int32_t cache_dtype, int64_t num_blocks, int32_t block_size, int32_t num_kv_heads,
                   int32_t head_dim, float k_scale, float v_scale, void* stream);

/*
 * paged_attn_workspace_size - upper bounds of the device workspace and the
 * host staging image for any plan over at most max_seqs sequences and
 * max_tokens query rows with the given query heads, head_dim and queues.
 * num_queues <= 0 asks for the current device's default (a HIP query).
 * ("How Easy Is It to Start Serving LLMs?", Phase 4 §3: the plan lives in a
 * GPU buffer of fixed size that every layer of the step reuses, so that the
 * step can be captured once and replayed; this bounds that buffer.)
 *   workspace_bytes, host_bytes   out (host); either may be NULL, not both
 * Errors: PKV_ERR_NULL, PKV_ERR_SHAPE (negative sizes, no heads), PKV_ERR_HIP
 * (the device query failed).
 */
int paged_attn_workspace_size(int32_t max_seqs, int32_t max_tokens, int32_t num_q_heads, int32_t head_dim,
                              int32_t num_queues, size_t* workspace_bytes, size_t* host_bytes);

/*
 * Default number of decode workgroups (queues) on the current device: one per
 * compute unit.  A plan with chunk rows adds two prefill queues per queue.
 */
int paged_attn_default_queues(int32_t* num_queues);

/*
 * paged_attn_plan_host - the split-KV planner, host memory only.
 *
 * Each sequence s brings q_lens[s] query rows (q_lens_host == NULL: one row
 * each, a decode batch) and context_lens_host[s] keys.  Work is counted in
 * 16-token tiles; the ideal share per queue is ceil(total tiles /
 * num_queues); sequences are taken longest first (ties: lower index) and cut
 * into pieces, each as long as the least-loaded queue (ties: lower index)
 * can take before it reaches the share, and given to that queue.  Pieces of
 * a sequence that was cut get rows in the partial-result area and one merge
 * record.  Query chunks (q_len > 1) are tiled in blocks of rows first and
 * every (row block, key piece) pair is a unit of its own.
 * ("How Easy Is It to Start Serving LLMs?", Phase 4 §3.)
 *
 * Writes the plan image (units, queue offsets, merge records) into
 * host_image and describes it in *plan; with host_image == NULL only *plan
 * is filled (image_bytes tells the size to provide).  No HIP call is made.
 * Errors: PKV_ERR_SHAPE for a negative length, q_len > context_len,
 * num_q_heads % num_kv_heads != 0 or num_queues < 1; PKV_ERR_WORKSPACE when
 * host_bytes < image_bytes.
 */
int paged_attn_plan_host(const int32_t* context_lens_host, const int32_t* q_lens_host, int32_t num_seqs,
                         int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim, int32_t num_queues,
                         void* host_image, size_t host_bytes, pkv_plan* plan);

/*
 * paged_attn_plan - paged_attn_plan_host (num_queues <= 0: the device
 * default) followed by one asynchronous copy of the image into the first
 * image_bytes of `workspace` on `stream`.  host_staging must stay unchanged
 * until that copy has run (pinned memory makes it asynchronous; pageable
 * memory is copied before the call returns).  Every layer of a step reuses
 * the plan; re-plan when the lengths change.
 * Errors as paged_attn_plan_host, plus PKV_ERR_WORKSPACE when
 * workspace_bytes < plan->workspace_bytes and PKV_ERR_HIP.
 */
int paged_attn_plan(const int32_t* context_lens_host, const int32_t* q_lens_host, int32_t num_seqs,
                    int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim, int32_t num_queues,
                    void* host_staging, size_t host_staging_bytes, void* workspace, size_t workspace_bytes,
                    pkv_plan* plan, void* stream);

/*
 * paged_attn_plan_capacity - paged_attn_plan with the image laid out for a
 * capacity: units, queue offsets, merge records and partial results sit at
 * the workspace offsets of any plan over at most max_seqs sequences and
 * max_tokens query rows (the sizes paged_attn_workspace_size bounds), so
 * every plan made with the same capacity, queues, heads and head_dim uses
 * the same offsets and sizes.  Calls of paged_attn_decode / paged_attn_mixed
 * captured once into a HIP graph with such a plan then stay valid for later
 * plans of the same capacity and the same q_lens made into the same
 * workspace (with the lengths, tables and pools updated in place): the
 * lengths reach the kernels through the workspace, and a merge launch made
 * while its stream is being captured is sized for max_row_merges and
 * max_block_merges records and reads the live counts from the workspace.  The upload copies the whole
 * image (image_bytes) each time.
 * Errors as paged_attn_plan, plus PKV_ERR_SHAPE when num_seqs > max_seqs or
 * the query rows exceed max_tokens.
 */
int paged_attn_plan_capacity(const int32_t* context_lens_host, const int32_t* q_lens_host, int32_t num_seqs,
                             int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim, int32_t num_queues,
                             int32_t max_seqs, int32_t max_tokens, void* host_staging, size_t host_staging_bytes,
                             void* workspace, size_t workspace_bytes, pkv_plan* plan, void* stream);

/*
 * paged_attn_plan_variant - paged_attn_plan_capacity for an attention
 * variant, which the plan carries to every paged_attn_decode(_csr) /
 * paged_attn_mixed(_csr) call made with it:
 *   logits_soft_cap c > 0: every score s = scale * q . k (k_scale folded in)
 *     becomes c * tanh(s / c) before the softmax (logit soft-capping);
 *   window_left W > 0: a row at position p sees the keys j with p - W < j <= p
 *     only (a sliding window of W keys ending at the row), and the planner
 *     skips the keys that no row of a piece can see.
 * ("How Easy Is It to Start Serving LLMs?", Phase 4 §2: soft-capping and
 * sliding windows are among the attention variants one kernel template
 * serves.  Here both are run-time switches of the same kernels: the decode
 * tile loop is built with and without the cap, the window is one more term
 * of each key's validity test, and the prefill tile takes both as uniform
 * branches.)
 * c = 0 and W = 0 give the plain plan.  max_seqs < 0 lays the image out at
 * the plan's own sizes (as paged_attn_plan); max_seqs >= 0 at the capacity
 * (as paged_attn_plan_capacity).  workspace == NULL: host only (as
 * paged_attn_plan_host, host_staging receiving the image, num_queues >= 1).
 * Errors as those calls, plus PKV_ERR_SHAPE for c < 0, a non-finite c or
 * W < 0.
 */
int paged_attn_plan_variant(const int32_t* context_lens_host, const int32_t* q_lens_host, int32_t num_seqs,
                            int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim, int32_t num_queues,
                            float logits_soft_cap, int32_t window_left, int32_t max_seqs, int32_t max_tokens,
                            void* host_staging, size_t host_staging_bytes, void* workspace, size_t workspace_bytes,
                            pkv_plan* plan, void* stream);

/*
 * paged_attn_decode - one query row per sequence (token s is sequence s).
 *
 *   out[s][h][:] = sum_j softmax_j(scale * q[s][h] . K_s[j][g]) V_s[j][g],
 *   g = h / (num_q_heads / num_kv_heads), j over the n = context_lens[s]
 *   keys of sequence s, K_s[j] = k_cache[block_tables[s][j / block_size]]
 *   [j % block_size].  An FP8 cache is read as code * k_scale (K) and
 *   code * v_scale (V).  Arithmetic in fp32; out has q's dtype (round to
 *   nearest even).  A plan from paged_attn_plan_variant applies its
 *   soft-cap to every scaled score and restricts j to its window.
 * ("nanoserve", Triton paged-attention decode bullet: the decode kernel
 * gathers no K/V into a padded copy but walks the block table itself, with
 * a running softmax; "How Easy Is It to Start Serving LLMs?", Phase 4 §1 and
 * §3.)
 *
 *   out, q            device, q_dtype (F32 or BF16), [num_seqs][num_q_heads][head_dim]
 *   q_token_stride    elements between tokens of q (>= num_q_heads * head_dim)
 *   kv_dtype          F32 (q F32), BF16 (q BF16), FP8_E4M3 (q BF16)
 *   head_dim          64 or 128; num_q_heads / num_kv_heads in {1, 2, 4, 8}
 *   plan, workspace   from paged_attn_plan (or _capacity, _variant) with q_lens NULL
 *                     (or all ones)
 * Errors: PKV_ERR_NULL, PKV_ERR_DTYPE, PKV_ERR_UNSUPPORTED, PKV_ERR_SHAPE,
 * PKV_ERR_PLAN (plan made for other shapes or a mixed batch),
 * PKV_ERR_WORKSPACE, PKV_ERR_HIP.
 */
int paged_attn_decode(void* out, const void* q, int32_t q_dtype, int64_t q_token_stride, const void* k_cache,
                      const void* v_cache, int32_t kv_dtype, const int32_t* block_tables,
                      int32_t max_blocks_per_seq, const int32_t* context_lens, int32_t num_seqs,
                      int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim, int64_t num_blocks,
                      int32_t block_size, float scale, float k_scale, float v_scale, const pkv_plan* plan,
                      void* workspace, size_t workspace_bytes, void* stream);

/*
 * paged_attn_mixed - a packed batch: sequence s owns query rows
 * cu_seqlens[s] .. cu_seqlens[s+1]-1 of q and out (num_tokens rows in all);
 * row i of its L rows attends causally to keys 0 .. n - L + i of its
 * n = context_lens[s] keys.  cu_seqlens (device int32 [num_seqs + 1]) must
 * be the exclusive prefix sums of the q_lens the plan was made from; the
 * rows of a sequence whose entries differ come out as NaN.  The rows of
 * one-row sequences run the decode unit (the plan's decode queues), the
 * chunks a tiled unit (its prefill queues) whose QK^T and PV products run on
 * the matrix cores with P rounded to bf16; then one merge of cut pieces.
 * With bf16 K/V on pages of a multiple of 16 tokens and 2 or 4 q heads per
 * kv head, both kinds of unit run in one launch (decode and prefill
 * workgroups side by side on every compute unit); otherwise the decode and
 * the prefill units are two launches.  So one call is one or two attention
 * launches followed by the merge launch.
 * Same arguments and errors as paged_attn_decode, with the plan made from
 * A step whose chunks all hold at most 16 (row, q head) pairs per kv head
 * (at most 16 / G rows: a speculative verify step) is planned as decode rows
 * are, each unit holding a sequence's rows and every kv head, and runs one
 * few-row launch (matrix-core tiles, one wave per kv head) and the merge.
 * Same arguments and errors as paged_attn_decode, with the plan made from
 * the same q_lens, plus: PKV_ERR_NULL for a NULL cu_seqlens with rows to
 * compute, PKV_ERR_UNSUPPORTED when the plan has chunk rows
 * and q is not bf16 (K/V bf16 or fp8; decode-only plans take every dtype
 * paged_attn_decode takes), PKV_ERR_SHAPE when chunk rows meet a cache not
 * aligned to 8 elements.  A block id outside the pool turns the rows of
 * every unit that reads it into NaN (a unit holds up to 128 / G rows of one
 * chunk) and is never dereferenced.
 * ("nanoserve", "Packed batches" and chunked-prefill bullets, and the
 * benchmark note on splitting each mixed step into decode rows and prefill
 * chunks; "How to design an LLM serving system", "Latency and scaling
 * knobs": chunked prefill and speculative verify.)
 */
int paged_attn_mixed(void* out, const void* q, int32_t q_dtype, int64_t q_token_stride, const void* k_cache,
                     const void* v_cache, int32_t kv_dtype, const int32_t* block_tables,
                     int32_t max_blocks_per_seq, const int32_t* cu_seqlens, const int32_t* context_lens,
                     int32_t num_seqs, int32_t num_tokens, int32_t num_q_heads, int32_t num_kv_heads,
                     int32_t head_dim, int64_t num_blocks, int32_t block_size, float scale, float k_scale,
                     float v_scale, const pkv_plan* plan, void* workspace, size_t workspace_bytes,
                     void* stream);

/*
 * paged_attn_decode_write - a decode step's write and attention in one call:
 * the same result as paged_kv_write(k_new, v_new, new_dtype,
 * new_token_stride, slot_mapping, num_seqs, k_cache, v_cache, kv_dtype,
 * num_blocks, block_size, num_kv_heads, head_dim, k_scale, v_scale, stream)
 * followed by paged_attn_decode(...) with the other arguments, where token s
 * of k_new / v_new is the new key and value of sequence s: slot_mapping[s]
 * is the slot of its key context_lens[s] - 1, or < 0 (nothing written for
 * it).  ("nanoserve", "One engine step", step 3: each layer writes this
 * step's K/V, then attends; "How to design an LLM serving system",
 * "PagedAttention": slot_mapping names each new token's slot.)
 *
 * With BF16 q, tokens and cache, pages of a multiple of 16 tokens,
 * num_kv_heads * head_dim <= 4096 and k_new, v_new and their token stride
 * 16-byte aligned, the decode launch writes the tokens itself:
 * the workgroup whose keys end at a sequence's key context_lens[s] - 1 reads
 * that key from k_new / v_new rather than from the pool, and copies the
 * token into its slot once done.  Then a sequence whose slot_mapping entry
 * is >= 0 but not that key's slot (or whose length differs from the plan's)
 * gets a NaN row and nothing is written for it; no other sequence of the
 * batch may read these slots (a page shared by two sequences is never the
 * one that receives a new token).  Otherwise the write kernel runs first,
 * then the decode call, exactly as the two calls.
 *
 *   k_new, v_new       device, new_dtype (F32 or BF16), [num_seqs][num_kv_heads][head_dim]
 *   slot_mapping       device int32 [num_seqs]
 *   other arguments    as paged_attn_decode (k_cache, v_cache writable here)
 * Errors: those of paged_kv_write and of paged_attn_decode, every one of
 * them checked before anything is launched.
 */
int paged_attn_decode_write(void* out, const void* q, int32_t q_dtype, int64_t q_token_stride, const void* k_new,
                            const void* v_new, int32_t new_dtype, int64_t new_token_stride,
                            const int32_t* slot_mapping, void* k_cache, void* v_cache, int32_t kv_dtype,
                            const int32_t* block_tables, int32_t max_blocks_per_seq, const int32_t* context_lens,
                            int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                            int64_t num_blocks, int32_t block_size, float scale, float k_scale, float v_scale,
                            const pkv_plan* plan, void* workspace, size_t workspace_bytes, void* stream);

/*
 * paged_attn_decode_noalloc - paged_attn_decode for callers that cannot
 * allocate device memory (code being captured into a HIP graph, serving loops
 * that must not allocate, harnesses that forbid it): the workspace is the
 * library's own device array of 32 MiB (one per device, held until the
 * process ends) instead of a caller buffer, and the call allocates nothing.
 *
 *   plan, plan_image_host   a decode plan (q_lens NULL or all ones) and its
 *                           image, from paged_attn_plan_host or the host-only
 *                           form of paged_attn_plan_variant; the call copies
 *                           the image into the array on `stream` (pinned
 *                           host memory makes the copy asynchronous; it must
 *                           stay unchanged until the copy has run)
 * Every other argument as for paged_attn_decode.  Nothing in the array needs
 * to start at zero: the copy writes the plan, and every partial result is
 * written before the merge reads it.
 * Errors as paged_attn_decode, plus PKV_ERR_WORKSPACE when the plan needs
 * more than the 32 MiB array (plan->workspace_bytes; checked before any
 * device work) and PKV_ERR_NULL for a NULL image with rows to compute.
 * Calls on one device share its array: calls that overlap in time on one
 * device (other streams, other threads) race and must be ordered by the
 * caller, like calls that share a workspace.
 */
int paged_attn_decode_noalloc(void* out, const void* q, int32_t q_dtype, int64_t q_token_stride,
                              const void* k_cache, const void* v_cache, int32_t kv_dtype,
                              const int32_t* block_tables, int32_t max_blocks_per_seq, const int32_t* context_lens,
                              int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                              int64_t num_blocks, int32_t block_size, float scale, float k_scale, float v_scale,
                              const pkv_plan* plan, const void* plan_image_host, void* stream);

/*
 * paged_attn_decode_csr / paged_attn_mixed_csr - paged_attn_decode and
 * paged_attn_mixed with the page table in CSR form ("How Easy Is It to Start
 * Serving LLMs?", Phase 4 §1: kv_indptr / kv_indices): sequence s reads the
 * page of its logical block b from kv_indices[kv_indptr[s] + b], for
 * b < kv_indptr[s+1] - kv_indptr[s]; a row may hold unused entries after its
 * last page, and rows of different sequences may name the same pages.
 *   kv_indptr   int32 [num_seqs + 1], device, non-decreasing, kv_indptr[0] >= 0
 *   kv_indices  int32 [kv_indptr[num_seqs]], device (non-NULL)
 * Every other argument, the plan and the workspace as for the dense forms.
 * The offsets are read on the device and not checked there: kv_indptr must
 * stay within kv_indices (a caller error otherwise, like a short dense row).
 * A key whose logical block is past its row, or whose entry is outside the
 * pool, makes its sequence's rows NaN, as with dense tables.
 * Errors as paged_attn_decode / paged_attn_mixed (PKV_ERR_NULL for a NULL
 * kv_indptr or kv_indices with rows to compute).
 */
int paged_attn_decode_csr(void* out, const void* q, int32_t q_dtype, int64_t q_token_stride, const void* k_cache,
                          const void* v_cache, int32_t kv_dtype, const int32_t* kv_indptr,
                          const int32_t* kv_indices, const int32_t* context_lens, int32_t num_seqs,
                          int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim, int64_t num_blocks,
                          int32_t block_size, float scale, float k_scale, float v_scale, const pkv_plan* plan,
                          void* workspace, size_t workspace_bytes, void* stream);

int paged_attn_mixed_csr(void* out, const void* q, int32_t q_dtype, int64_t q_token_stride, const void* k_cache,
                         const void* v_cache, int32_t kv_dtype, const int32_t* kv_indptr, const int32_t* kv_indices,
                         const int32_t* cu_seqlens, const int32_t* context_lens, int32_t num_seqs,
                         int32_t num_tokens, int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                         int64_t num_blocks, int32_t block_size, float scale, float k_scale, float v_scale,
                         const pkv_plan* plan, void* workspace, size_t workspace_bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* PKV_H_ */
