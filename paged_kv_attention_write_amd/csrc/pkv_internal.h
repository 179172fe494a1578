// Host-side structures shared by the planner, the C-ABI layer and the kernel
// launchers.  The device reads the same records from the workspace.
#pragma once

#include <cstddef>
#include <cstdint>

#include "pkv.h"

namespace pkv {

// Work is counted in tiles of this many keys; piece boundaries inside a
// sequence fall on tile boundaries.
constexpr int kTileTokens = 16;
// A prefill unit covers this many (row, q head) pairs of one kv head: the
// rows of a chunk are taken in blocks of kPrefillQRows / G rows (G = q heads
// per kv head), each block times each kv head times each key piece.
constexpr int kPrefillQRows = 128;
// Key pieces of one prefill row block: at most this many, each at least
// kPrefillPieceMin keys (the last may be shorter).  Within those limits a row
// block gets pieces in proportion to its share of the chunks' work.
constexpr int kPrefillMaxPieces = 8;
constexpr int kPrefillPieceMin = 512;
// Prefill queues per decode queue: a step of chunks alone runs two prefill
// workgroups per CU.  A step with decode rows as well runs one: the launch
// that holds both halves fits one decode and one prefill workgroup on a CU,
// and with a second prefill workgroup per CU half of the prefill queues
// would wait for the first to finish (measured: the 63-row + 512-row-chunk
// step 96.9 -> 84.5 us with one).
constexpr int kPrefillQueuesPerQueue = 2;
constexpr int kPrefillQueuesPerQueueMixed = 1;
// Beside those, a step with decode rows and chunks gives each decode queue a
// tail queue of prefill pieces, run by the decode workgroup once its decode
// units are done.  The tails are sized by the time a decode queue's work
// takes, counted in prefill flops: this many per byte of its K/V tiles (one
// launch of the 63-row + 512-row-chunk step on MI355X: decode workgroups
// ended at about 49 us of 18 tiles each, prefill workgroups sharing their CUs
// at about 64 us of 75.5 MFLOP each).
constexpr int64_t kMixedFlopsPerDecodeByte = 42;

// A step whose longest chunk has at most this many (row, q head) pairs per
// kv head (a speculative verify step: a few rows per sequence) is planned as
// decode rows are: every sequence, whatever its row count, is cut by key
// tiles over the decode queues, and a unit holds all its rows and every kv
// head, so that a workgroup streams whole key rows of the pool.
constexpr int kFewRowPairs = 16;

// Decode queue loads count each piece placed on a queue as this many tiles
// more than its keys: the set-up of a unit (its first page lookups and
// loads, its flush) costs about one tile's time, so a queue that runs two
// pieces is given about a tile less.
constexpr int kDecodeUnitCost = 1;
// Placements of the decode requests at most (the share raised after each
// that overflows it).
constexpr int kDecodeShareAttempts = 4;

// Alignment of the sections of the workspace.
// A one-row merge record with at least this many pieces is "wide": its
// merge gives every q head a workgroup whose waves split the pieces.
constexpr int kWideMergeParts = 8;

constexpr size_t kAlign = 256;

// kind == kUnitDecode: a decode unit (every kv head; one row, or the few
// rows of a sequence in a few-row step).  kind >= 1: a prefill unit of kv
// head kind - 1.
enum UnitKind : int32_t { kUnitDecode = 0, kUnitPrefill = 1 };

// One piece of work: query rows [row0, row0 + nrows) of sequence `seq` (rows
// are packed token indices) against keys [kv_begin, kv_end).  Row r of the
// unit sits at position pos0 + r.  prow >= 0: write the normalised partial
// result of row r to partial row prow + r; prow < 0: write the output.
struct Unit {
    int32_t seq;
    int32_t kv_begin;
    int32_t kv_end;
    int32_t row0;
    int32_t nrows;
    int32_t pos0;
    int32_t prow;
    int32_t kind;
};
static_assert(sizeof(Unit) == 32, "unit record is 32 bytes");

// Rows [row0, row0 + nrows) whose `parts` partial results sit at partial
// rows prow0 + c * nrows + r, c = 0 .. parts-1, in key order.
struct Merge {
    int32_t row0;
    int32_t nrows;
    int32_t prow0;
    int32_t parts;
};
static_assert(sizeof(Merge) == 16, "merge record is 16 bytes");

inline size_t align_up(size_t x, size_t a = kAlign) { return (x + a - 1) / a * a; }

// Element counts of the sections of a plan image: units, int32 entries of
// the queue-offset section (num_queues + prefill queues + 1 offsets, then
// kPlanCounts live counts at a fixed index), merge records and partial rows.
struct PlanSections {
    int64_t units, queue_ints, merges, prows;
};

// The live counts that follow the queue offsets (index plan_counts_index):
// merge records, wide records, row-block records.
constexpr int kPlanCounts = 3;
inline int64_t plan_counts_index(int32_t num_queues) {
    return static_cast<int64_t>(1 + kPrefillQueuesPerQueue) * num_queues + 1;
}

// Section sizes that hold any plan over at most max_seqs sequences and
// max_tokens query rows.
PlanSections plan_capacity(int64_t max_seqs, int64_t max_tokens, int32_t num_q_heads, int32_t num_kv_heads,
                           int32_t num_queues);

// Planner (pkv_plan.cpp).  Pure host code.  cap_seqs >= 0 lays the image
// out at the offsets of plan_capacity(cap_seqs, cap_tokens, ...) instead of
// the plan's own sizes.  soft_cap and window are recorded in the plan; the
// window also trims the key ranges.
int plan_host(const int32_t* ctx, const int32_t* q_lens, int32_t num_seqs, int32_t num_q_heads,
              int32_t num_kv_heads, int32_t head_dim, int32_t num_queues, void* host_image,
              size_t host_bytes, pkv_plan* plan, int32_t cap_seqs = -1, int32_t cap_tokens = -1,
              float soft_cap = 0.f, int32_t window = 0);

// Size of the device scratch array of the entry point that allocates nothing
// (one per device, held until the process ends), and its device address on
// the current device (pkv_noalloc.hip; asked of the runtime once per device).
constexpr size_t kNoallocScratchBytes = size_t(32) << 20;
int noalloc_scratch(void** ptr);

// Upper bounds used by paged_attn_workspace_size.
void plan_bounds(int32_t max_seqs, int32_t max_tokens, int32_t num_q_heads, int32_t head_dim,
                 int32_t num_queues, size_t* workspace_bytes, size_t* host_bytes);

}  // namespace pkv
