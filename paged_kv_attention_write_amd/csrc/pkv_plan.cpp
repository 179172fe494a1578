// Split-KV planner: host code, once per step, reused by every layer.
//
// "How Easy Is It to Start Serving LLMs?", Phase 4 §3 (load balancing): the
// ideal work per processor is the total over the processor count; requests
// are taken longest first and cut into pieces no longer than that share;
// every piece goes to the least-loaded queue.  Here work is counted in
// 16-token tiles, the share is rounded up to whole tiles, and each piece is
// cut to what the least-loaded queue can still take before it reaches the
// share, so queues end within one tile of each other and a request is cut
// only where a queue fills up (at most queues + requests pieces in all).
// Every piece also counts one tile of set-up in its queue's load (and the
// share includes one per queue), so a queue running two pieces gets about
// one tile less; when the cuts make more set-up than the share leaves room
// for, the share is raised to cover it and the requests are placed again.
//
// Query chunks (more than one new row) are split into blocks of rows, one
// unit per (row block, kv head, key piece), and run over a second set of
// queues: the key range of a row block is cut into as many pieces as its
// share of the chunks' work is of those queues, so that the units fill them
// about once; a unit's cost is its matrix-core flops, and the units are
// placed largest first, each whole on the least-loaded prefill queue.  In a
// step with decode rows as well, every decode queue also gets a tail queue
// of prefill pieces, sized by the time its decode work takes, which its
// workgroup runs after its decode units; the row blocks are then cut by
// flops into pieces that fill a prefill queue and pieces about a tail's
// size.
//
// With a sliding window of W keys a row at position p sees keys
// p - W < j <= p only: the ranges above then start at the first tile that
// holds a key some row of the piece can see, and the work counts only the
// visible (row, key) pairs.

#include <algorithm>
#include <cmath>
#include <cstring>
#include <queue>
#include <vector>

#include "pkv_internal.h"

namespace pkv {
namespace {

struct QueueHeap {
    // (load, index) min-heap: the lightest queue, ties to the lowest index.
    using Item = std::pair<int64_t, int32_t>;
    std::priority_queue<Item, std::vector<Item>, std::greater<Item>> heap;
    explicit QueueHeap(int32_t n) {
        std::vector<Item> init;
        init.reserve(n);
        for (int32_t i = 0; i < n; ++i) init.emplace_back(0, i);
        heap = decltype(heap)(std::greater<Item>(), std::move(init));
    }
    explicit QueueHeap(const std::vector<int64_t>& loads) {
        std::vector<Item> init;
        init.reserve(loads.size());
        for (size_t i = 0; i < loads.size(); ++i) init.emplace_back(loads[i], static_cast<int32_t>(i));
        heap = decltype(heap)(std::greater<Item>(), std::move(init));
    }
    Item pop() {
        Item it = heap.top();
        heap.pop();
        return it;
    }
    void push(int64_t load, int32_t q) { heap.emplace(load, q); }
};

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

// A prefill unit and its cost; equal costs keep their creation order (the
// sort is stable).
struct PrefillPiece {
    Unit unit;
    int64_t cost;  // flops of the unit's visible (row, key) pairs
};

}  // namespace

PlanSections plan_capacity(int64_t max_seqs, int64_t max_tokens, int32_t num_q_heads, int32_t num_kv_heads,
                           int32_t num_queues) {
    const int64_t seqs = std::max<int64_t>(max_seqs, 0);
    const int64_t toks = std::max<int64_t>(max_tokens, 0);
    const int64_t nq = std::max<int32_t>(num_queues, 1);
    // decode pieces: at most queues + requests (lazy fill).  Prefill row
    // blocks: blocks of kPrefillQRows / G >= kPrefillQRows / num_q_heads
    // rows, at most one partial block per sequence; a unit per kv head and
    // piece.  A merge record per decode row or row block.
    const int64_t hq = std::max<int32_t>(num_q_heads, 1);
    const int64_t hkv = std::min<int64_t>(hq, std::max<int32_t>(num_kv_heads, 1));
    const int64_t rmin = std::max<int64_t>(1, kPrefillQRows / hq);
    const int64_t blocks = toks / rmin + seqs;
    PlanSections c;
    c.units = nq + seqs + blocks * kPrefillMaxPieces * hkv;
    c.queue_ints = plan_counts_index(static_cast<int32_t>(nq)) + kPlanCounts;
    c.merges = seqs + blocks;
    // (a few-row step cuts each sequence by the decode rule: at most
    // queues - 1 cuts, each adding at most kFewRowPairs rows)
    c.prows = nq + seqs + toks * kPrefillMaxPieces + nq * kFewRowPairs;
    return c;
}

int plan_host(const int32_t* ctx, const int32_t* q_lens, int32_t num_seqs, int32_t num_q_heads,
              int32_t num_kv_heads, int32_t head_dim, int32_t num_queues, void* host_image,
              size_t host_bytes, pkv_plan* plan, int32_t cap_seqs, int32_t cap_tokens, float soft_cap,
              int32_t window) {
    if (plan == nullptr || (num_seqs > 0 && ctx == nullptr)) return PKV_ERR_NULL;
    std::memset(plan, 0, sizeof(*plan));
    if (num_seqs < 0 || num_queues < 1 || num_q_heads < 1 || num_kv_heads < 1 || head_dim < 1 ||
        num_q_heads % num_kv_heads != 0)
        return PKV_ERR_SHAPE;
    if (!(soft_cap >= 0.f) || !std::isfinite(soft_cap) || window < 0) return PKV_ERR_SHAPE;
    if (cap_seqs >= 0 && (num_seqs > cap_seqs || cap_tokens < 0)) return PKV_ERR_SHAPE;

    // Validate lengths and collect packed row offsets.
    std::vector<int32_t> row0(static_cast<size_t>(num_seqs) + 1, 0);
    int64_t rows = 0;
    int32_t max_q = 0;
    for (int32_t s = 0; s < num_seqs; ++s) {
        const int32_t n = ctx[s];
        const int32_t L = q_lens ? q_lens[s] : 1;
        if (n < 0 || L < 0 || L > n) return PKV_ERR_SHAPE;
        row0[s] = static_cast<int32_t>(rows);
        rows += L;
        if (rows > INT32_MAX) return PKV_ERR_SHAPE;
        max_q = std::max(max_q, L);
    }
    row0[num_seqs] = static_cast<int32_t>(rows);

    const int64_t hd = static_cast<int64_t>(num_q_heads) * head_dim;
    const int32_t group = num_q_heads / num_kv_heads;
    const int32_t block_rows = std::max(1, kPrefillQRows / group);

    // first key a row at position p sees, and the first key of the tile
    // holding it (the start of a range over rows from position p on)
    auto first_key = [window](int64_t p) { return window > 0 ? std::max<int64_t>(0, p - window + 1) : 0; };
    auto range_start = [&](int64_t p) { return first_key(p) / kTileTokens * kTileTokens; };
    // visible (row, key) pairs of rows [r0, r1) of a chunk of L rows over n
    // keys, against keys [kb, ke)
    auto pairs_of = [&](int32_t n, int32_t L, int32_t r0, int32_t r1, int64_t kb, int64_t ke) {
        int64_t pairs = 0;
        for (int32_t r = r0; r < r1; ++r) {
            const int64_t last = static_cast<int64_t>(n) - L + r;  // position of row r
            pairs += std::max<int64_t>(0, std::min<int64_t>(ke - 1, last) - std::max<int64_t>(kb, first_key(last)) + 1);
        }
        return pairs;
    };
    // flops of one kv head: 2 (q.k) + 2 (p.v) per pair, q head and dimension
    const int64_t flops_per_pair = 4LL * group * head_dim;
    // a few-row step: every sequence is cut and placed as a decode row is
    const bool few = max_q > 1 && static_cast<int64_t>(max_q) * group <= kFewRowPairs;
    // rows a sequence sends through the decode queues
    auto decode_rows = [&](int32_t L) { return (L == 1 || (few && L > 1)) ? L : 0; };

    // Total work and the share per queue.
    int64_t decode_tiles = 0;
    int64_t prefill_flops = 0;
    for (int32_t s = 0; s < num_seqs; ++s) {
        const int32_t n = ctx[s];
        const int32_t L = q_lens ? q_lens[s] : 1;
        if (decode_rows(L) > 0) decode_tiles += ceil_div(n - range_start(n - L), kTileTokens);
        else if (L > 1) prefill_flops += pairs_of(n, L, 0, L, 0, n) * flops_per_pair * num_kv_heads;
    }
    // Decode rows and prefill chunks are balanced each on their own queues
    // (whether they then run in one launch or two).
    const int32_t prefill_queues =
        prefill_flops > 0 ? (decode_tiles > 0 ? kPrefillQueuesPerQueueMixed : kPrefillQueuesPerQueue) * num_queues
                          : 0;

    // merge records with their kind: 0 wide (one decode row, many pieces),
    // 1 a block of chunk rows (whatever its row count: a chunk's last block
    // may hold a single row), 2 the other decode rows
    std::vector<std::pair<int32_t, Merge>> merges;
    int64_t partial_rows = 0;

    // Decode requests, longest first, cut to fill the lightest queue.
    std::vector<int32_t> order;
    for (int32_t s = 0; s < num_seqs; ++s)
        if (decode_rows(q_lens ? q_lens[s] : 1) > 0 && ctx[s] > 0) order.push_back(s);
    auto rows_of = [&](int32_t s) { return q_lens ? q_lens[s] : 1; };
    // keys the rows of a request read: from the tile of its first row's
    // first visible key on
    auto decode_keys = [&](int32_t s) { return ctx[s] - range_start(ctx[s] - rows_of(s)); };
    std::stable_sort(order.begin(), order.end(),
                     [&](int32_t a, int32_t b) { return decode_keys(a) > decode_keys(b); });

    // The decode share: the decode tiles and a unit's set-up per queue, over
    // the queues.  Cutting makes more units than queues, and when their
    // set-up no longer fits the share (a lightest queue with no room while a
    // request still has tiles) the share is raised to cover the units of
    // that cut and the requests are placed again: taking the rest on that
    // queue would leave it up to twice as long as the others.
    int64_t target =
        decode_tiles > 0 ? ceil_div(decode_tiles + static_cast<int64_t>(kDecodeUnitCost) * num_queues, num_queues) : 0;
    std::vector<std::vector<Unit>> queues(static_cast<size_t>(num_queues));
    const size_t merges0 = merges.size();
    const int64_t partial_rows0 = partial_rows;
    std::vector<std::pair<int32_t, size_t>> placed;  // (queue, index) of the pieces of one request
    for (int attempt = 0;; ++attempt) {
        for (auto& q : queues) q.clear();
        merges.resize(merges0);
        partial_rows = partial_rows0;
        QueueHeap heap(num_queues);
        int64_t units = 0;
        bool over = false;
        for (int32_t s : order) {
            const int32_t n = ctx[s];
            const int32_t L = rows_of(s);
            const int64_t start = range_start(n - L);
            int64_t remaining = ceil_div(n - start, kTileTokens);
            int64_t first = 0;
            placed.clear();
            while (remaining > 0) {
                auto [load, q] = heap.pop();
                // what the lightest queue can still take after a unit's
                // set-up; with no room left anywhere it takes the rest (and
                // the share is raised for the next attempt)
                const int64_t room = target - load - kDecodeUnitCost;
                over |= room <= 0;
                const int64_t take = room > 0 ? std::min(remaining, room) : remaining;
                const int32_t kb = static_cast<int32_t>(start + first * kTileTokens);
                const int32_t ke = static_cast<int32_t>(std::min<int64_t>(n, start + (first + take) * kTileTokens));
                queues[q].push_back(Unit{s, kb, ke, row0[s], L, n - L, -1, kUnitDecode});
                placed.emplace_back(q, queues[q].size() - 1);
                heap.push(load + take + kDecodeUnitCost, q);
                remaining -= take;
                first += take;
                ++units;
            }
            if (placed.size() > 1) {
                // piece c's rows at prow0 + c L; a request of several rows
                // merges as a row block
                const int32_t prow0 = static_cast<int32_t>(partial_rows);
                for (size_t c = 0; c < placed.size(); ++c)
                    queues[placed[c].first][placed[c].second].prow = prow0 + static_cast<int32_t>(c) * L;
                const int32_t parts = static_cast<int32_t>(placed.size());
                merges.emplace_back(L > 1 ? 1 : parts >= kWideMergeParts ? 0 : 2, Merge{row0[s], L, prow0, parts});
                partial_rows += static_cast<int64_t>(placed.size()) * L;
            }
        }
        if (!over || kDecodeUnitCost == 0 || attempt >= kDecodeShareAttempts - 1) break;
        target = std::max(target + 1,
                          ceil_div(decode_tiles + static_cast<int64_t>(kDecodeUnitCost) * units, num_queues));
    }

    // A step with decode rows and chunks: each decode queue's workgroup, once
    // its decode units are done, runs a tail queue of prefill pieces.  In
    // prefill flops, a decode queue's work counts kMixedFlopsPerDecodeByte per
    // byte of its tiles' K and V (bf16) and every prefill piece one decode
    // tile of set-up; T is the load at which the prefill queues (one piece of
    // T - set-up each) and the tails (T - decode work - set-up, when that is
    // positive) hold all the prefill work.  The chunk row blocks are then cut
    // into pieces of T - set-up and a remainder in pieces of about a tail's
    // size, and every piece is placed, largest first, on the least-loaded of
    // the prefill and tail queues (a tail starting at its decode work).
    const int32_t tail_queues = decode_tiles > 0 && prefill_flops > 0 ? num_queues : 0;
    const int64_t tile_flops = kMixedFlopsPerDecodeByte * 2LL * 2LL * kTileTokens * num_kv_heads * head_dim;
    std::vector<int64_t> tail_load0(static_cast<size_t>(tail_queues), 0);
    double main_cap = 0.0, tail_cap = 0.0;  // flops of a prefill queue's piece and of a typical tail piece
    if (tail_queues > 0) {
        for (int32_t q = 0; q < num_queues; ++q) {
            int64_t tiles = 0;
            for (const Unit& u : queues[q]) tiles += ceil_div(u.kv_end - u.kv_begin, kTileTokens) + kDecodeUnitCost;
            tail_load0[q] = tiles * tile_flops;
        }
        const double setup = static_cast<double>(tile_flops);
        auto held = [&](double T) {
            double h = static_cast<double>(prefill_queues) * (T - setup);
            for (int64_t e : tail_load0) h += std::max(0.0, T - static_cast<double>(e) - setup);
            return h;
        };
        double lo = setup, hi = setup + static_cast<double>(prefill_flops) / prefill_queues;
        for (int it = 0; it < 64; ++it) {
            const double mid = 0.5 * (lo + hi);
            (held(mid) < static_cast<double>(prefill_flops) ? lo : hi) = mid;
        }
        const double T = hi;
        main_cap = T - setup;
        int32_t open = 0;
        double room = 0.0;
        for (int64_t e : tail_load0) {
            const double r = T - static_cast<double>(e) - setup;
            if (r > 0.0) {
                room += r;
                ++open;
            }
        }
        tail_cap = open > 0 ? room / open : 0.0;
    }

    // Prefill units: row blocks x kv heads x key pieces of every chunk.
    std::vector<PrefillPiece> prefill;
    for (int32_t s = 0; s < num_seqs; ++s) {
        const int32_t n = ctx[s];
        const int32_t L = q_lens ? q_lens[s] : 1;
        if (L <= 1 || decode_rows(L) > 0) continue;
        for (int32_t r0 = 0; r0 < L; r0 += block_rows) {
            const int32_t r1 = std::min(L, r0 + block_rows);
            const int32_t nr = r1 - r0;
            const int32_t extent = n - L + r1;  // keys the last row of the block sees
            const int64_t start = range_start(n - L + r0);  // the first row's first tile
            const int64_t span = extent - start;
            // pieces per kv head: the row block's share of the prefill queues
            // (its work over the chunks' total, rounded to the nearest
            // count), so that the chunk units fill the prefill queues about
            // once; at least one, at most kPrefillMaxPieces, none shorter than
            // kPrefillPieceMin keys.  A row block that fills under half a
            // unit's pairs (a few speculative rows, say) costs little to cut,
            // having few partial rows, so it is cut 3x finer and the
            // least-loaded placement packs the pieces evenly.
            const int64_t block_flops = pairs_of(n, L, r0, r1, start, extent) * flops_per_pair * num_kv_heads;
            const int64_t fine = static_cast<int64_t>(nr) * group * 2 < kPrefillQRows ? 3 : 1;
            const int64_t share = static_cast<int64_t>(std::llround(
                static_cast<double>(fine * prefill_queues) * static_cast<double>(block_flops) /
                (static_cast<double>(prefill_flops) * num_kv_heads)));
            const int64_t most = std::min<int64_t>(kPrefillMaxPieces, std::max<int64_t>(1, span / kPrefillPieceMin));
            const int64_t ask = std::min<int64_t>(most, std::max<int64_t>(1, share));
            const int64_t piece = ceil_div(ceil_div(span, ask), kTileTokens) * kTileTokens;
            // piece boundaries: key starts of the pieces and the extent
            std::vector<int64_t> cuts;
            for (int64_t kb = start; kb < extent; kb += piece) cuts.push_back(kb);
            cuts.push_back(extent);
            if (tail_queues > 0 && main_cap > 0.0) {
                // with tails: pieces of main_cap flops (the remainder of a
                // block spread over them when it is under half a tail piece),
                // then the remainder in pieces of about tail_cap (at most
                // kPrefillMaxPieces in all); each cut on the first 16-key tile
                // boundary that reaches its share
                const double u = static_cast<double>(block_flops) / num_kv_heads;
                // (at most `most` of them, as without tails)
                int64_t m = std::min<int64_t>(static_cast<int64_t>(u / main_cap), most);
                double r = u - static_cast<double>(m) * main_cap;
                int64_t k = 0;
                if (m == 0) {
                    k = 1;
                } else if (r < 0.5 * tail_cap || tail_cap <= 0.0) {
                    r = 0.0;
                } else {
                    k = std::max<int64_t>(1, std::llround(r / tail_cap));
                }
                k = std::min<int64_t>(k, std::max<int64_t>(kPrefillMaxPieces - m, 1));
                m = std::min<int64_t>(m, kPrefillMaxPieces - k);
                std::vector<double> at;  // cumulative flops at each inner cut
                const double mainc = m > 0 ? (u - r) / static_cast<double>(m) : 0.0;
                for (int64_t c = 1; c <= m; ++c) at.push_back(mainc * static_cast<double>(c));
                for (int64_t c = 1; c < k; ++c) at.push_back(u - r + r * static_cast<double>(c) / static_cast<double>(k));
                if (!at.empty() && at.back() >= u - 0.5) at.pop_back();  // no empty last piece
                cuts.assign(1, start);
                const int64_t tiles = ceil_div(span, kTileTokens);
                for (double want : at) {
                    // the smallest tile count whose keys reach `want` flops
                    int64_t lo = 1, hi = tiles;
                    while (lo < hi) {
                        const int64_t mid = (lo + hi) / 2;
                        const double got = static_cast<double>(
                            pairs_of(n, L, r0, r1, start, std::min<int64_t>(extent, start + mid * kTileTokens)) *
                            flops_per_pair);
                        if (got >= want) hi = mid;
                        else lo = mid + 1;
                    }
                    const int64_t kb = std::min<int64_t>(extent, start + lo * kTileTokens);
                    if (kb > cuts.back() && kb < extent) cuts.push_back(kb);
                }
                cuts.push_back(extent);
            }
            const int32_t parts = static_cast<int32_t>(cuts.size()) - 1;
            const int32_t prow0 = parts > 1 ? static_cast<int32_t>(partial_rows) : -1;
            if (parts > 1) {
                merges.emplace_back(1, Merge{row0[s] + r0, nr, prow0, parts});
                partial_rows += static_cast<int64_t>(parts) * nr;
            }
            for (int32_t c = 0; c < parts; ++c) {
                const int64_t kb = cuts[c];
                const int64_t ke = cuts[c + 1];
                const int64_t cost = pairs_of(n, L, r0, r1, kb, ke) * flops_per_pair;
                for (int32_t h = 0; h < num_kv_heads; ++h) {
                    const Unit u{s, static_cast<int32_t>(kb), static_cast<int32_t>(ke), row0[s] + r0, nr,
                                 n - L + r0, parts > 1 ? prow0 + c * nr : -1, kUnitPrefill + h};
                    prefill.push_back(PrefillPiece{u, cost});
                }
            }
        }
    }

    // Prefill units, largest first, each whole on the least-loaded prefill queue.
    // With tails: over the prefill queues, then the tails (queue
    // prefill_queues + q: decode queue q's), each piece adding its set-up.
    std::vector<std::vector<Unit>> pqueues(static_cast<size_t>(prefill_queues + tail_queues));
    if (prefill_queues > 0) {
        std::vector<int64_t> load0(static_cast<size_t>(prefill_queues + tail_queues), 0);
        for (int32_t q = 0; q < tail_queues; ++q) load0[prefill_queues + q] = tail_load0[q];
        QueueHeap pheap(load0);
        const int64_t setup = tail_queues > 0 ? tile_flops : 0;
        std::stable_sort(prefill.begin(), prefill.end(), [](const PrefillPiece& a, const PrefillPiece& b) {
            return a.cost > b.cost;
        });
        for (const auto& p : prefill) {
            auto [load, q] = pheap.pop();
            pqueues[q].push_back(p.unit);
            pheap.push(load + p.cost + setup, q);
        }
    }

    // merge records: wide ones, then row blocks, then the other one-row
    // records, each kind in its order
    std::stable_sort(merges.begin(), merges.end(),
                     [](const auto& x, const auto& y) { return x.first < y.first; });
    int32_t num_wide = 0, num_block = 0;
    for (const auto& m : merges) {
        num_wide += m.first == 0 ? 1 : 0;
        num_block += m.first == 1 ? 1 : 0;
    }
    // records any plan with these q_lens can have: one per decode row, one
    // per block of chunk rows
    int64_t row_slots = 0, block_slots = 0;
    for (int32_t s = 0; s < num_seqs; ++s) {
        const int32_t L = q_lens ? q_lens[s] : 1;
        if (L == 1) ++row_slots;
        if (L > 1) block_slots += ceil_div(L, block_rows);
    }

    int64_t num_units = 0;
    for (const auto& q : queues) num_units += static_cast<int64_t>(q.size());
    const int64_t num_prefill_units = static_cast<int64_t>(prefill.size());
    num_units += num_prefill_units;
    if (num_units > INT32_MAX || partial_rows > INT32_MAX) return PKV_ERR_SHAPE;

    // Image: [units][queue offsets][merges], then the partial results.  The
    // decode queues' units come first, then the prefill queues', then the
    // tails'; the queue offsets run over all of them (num_queues +
    // prefill_queues + tail_queues + 1 entries, at most 3 num_queues + 1).
    // Section sizes: the plan's own, or those of the capacity (the same
    // offsets for every plan of that capacity, queues and heads).
    PlanSections sec{num_units, plan_counts_index(num_queues) + kPlanCounts, static_cast<int64_t>(merges.size()),
                     partial_rows};
    if (cap_seqs >= 0) {
        if (rows > cap_tokens) return PKV_ERR_SHAPE;
        const PlanSections cap = plan_capacity(cap_seqs, cap_tokens, num_q_heads, num_kv_heads, num_queues);
        if (num_units > cap.units || sec.merges > cap.merges || partial_rows > cap.prows) return PKV_ERR_SHAPE;
        sec = cap;
    }
    const size_t units_bytes = align_up(static_cast<size_t>(sec.units) * sizeof(Unit));
    const size_t queues_bytes = align_up(static_cast<size_t>(sec.queue_ints) * sizeof(int32_t));
    const size_t merges_bytes = align_up(static_cast<size_t>(sec.merges) * sizeof(Merge));
    const size_t image = units_bytes + queues_bytes + merges_bytes;
    const size_t po_bytes = align_up(static_cast<size_t>(sec.prows) * static_cast<size_t>(hd) * sizeof(float));
    const size_t pl_bytes =
        align_up(static_cast<size_t>(sec.prows) * static_cast<size_t>(num_q_heads) * sizeof(float));

    plan->num_seqs = num_seqs;
    plan->num_tokens = static_cast<int32_t>(rows);
    plan->num_q_heads = num_q_heads;
    plan->num_kv_heads = num_kv_heads;
    plan->head_dim = head_dim;
    plan->num_queues = num_queues;
    plan->num_units = static_cast<int32_t>(num_units);
    plan->num_merges = static_cast<int32_t>(merges.size());
    plan->num_partial_rows = static_cast<int32_t>(partial_rows);
    plan->target_tiles = static_cast<int32_t>(std::min<int64_t>(target, INT32_MAX));
    plan->max_q_len = max_q;
    plan->num_prefill_queues = prefill_queues + tail_queues;
    plan->num_tail_queues = tail_queues;
    plan->num_prefill_units = static_cast<int32_t>(num_prefill_units);
    plan->num_wide_merges = num_wide;
    plan->num_block_merges = num_block;
    plan->max_row_merges = static_cast<int32_t>(row_slots);
    plan->max_block_merges = static_cast<int32_t>(std::min<int64_t>(block_slots, INT32_MAX));
    plan->window_left = window;
    plan->logits_soft_cap = soft_cap;
    plan->off_units = 0;
    plan->off_queues = static_cast<int64_t>(units_bytes);
    plan->off_merges = static_cast<int64_t>(units_bytes + queues_bytes);
    plan->off_partial_o = static_cast<int64_t>(image);
    plan->off_partial_lse = static_cast<int64_t>(image + po_bytes);
    plan->image_bytes = static_cast<int64_t>(image);
    plan->workspace_bytes = static_cast<int64_t>(image + po_bytes + pl_bytes);

    if (host_image == nullptr) {
        plan->magic = PKV_PLAN_MAGIC;
        return PKV_OK;
    }
    if (host_bytes < image) return PKV_ERR_WORKSPACE;
    char* base = static_cast<char*>(host_image);
    std::memset(base, 0, image);
    Unit* u = reinterpret_cast<Unit*>(base);
    int32_t* qoff = reinterpret_cast<int32_t*>(base + units_bytes);
    int32_t cursor = 0;
    for (int32_t q = 0; q < num_queues; ++q) {
        qoff[q] = cursor;
        for (const Unit& x : queues[q]) u[cursor++] = x;
    }
    for (int32_t q = 0; q < prefill_queues + tail_queues; ++q) {
        qoff[num_queues + q] = cursor;
        for (const Unit& x : pqueues[q]) u[cursor++] = x;
    }
    qoff[num_queues + prefill_queues + tail_queues] = cursor;
    int32_t* counts = qoff + plan_counts_index(num_queues);
    counts[0] = static_cast<int32_t>(merges.size());
    counts[1] = num_wide;
    counts[2] = num_block;
    Merge* mrec = reinterpret_cast<Merge*>(base + units_bytes + queues_bytes);
    for (size_t i = 0; i < merges.size(); ++i) mrec[i] = merges[i].second;
    plan->magic = PKV_PLAN_MAGIC;
    return PKV_OK;
}

void plan_bounds(int32_t max_seqs, int32_t max_tokens, int32_t num_q_heads, int32_t head_dim,
                 int32_t num_queues, size_t* workspace_bytes, size_t* host_bytes) {
    // a unit per kv head and piece: num_q_heads bounds the kv heads
    const PlanSections c = plan_capacity(max_seqs, max_tokens, num_q_heads, num_q_heads, num_queues);
    const size_t image = align_up(static_cast<size_t>(c.units) * sizeof(Unit)) +
                         align_up(static_cast<size_t>(c.queue_ints) * sizeof(int32_t)) +
                         align_up(static_cast<size_t>(c.merges) * sizeof(Merge));
    const size_t hd = static_cast<size_t>(std::max(num_q_heads, 1)) * static_cast<size_t>(std::max(head_dim, 1));
    const size_t po = align_up(static_cast<size_t>(c.prows) * hd * sizeof(float));
    const size_t pl = align_up(static_cast<size_t>(c.prows) * static_cast<size_t>(std::max(num_q_heads, 1)) * sizeof(float));
    if (workspace_bytes) *workspace_bytes = image + po + pl;
    if (host_bytes) *host_bytes = image;
}

}  // namespace pkv
