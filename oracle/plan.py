"""Split-KV planner, as the pages describe it (TEST INFRASTRUCTURE ONLY).

Source: "How Easy Is It to Start Serving LLMs?", Phase 4 §3 "Load balancing:
keep every SM busy".  Once per decode step a host-side plan looks at the
current KV lengths, takes the ideal work per processor as the total divided by
the number of processors, walks the requests longest first, cuts each into
pieces no longer than that ideal share, and gives every piece to the queue
with the least work so far.  Every layer of the step reuses the plan; a merge
step joins the pieces of a request that was cut.

Readings of what the illustration leaves open:

* Work is counted in 16-token tiles, the granularity the kernels walk the
  cache in; a request of ``n`` tokens is ``ceil(n / 16)`` tiles, and every
  piece boundary inside a request falls on a tile boundary.
* The ideal share is ``target = ceil(total_tiles / num_queues)`` tiles.
* "Longest first" sorts by token count, ties by request index.
* "Lightest queue" is the queue with the smallest tile count, ties by the
  lowest queue index.
* The pieces of a request are cut as the request is placed: each piece is as
  long as the lightest queue can still take before it reaches the target
  (never more than the target, never more than what is left of the
  request).  Cutting every request into target-sized pieces up front instead
  leaves queues up to ~1.7x the target on the 64-request decode workload,
  while this reading stays within one tile of it.
* Requests with no keys get no piece.

The result is a list of queues; each queue is a list of
``(request, kv_begin, kv_end)`` token ranges in the order they were placed.
This is integer work: the native planner must reproduce it exactly.
"""

from __future__ import annotations

TILE_TOKENS = 16


def split_lengths(kv_lens, tile: int = TILE_TOKENS):
    """Tiles of each request: ``ceil(n / tile)``."""
    return [-(-int(n) // tile) for n in kv_lens]


def split_kv_plan(kv_lens, num_queues: int, tile: int = TILE_TOKENS):
    """Return ``queues``: ``num_queues`` lists of ``(request, kv_begin, kv_end)``."""
    if num_queues < 1:
        raise ValueError("num_queues must be >= 1")
    lens = [int(n) for n in kv_lens]
    tiles = split_lengths(lens, tile)
    total = sum(tiles)
    queues = [[] for _ in range(num_queues)]
    if total == 0:
        return queues
    target = -(-total // num_queues)
    loads = [0] * num_queues
    order = sorted(range(len(lens)), key=lambda r: (-lens[r], r))
    for r in order:
        remaining = tiles[r]
        first_tile = 0
        while remaining > 0:
            lightest = min(range(num_queues), key=lambda q: (loads[q], q))
            take = min(remaining, target - loads[lightest])
            begin = first_tile * tile
            end = min(lens[r], (first_tile + take) * tile)
            queues[lightest].append((r, begin, end))
            loads[lightest] += take
            remaining -= take
            first_tile += take
    return queues
