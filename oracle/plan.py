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
  request).  This fuses the illustration's two steps (cut, then place) into
  one; :func:`illustration_plan` keeps them apart, as printed, and
  ``tests/test_oracle_plan.py`` measures both on the 64-request decode
  workload at 256 queues: the largest queue holds 1.61x the mean work with
  the illustration's steps and 1.02x with this reading.
* Requests with no keys get no piece.
* ``unit_cost`` (tiles): every piece also adds this much to its queue's load
  (the set-up of a unit of work: its first table reads and loads, its
  flush), and the target grows by that much per queue.  0 is the page's
  reading; the library plans with 1, the set-up time of a unit it measured
  as about one tile's.  Cutting makes more pieces than queues; if their
  set-up overflows the target (the lightest queue has no room while a
  request still has tiles, so it would take the whole rest), the target is
  raised to ``ceil((total + unit_cost * pieces) / num_queues)`` (at least one
  more) and every request is placed again, at most 4 placements in all.
  With ``unit_cost == 0`` the target always holds the total and one
  placement is made.

``split_kv_plan`` returns a list of queues; each queue is a list of
``(request, kv_begin, kv_end)`` token ranges in the order they were placed.
This is integer work: the native planner must reproduce it exactly.
"""

from __future__ import annotations

TILE_TOKENS = 16


def split_lengths(kv_lens, tile: int = TILE_TOKENS):
    """Tiles of each request: ``ceil(n / tile)``."""
    return [-(-int(n) // tile) for n in kv_lens]


def split_kv_plan(kv_lens, num_queues: int, tile: int = TILE_TOKENS, unit_cost: int = 0):
    """Return ``queues``: ``num_queues`` lists of ``(request, kv_begin, kv_end)``."""
    if num_queues < 1:
        raise ValueError("num_queues must be >= 1")
    lens = [int(n) for n in kv_lens]
    tiles = split_lengths(lens, tile)
    total = sum(tiles)
    queues = [[] for _ in range(num_queues)]
    if total == 0:
        return queues
    target = -(-(total + unit_cost * num_queues) // num_queues)
    order = sorted(range(len(lens)), key=lambda r: (-lens[r], r))
    for attempt in range(4):
        queues = [[] for _ in range(num_queues)]
        loads = [0] * num_queues
        pieces = 0
        over = False
        for r in order:
            remaining = tiles[r]
            first_tile = 0
            while remaining > 0:
                lightest = min(range(num_queues), key=lambda q: (loads[q], q))
                room = target - loads[lightest] - unit_cost
                over = over or room <= 0
                take = min(remaining, room) if room > 0 else remaining
                begin = first_tile * tile
                end = min(lens[r], (first_tile + take) * tile)
                queues[lightest].append((r, begin, end))
                loads[lightest] += take + unit_cost
                remaining -= take
                first_tile += take
                pieces += 1
        if not over or unit_cost == 0:
            break
        target = max(target + 1, -(-(total + unit_cost * pieces) // num_queues))
    return queues


def illustration_plan(kv_lens, num_queues: int, tile: int = 1):
    """The planner with the illustration's two steps kept apart.

    Work is counted in units of ``tile`` tokens (1: tokens, as printed).  The
    ideal work per queue is the total divided by the queue count (a real
    number); every request, longest first (ties: lower index), is first cut
    by ``split(n, max_len=target)`` and the chunks are then placed one by one,
    each on the queue with the least work so far (ties: lower index).
    ``split`` is not printed; read as consecutive chunks of
    ``max(1, floor(target))`` units from the start of the request, the last
    one shorter: the longest integer length that does not exceed the target,
    and it depends only on ``n`` and the target.

    Returns ``queues``: ``num_queues`` lists of ``(request, kv_begin,
    kv_end)`` token ranges in placement order.
    """
    if num_queues < 1:
        raise ValueError("num_queues must be >= 1")
    lens = [int(n) for n in kv_lens]
    work = [-(-n // tile) for n in lens]
    queues = [[] for _ in range(num_queues)]
    total = sum(work)
    if total == 0:
        return queues
    target = total / num_queues
    max_len = max(1, int(target // 1))
    loads = [0] * num_queues
    for r in sorted(range(len(lens)), key=lambda r: (-work[r], r)):
        chunks = [(b, min(work[r], b + max_len)) for b in range(0, work[r], max_len)]   # split(n, max_len)
        for b, e in chunks:
            lightest = min(range(num_queues), key=lambda q: (loads[q], q))
            queues[lightest].append((r, b * tile, min(lens[r], e * tile)))
            loads[lightest] += e - b
    return queues
