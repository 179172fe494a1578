"""Pins of the oracle's split-KV planner (CPU).

The planner is integer work; it is pinned by a hand-worked example
(tests/golden/plan_worked_example.txt) and by the properties the blog states
for it ("How Easy Is It to Start Serving LLMs?", Phase 4 §3): every token of
every request is covered once, pieces never exceed the ideal share, requests
are placed longest first, each piece goes to the least-loaded queue, and the
queues end balanced.
"""

import os

import numpy as np
import pytest

from oracle.plan import illustration_plan, split_kv_plan, split_lengths, TILE_TOKENS

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden(name="plan_worked_example.txt"):
    lens, nq, rows = None, None, []
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if line.startswith("# lengths:"):
                lens = [int(x) for x in line.split(":")[1].split()]
            elif line.startswith("# queues:"):
                nq = int(line.split(":")[1])
            elif line and not line.startswith("#"):
                rows.append(tuple(int(x) for x in line.split()))
    return lens, nq, rows


def test_worked_example():
    lens, nq, rows = _golden()
    queues = split_kv_plan(lens, nq)
    got = [(q, r, b, e) for q, items in enumerate(queues) for (r, b, e) in items]
    assert got == rows


def test_worked_example_with_unit_cost():
    """One tile of set-up per piece, including a first placement whose
    set-up overflows the target (every queue full while a request has
    tiles), so the target is raised and the requests are placed again."""
    lens, nq, rows = _golden("plan_unit_cost_example.txt")
    queues = split_kv_plan(lens, nq, unit_cost=1)
    got = [(q, r, b, e) for q, items in enumerate(queues) for (r, b, e) in items]
    assert got == rows


@pytest.mark.parametrize("seed", range(6))
@pytest.mark.parametrize("nq", [1, 3, 16, 256])
def test_unit_cost_covers_once_and_bounds_loads(seed, nq):
    """With set-up per piece: every token covered once in tile-aligned
    pieces; every queue's load (tiles + one per piece) stays within one
    tile of the balanced share ceil((tiles + pieces) / queues) of the plan
    made (the target is raised when the set-up overflows it, so no queue
    takes a whole rest); zero set-up is the page's reading."""
    rng = np.random.default_rng(90 + seed)
    lens = [int(x) for x in rng.integers(0, 3000, size=int(rng.integers(1, 70)))]
    assert split_kv_plan(lens, nq, unit_cost=0) == split_kv_plan(lens, nq)
    queues = split_kv_plan(lens, nq, unit_cost=1)
    tiles = split_lengths(lens)
    pieces = sum(len(items) for items in queues)
    share = -(-(sum(tiles) + pieces) // nq)
    spans = {r: [] for r in range(len(lens))}
    for items in queues:
        load = 0
        for r, b, e in items:
            assert b % TILE_TOKENS == 0 and (e % TILE_TOKENS == 0 or e == lens[r])
            load += -(-(e - b) // TILE_TOKENS) + 1
            spans[r].append((b, e))
        assert load <= share + 1
    for r, sp in spans.items():
        sp.sort()
        pos = 0
        for b, e in sp:
            assert b == pos
            pos = e
        assert pos == lens[r]


def _check_properties(lens, nq):
    queues = split_kv_plan(lens, nq)
    assert len(queues) == nq
    tiles = split_lengths(lens)
    target = -(-sum(tiles) // nq) if sum(tiles) else 0
    covered = {r: [] for r in range(len(lens))}
    for items in queues:
        load = 0
        for r, b, e in items:
            assert 0 <= b < e <= lens[r]
            assert b % TILE_TOKENS == 0
            assert e % TILE_TOKENS == 0 or e == lens[r]
            t = -(-(e - b) // TILE_TOKENS)
            assert t <= target
            load += t
            covered[r].append((b, e))
        assert load <= target
    for r, spans in covered.items():
        spans.sort()
        pos = 0
        for b, e in spans:
            assert b == pos
            pos = e
        assert pos == lens[r]
    return queues, target


@pytest.mark.parametrize("seed", range(6))
@pytest.mark.parametrize("nq", [1, 3, 16, 256])
def test_cover_once_pieces_bounded_balanced(seed, nq):
    rng = np.random.default_rng(seed)
    lens = list(rng.integers(0, 3000, size=int(rng.integers(1, 70))))
    _check_properties(lens, nq)


def test_longest_first_and_lightest_queue_by_replay():
    rng = np.random.default_rng(42)
    lens = list(rng.integers(1, 5000, size=40))
    nq = 13
    queues = split_kv_plan(lens, nq)
    # replay the placement order: requests in longest-first order, pieces of a
    # request in token order; each placement must have gone to a lightest queue
    pieces = [(r, b, e, q) for q, items in enumerate(queues) for (r, b, e) in items]
    order = sorted(range(len(lens)), key=lambda r: (-lens[r], r))
    rank = {r: i for i, r in enumerate(order)}
    pieces.sort(key=lambda p: (rank[p[0]], p[1]))
    loads = [0] * nq
    seen_in_queue = [0] * nq
    for r, b, e, q in pieces:
        assert loads[q] == min(loads)
        assert q == loads.index(min(loads))  # ties to the lowest index
        # and a queue's list keeps placement order
        assert queues[q][seen_in_queue[q]] == (r, b, e)
        seen_in_queue[q] += 1
        loads[q] += -(-(e - b) // TILE_TOKENS)


def test_balance_on_the_decode_workload():
    rng = np.random.default_rng([1, 0])
    lens = list(rng.integers(512, 4096, size=64, endpoint=True))
    for nq in (256, 512):
        queues, target = _check_properties(lens, nq)
        loads = [sum(-(-(e - b) // 16) for _, b, e in q) for q in queues]
        assert max(loads) <= target
        assert max(loads) * nq <= 1.05 * sum(split_lengths(lens)) + nq
        # every request cut at most at queue boundaries: pieces <= queues + requests
        assert sum(len(q) for q in queues) <= nq + len(lens)


def test_empty_and_zero_lengths():
    assert split_kv_plan([], 4) == [[], [], [], []]
    assert split_kv_plan([0, 0], 2) == [[], []]
    q = split_kv_plan([0, 5, 0], 2)
    assert sum(len(x) for x in q) == 1 and q[0] == [(1, 0, 5)]
    with pytest.raises(ValueError):
        split_kv_plan([3], 0)


def _illustration_golden():
    cases = {}
    with open(os.path.join(GOLDEN, "plan_illustration_example.txt")) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            head, row = line.split("|")
            ex, lens, nq, tile = head.split()
            key = (int(ex), tuple(int(x) for x in lens.split(",")), int(nq), int(tile))
            cases.setdefault(key, []).append(tuple(int(x) for x in row.split()))
    return cases


def test_illustration_worked_examples():
    """The illustration's steps as printed (cut every request, then place
    each chunk on the least-loaded queue), against hand-derived placements."""
    cases = _illustration_golden()
    assert len(cases) == 3
    for (_, lens, nq, tile), rows in cases.items():
        queues = illustration_plan(list(lens), nq, tile)
        got = [(q, r, b, e) for q, items in enumerate(queues) for (r, b, e) in items]
        assert got == rows, (lens, nq, tile)


@pytest.mark.parametrize("seed", range(4))
@pytest.mark.parametrize("nq", [1, 7, 64])
def test_illustration_covers_once_with_chunks_of_the_target(seed, nq):
    rng = np.random.default_rng(50 + seed)
    lens = [int(x) for x in rng.integers(0, 3000, size=int(rng.integers(1, 60)))]
    queues = illustration_plan(lens, nq)
    target = sum(lens) / nq
    chunk = max(1, int(target // 1))
    spans = {r: [] for r in range(len(lens))}
    for items in queues:
        for r, b, e in items:
            assert 0 <= b < e <= lens[r] and e - b <= chunk
            spans[r].append((b, e))
    for r, sp in spans.items():
        sp.sort()
        # every chunk but the last is exactly `chunk` long and they tile [0, n)
        assert [b for b, _ in sp] == list(range(0, lens[r], chunk))
        assert (sp[-1][1] if sp else 0) == lens[r]


def test_queue_balance_of_the_two_readings_on_the_decode_workload():
    """Largest over mean queue work on the 64-request decode workload
    (context U[512, 4096]) at 256 queues: cutting every request into
    target-sized chunks before placing them (the illustration's steps) leaves
    the largest queue at 1.61x the mean; cutting each piece to what the
    least-loaded queue can still take leaves it at 1.02x.  These are the
    figures quoted for the planner reading the library follows."""
    import workloads

    lens = [int(x) for x in workloads.decode_lengths("decode")]
    assert len(lens) == 64

    def ratio(queues, tile):
        loads = [sum(-(-(e - b) // tile) for _, b, e in q) for q in queues]
        return max(loads) / (sum(loads) / len(loads))

    printed = ratio(illustration_plan(lens, 256), 1)
    printed_tiles = ratio(illustration_plan(lens, 256, TILE_TOKENS), TILE_TOKENS)
    lazy = ratio(split_kv_plan(lens, 256), TILE_TOKENS)
    assert round(printed, 2) == 1.61 and round(printed_tiles, 2) == 1.62
    assert round(lazy, 2) == 1.02
