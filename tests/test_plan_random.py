"""Seeded random batches through the host planner (CPU only).

For every case the plan image is decoded and checked against what the
planner promises, independently of how it cuts and places the work:
- every visible (row, key) pair of every sequence is in exactly one unit of
  its kv head (decode units hold every kv head), under causal alignment and,
  when set, the sliding window;
- a unit with a partial row belongs to exactly one merge record, whose
  pieces sit at prow0 + c * nrows + r in key order, and a unit without one
  covers its rows' whole visible range;
- the counts after the queue offsets match the records, which come as wide
  one-row records, row blocks, then the other one-row records;
- a plan laid out at a capacity holds the same units, queues and records
  as the compact plan of the same batch, and fits the workspace bound.
"""

import ctypes

import numpy as np
import pytest

import paged_kv_attention_write_amd as pkv
from paged_kv_attention_write_amd import _abi


def merge_kinds(merges, q_lens):
    """Kind of each merge record by where it comes from: 1 for a block of
    chunk rows (even one of a single row), else 0 for a decode row with at
    least 8 pieces and 2 for one with fewer."""
    ql = np.asarray(q_lens, np.int64)
    cu = np.concatenate([[0], np.cumsum(ql)])
    seq = np.searchsorted(cu, merges[:, 0], side="right") - 1
    chunk = ql[seq] > 1 if len(merges) else np.zeros(0, bool)
    return np.where(chunk, 1, np.where(merges[:, 3] >= 8, 0, 2))


def check_merge_room(p, merges, q_lens, group):
    """The counts the attention calls check before launching (and that size
    a merge launch made under stream capture) hold for the plan the planner
    made: one-row records fit the room of the decode rows, row-block records
    the room of the chunks' row blocks."""
    ql = np.asarray(q_lens, np.int64)
    kind = merge_kinds(merges, ql)
    assert int(p.num_merges) == len(merges)
    assert int(p.num_wide_merges) == int((kind == 0).sum())
    assert int(p.num_block_merges) == int((kind == 1).sum())
    rows = max(1, 128 // group)
    assert int(p.max_row_merges) == int((ql == 1).sum())
    assert int(p.max_block_merges) == int(sum(-(-int(L) // rows) for L in ql if L > 1))
    assert p.num_wide_merges + p.num_block_merges <= p.num_merges
    assert p.num_wide_merges <= p.max_row_merges
    assert p.num_block_merges <= p.max_block_merges
    assert p.num_merges - p.num_block_merges <= p.max_row_merges


def _random_batch(rng):
    B = int(rng.integers(1, 40))
    lens = rng.integers(0, 6000, size=B)
    lens[rng.random(B) < 0.1] = 0
    ql = np.ones(B, np.int64)
    chunky = rng.random(B) < 0.3
    ql[chunky] = rng.integers(2, 400, size=int(chunky.sum()))
    ql = np.minimum(ql, np.maximum(lens, 0))
    ql[(lens > 0) & (ql == 0)] = 1
    whole = (rng.random(B) < 0.1) & (lens > 0) & (lens < 500)
    ql[whole] = lens[whole]  # a whole prompt as one chunk
    return lens.astype(np.int32), ql.astype(np.int32)


def _capacity_plan(lens, ql, hq, hkv, d, nq, window, cap_seqs, cap_tokens):
    p = _abi.PkvPlan()
    L = pkv.lib()
    args = (lens.ctypes.data, ql.ctypes.data, lens.shape[0], hq, hkv, d, nq, 0.0, window, cap_seqs, cap_tokens)
    assert L.paged_attn_plan_variant(*args, None, 0, None, 0, ctypes.byref(p), None) == 0
    image = np.zeros(max(int(p.image_bytes), 1), np.uint8)
    assert L.paged_attn_plan_variant(*args, image.ctypes.data, image.nbytes, None, 0, ctypes.byref(p), None) == 0
    return p, image


def _check_plan(p, image, lens, ql, hq, hkv, window):
    units, qoff, merges = pkv.decode_plan_image(p, image)
    cu = np.concatenate([[0], np.cumsum(ql)])
    assert p.num_tokens == cu[-1] and p.num_units == len(units)
    # a few-row step: every chunk within 16 (row, q head) pairs per kv head
    few = int(ql.max(initial=0)) > 1 and int(ql.max()) * (hq // hkv) <= 16
    if few:
        assert p.num_prefill_units == 0
    assert qoff[0] == 0 and qoff[-1] == p.num_units and np.all(np.diff(qoff) >= 0)
    nq = p.num_queues
    # decode units on decode queues, prefill units on prefill queues
    assert np.all(units[:qoff[nq], 7] == 0) and np.all(units[qoff[nq]:, 7] >= 1)
    # counts after the queue offsets
    q32 = np.asarray(image[p.off_queues:p.off_merges]).view(np.int32)
    ci = 3 * nq + 1
    assert list(q32[ci:ci + 3]) == [p.num_merges, p.num_wide_merges, p.num_block_merges]
    kind = merge_kinds(merges, ql)
    assert np.all(np.diff(kind) >= 0)
    check_merge_room(p, merges, ql, hq // hkv)
    # merge records and partial rows
    owner = {}
    for m, (row0, nrows, prow0, parts) in enumerate(merges):
        assert parts >= 2
        for c in range(parts):
            for r in range(nrows):
                assert prow0 + c * nrows + r not in owner
                owner[prow0 + c * nrows + r] = (m, c, r)
    assert len(owner) == p.num_partial_rows
    for s in range(lens.shape[0]):
        n, L = int(lens[s]), int(ql[s])
        mine = units[units[:, 0] == s]
        if n == 0 or L == 0:
            assert len(mine) == 0
            continue
        # a chunk unit holds one kv head; decode units (one row, or the few
        # rows of a few-row step) every kv head
        heads = hkv if L > 1 and not few else 1
        cover = np.zeros((heads, L, n), np.int32)
        for u in mine:
            seq, kb, ke, row0, nrows, pos0, prow, k = (int(x) for x in u)
            r0 = row0 - cu[s]
            assert 0 <= r0 and r0 + nrows <= L and pos0 == n - L + r0 and kb < ke <= n
            for i in range(nrows):
                pos = pos0 + i
                lo = max(kb, pos - window + 1) if window > 0 else kb
                hi = min(ke, pos + 1)
                if hi > lo:
                    cover[max(k - 1, 0), r0 + i, lo:hi] += 1
            if prow >= 0:
                m, c, r = owner[prow]
                assert r == 0 and merges[m][0] == row0 and merges[m][1] == nrows
            else:  # not cut: from its first row's first visible key to its last row
                first = max(0, pos0 - window + 1) if window > 0 else 0
                assert kb <= first and ke == pos0 + nrows
        pos = n - L + np.arange(L)
        j = np.arange(n)[None, :]
        vis = j <= pos[:, None]
        if window > 0:
            vis &= j > pos[:, None] - window
        assert np.array_equal(cover, np.broadcast_to(vis.astype(np.int32), cover.shape)), s


@pytest.mark.parametrize("seed", range(24))
def test_random_batches(seed):
    rng = np.random.default_rng(1000 + seed)
    lens, ql = _random_batch(rng)
    hkv = int(rng.choice([1, 2, 4, 8]))
    hq = hkv * int(rng.choice([1, 2, 4, 8]))
    d = int(rng.choice([64, 128]))
    nq = int(rng.integers(1, 300))
    window = int(rng.choice([0, 0, 1, 17, 300, 5000]))
    p, image = pkv.plan_host(lens, ql, hq, hkv, d, nq, window=window)
    assert p.window_left == window
    _check_plan(p, image, lens, ql, hq, hkv, window)
    # tail queues (one per decode queue, the last prefill queues) exactly
    # when the step has decode units and chunk units
    decode_units = int(p.num_units) - int(p.num_prefill_units)
    tails = nq if decode_units > 0 and int(p.num_prefill_units) > 0 else 0
    assert int(p.num_tail_queues) == tails
    if tails:
        assert int(p.num_prefill_queues) == 2 * nq

    # the same batch at a capacity: same content at the capacity's offsets
    cap_seqs = lens.shape[0] + int(rng.integers(0, 8))
    cap_tokens = int(ql.sum()) + int(rng.integers(0, 64))
    pc, imc = _capacity_plan(lens, ql, hq, hkv, d, nq, window, cap_seqs, cap_tokens)
    uc, qc, mc = pkv.decode_plan_image(pc, imc)
    u0, q0, m0 = pkv.decode_plan_image(p, image)
    assert np.array_equal(uc, u0) and np.array_equal(qc, q0) and np.array_equal(mc, m0)
    ws, host = ctypes.c_size_t(0), ctypes.c_size_t(0)
    assert pkv.lib().paged_attn_workspace_size(cap_seqs, cap_tokens, hq, d, nq, ctypes.byref(ws),
                                               ctypes.byref(host)) == 0
    assert pc.workspace_bytes <= ws.value and pc.image_bytes <= host.value


@pytest.mark.parametrize("seed", range(16))
def test_random_few_row_batches(seed):
    """Few-row steps (every sequence with at most 16 / G rows, some with one):
    planned through the decode queues, every visible pair once, the capacity
    layout and the workspace bound as for any plan."""
    rng = np.random.default_rng(2000 + seed)
    B = int(rng.integers(1, 80))
    hkv = int(rng.choice([1, 2, 4, 8]))
    g = int(rng.choice([1, 2, 4, 8]))
    lens = rng.integers(0, 5000, size=B)
    ql = rng.integers(1, 16 // g + 1, size=B)
    ql = np.minimum(ql, lens)
    ql[(lens > 0) & (ql == 0)] = 1
    lens, ql = lens.astype(np.int32), ql.astype(np.int32)
    nq = int(rng.integers(1, 300))
    window = int(rng.choice([0, 0, 1, 17, 300]))
    p, image = pkv.plan_host(lens, ql, hkv * g, hkv, 128, nq, window=window)
    if int(ql.max(initial=0)) > 1:
        assert p.num_prefill_units == 0 and p.num_prefill_queues == 0
    _check_plan(p, image, lens, ql, hkv * g, hkv, window)
    cap_seqs, cap_tokens = B + 3, int(ql.sum()) + 5
    pc, imc = _capacity_plan(lens, ql, hkv * g, hkv, 128, nq, window, cap_seqs, cap_tokens)
    uc, qc, mc = pkv.decode_plan_image(pc, imc)
    u0, q0, m0 = pkv.decode_plan_image(p, image)
    assert np.array_equal(uc, u0) and np.array_equal(qc, q0) and np.array_equal(mc, m0)
    ws, host = ctypes.c_size_t(0), ctypes.c_size_t(0)
    assert pkv.lib().paged_attn_workspace_size(cap_seqs, cap_tokens, hkv * g, 128, nq, ctypes.byref(ws),
                                               ctypes.byref(host)) == 0
    assert pc.workspace_bytes <= ws.value and pc.image_bytes <= host.value


@pytest.mark.parametrize("lens,ql,nq", [([4000], [33], 256), ([4000, 3000], [33, 1], 256), ([4000], [65], 256),
                                        ([9000, 100], [97, 1], 64), ([2048 + 33], [33], 1024)])
def test_single_row_chunk_block_is_a_block_record(lens, ql, nq):
    """A chunk whose last row block holds one row (q_len = 1 mod 128 / G) over
    a long prefix is cut into pieces; its merge record is a row-block record,
    so the plan passes the attention calls' room checks."""
    lens, ql = np.array(lens, np.int32), np.array(ql, np.int32)
    p, image = pkv.plan_host(lens, ql, 32, 8, 128, nq)
    _, _, merges = pkv.decode_plan_image(p, image)
    assert p.num_block_merges >= 1
    check_merge_room(p, merges, ql, 4)
    _check_plan(p, image, lens, ql, 32, 8, 0)
