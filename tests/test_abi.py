"""CPU tests of the C-ABI library: it loads, exports what include/pkv.h declares,
its host planner reproduces the oracle's plan exactly, and its argument checks
return the documented status before anything is launched.

The argument-check tests pass dummy device addresses: they are skipped when a
GPU is present so that a checking bug can never launch a kernel on them.
"""

import os
import re

import numpy as np
import pytest

import paged_kv_attention_write_amd as pkv
from paged_kv_attention_write_amd import _abi
from oracle.plan import split_kv_plan
from conftest import gpu_available

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

cpu_only = pytest.mark.skipif(gpu_available(), reason="dummy-pointer checks run on the CPU tier only")


def _header_functions():
    text = open(os.path.join(ROOT, "include", "pkv.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[a-z_0-9]+\s*\*?\s*([a-z_0-9]+)\s*\(", text, flags=re.M)))


def test_library_loads_and_exports_every_declared_symbol():
    L = pkv.lib()
    declared = _header_functions()
    assert set(declared) == set(_abi.EXPORTS), declared
    for name in declared:
        assert hasattr(L, name), name
    assert L.pkv_abi_version() == 6
    assert L.pkv_set_split_event(None) == 0  # the timing hook, off


def test_strerror_covers_all_codes():
    for code in range(0, -8, -1):
        msg = pkv.strerror(code)
        assert msg and msg != "unknown status"
    assert pkv.strerror(-99) == "unknown status"


def _queues_from_image(p, image):
    units, qoff, _ = pkv.decode_plan_image(p, image)
    out = []
    for q in range(p.num_queues):
        out.append([(int(u[0]), int(u[1]), int(u[2])) for u in units[qoff[q]:qoff[q + 1]]])
    return out


@pytest.mark.parametrize("seed", range(8))
@pytest.mark.parametrize("nq", [1, 5, 64, 512])
def test_native_plan_equals_oracle_plan(seed, nq):
    rng = np.random.default_rng(seed)
    lens = rng.integers(1, 5000, size=int(rng.integers(1, 100)))
    p, image = pkv.plan_host(lens, None, 32, 8, 128, nq)
    assert _queues_from_image(p, image) == split_kv_plan(lens.tolist(), nq, unit_cost=1)


@pytest.mark.parametrize("config", ["tiny", "decode", "long", "fp8prefix"])
def test_native_plan_equals_oracle_plan_on_workloads(config):
    import workloads

    lens = workloads.decode_lengths(config)
    for nq in (256, 512):
        p, image = pkv.plan_host(lens, None, 32, 8, 128, nq)
        assert _queues_from_image(p, image) == split_kv_plan(lens.tolist(), nq, unit_cost=1)


def test_plan_partials_and_merges_are_consistent():
    rng = np.random.default_rng(3)
    lens = rng.integers(1, 3000, size=50)
    p, image = pkv.plan_host(lens, None, 32, 8, 128, 37)
    units, qoff, merges = pkv.decode_plan_image(p, image)
    assert qoff[0] == 0 and qoff[-1] == p.num_units and np.all(np.diff(qoff) >= 0)
    prows = units[units[:, 6] >= 0, 6]
    assert len(set(prows.tolist())) == len(prows) == p.num_partial_rows
    for row0, nrows, prow0, parts in merges:
        assert nrows == 1
        mine = units[(units[:, 0] == row0) & (units[:, 6] >= 0)]
        mine = mine[np.argsort(mine[:, 1])]
        assert len(mine) == parts >= 2
        assert list(mine[:, 6]) == [prow0 + c for c in range(parts)]
    split = {int(m[0]) for m in merges}
    whole = units[units[:, 6] < 0]
    assert not split & set(whole[:, 0].tolist())
    assert p.workspace_bytes >= p.off_partial_lse + 4 * 32 * p.num_partial_rows
    _check_wide_first(p, merges)


def _check_wide_first(p, merges, q_lens=None, group=4):
    """Merge records come as wide ones (one row, at least 8 pieces), then row
    blocks, then one-row records with few pieces, counted in the plan; the
    room bounds follow from q_lens alone."""
    from test_plan_random import check_merge_room, merge_kinds

    ql = np.ones(p.num_seqs, np.int64) if q_lens is None else np.asarray(q_lens)
    kind = merge_kinds(merges, ql)
    assert np.all(np.diff(kind) >= 0)
    check_merge_room(p, merges, ql, group)


@pytest.mark.parametrize("mix", ["uniform", "one-long", "heavy"])
@pytest.mark.parametrize("batch", [4, 64, 128])
def test_wide_merges_first_on_skew_mixes(mix, batch):
    import workloads

    lens = workloads.skew_lengths(mix, batch)
    p, image = pkv.plan_host(lens, None, 32, 8, 128, 256)
    _, _, merges = pkv.decode_plan_image(p, image)
    _check_wide_first(p, merges, np.ones(batch, int))


def _mixed_case():
    rng = np.random.default_rng(11)
    dec = rng.integers(256, 2049, size=20)
    lens = np.concatenate([dec, [2560, 700, 130]])
    ql = np.concatenate([np.ones(20, int), [512, 700, 65]])
    return lens.astype(np.int32), ql.astype(np.int32)


def test_mixed_plan_covers_every_visible_pair_once():
    lens, ql = _mixed_case()
    p, image = pkv.plan_host(lens, ql, 32, 8, 128, 96)
    units, qoff, merges = pkv.decode_plan_image(p, image)
    cu = np.concatenate([[0], np.cumsum(ql)])
    assert p.num_tokens == cu[-1] and p.max_q_len == 700
    hkv = 8
    for s in range(len(lens)):
        n, L = int(lens[s]), int(ql[s])
        heads = hkv if L > 1 else 1  # a prefill unit holds one kv head, a decode unit all of them
        cover = np.zeros((heads, L, n), np.int32)
        for u in units[units[:, 0] == s]:
            seq, kb, ke, row0, nrows, pos0, prow, kind = (int(x) for x in u)
            assert (1 <= kind <= hkv) if L > 1 else kind == 0
            assert kb < ke
            r = row0 - cu[s]
            assert pos0 == n - L + r
            for i in range(nrows):
                pos = pos0 + i
                lo, hi = kb, min(ke, pos + 1)
                if hi > lo:
                    cover[max(kind - 1, 0), r + i, lo:hi] += 1
        visible = np.arange(n)[None, :] <= (n - L + np.arange(L))[:, None]
        assert np.array_equal(cover, np.broadcast_to(visible.astype(np.int32), cover.shape)), s
    _check_wide_first(p, merges, ql)
    # every merged block lists its pieces at prow0 + c * nrows
    for row0, nrows, prow0, parts in merges:
        us = units[(units[:, 3] == row0) & (units[:, 6] >= 0)]
        for kind in sorted(set(us[:, 7].tolist())):
            mine = us[us[:, 7] == kind]
            assert sorted(mine[:, 6].tolist()) == [prow0 + c * nrows for c in range(parts)]
        assert len(us) == parts * (hkv if us[0, 7] >= 1 else 1)


def _first_key(pos, window):
    return max(0, pos - window + 1) if window > 0 else 0


@pytest.mark.parametrize("window", [1, 16, 100, 700, 5000])
def test_window_plan_covers_every_visible_pair_once(window):
    """With a sliding window each (row, key) pair with pos - W < key <= pos is
    in exactly one unit of its kv head, and a range starts no earlier than the
    tile that holds its first row's first visible key."""
    lens, ql = _mixed_case()
    p, image = pkv.plan_host(lens, ql, 32, 8, 128, 96, window=window)
    assert p.window_left == window and p.logits_soft_cap == 0.0
    units, qoff, merges = pkv.decode_plan_image(p, image)
    cu = np.concatenate([[0], np.cumsum(ql)])
    hkv = 8
    for s in range(len(lens)):
        n, L = int(lens[s]), int(ql[s])
        heads = hkv if L > 1 else 1
        cover = np.zeros((heads, L, n), np.int32)
        mine = units[units[:, 0] == s]
        for u in mine:
            seq, kb, ke, row0, nrows, pos0, prow, kind = (int(x) for x in u)
            assert kb < ke
            r = row0 - cu[s]
            assert kb >= _first_key(pos0, window) // 16 * 16
            for i in range(nrows):
                pos = pos0 + i
                lo, hi = max(kb, _first_key(pos, window)), min(ke, pos + 1)
                if hi > lo:
                    cover[max(kind - 1, 0), r + i, lo:hi] += 1
        pos = n - L + np.arange(L)
        j = np.arange(n)[None, :]
        visible = (j <= pos[:, None]) & (j > pos[:, None] - window)
        assert np.array_equal(cover, np.broadcast_to(visible.astype(np.int32), cover.shape)), s
        # the first piece of each row block starts at its first row's tile
        for row0 in set(mine[:, 3].tolist()):
            blk = mine[mine[:, 3] == row0]
            assert blk[:, 1].min() == _first_key(int(blk[0, 5]), window) // 16 * 16
    _check_wide_first(p, merges, ql)


def test_variant_plan_without_variant_equals_the_plain_plan():
    lens, ql = _mixed_case()
    p0, img0 = pkv.plan_host(lens, ql, 32, 8, 128, 96)
    # a soft-cap changes no range; a window at least as long as every context
    # sees every key
    for kw in (dict(soft_cap=30.0), dict(window=int(lens.max())), dict(window=10**6, soft_cap=50.0)):
        p1, img1 = pkv.plan_host(lens, ql, 32, 8, 128, 96, **kw)
        assert np.array_equal(img0, img1), kw
        assert p1.num_units == p0.num_units and p1.workspace_bytes == p0.workspace_bytes
        assert p1.window_left == kw.get("window", 0)
        assert p1.logits_soft_cap == np.float32(kw.get("soft_cap", 0.0))


def test_variant_plan_rejects_bad_variants():
    for kw in (dict(window=-1), dict(soft_cap=-1.0), dict(soft_cap=float("nan")), dict(soft_cap=float("inf"))):
        with pytest.raises(pkv.PkvError) as e:
            pkv.plan_host([50, 9], None, 8, 2, 64, 4, **kw)
        assert e.value.status == _abi.PKV_ERR_SHAPE, kw


def test_window_shrinks_decode_work():
    """Long decode rows under a window read only the last W keys (rounded
    down to a tile): the share per queue follows the windowed work (plus one
    tile of set-up per queue)."""
    lens = np.full(64, 8192, np.int32)
    p, image = pkv.plan_host(lens, None, 32, 8, 128, 256, window=1000)
    units, _, _ = pkv.decode_plan_image(p, image)
    keys = int((units[:, 2] - units[:, 1]).sum())
    assert keys == 64 * (8192 - (8192 - 1000) // 16 * 16)
    assert p.target_tiles == -(-(keys // 16 + 256) // 256)


def test_mixed_plan_decode_queues_equal_the_decode_plan():
    """Decode rows of a mixed step are placed exactly as a decode-only plan of
    those sequences would place them; chunk units sit on the prefill queues:
    one per decode queue, then a tail queue per decode queue."""
    lens, ql = _mixed_case()
    nq = 96
    p, image = pkv.plan_host(lens, ql, 32, 8, 128, nq)
    units, qoff, _ = pkv.decode_plan_image(p, image)
    npq = p.num_prefill_queues
    assert p.num_tail_queues == nq and npq == 2 * nq and len(qoff) == nq + npq + 1
    dec = np.nonzero(ql == 1)[0]
    want = split_kv_plan(lens[dec].tolist(), nq, unit_cost=1)
    got = [[(int(dec.tolist().index(u[0])), int(u[1]), int(u[2])) for u in units[qoff[q]:qoff[q + 1]]]
           for q in range(nq)]
    assert got == want
    pre = units[qoff[nq]:qoff[nq + npq]]
    assert len(pre) == p.num_prefill_units and np.all(pre[:, 7] >= 1)
    assert np.all(units[:qoff[nq], 7] == 0)
    assert qoff[nq + npq] == p.num_units


def test_decode_only_plan_has_no_prefill_queues():
    lens = np.array([100, 2000, 5], np.int32)
    p, image = pkv.plan_host(lens, None, 32, 8, 128, 16)
    units, qoff, _ = pkv.decode_plan_image(p, image)
    assert p.num_prefill_queues == 0 and p.num_prefill_units == 0 and len(qoff) == 17


def test_workspace_bound_covers_plans():
    rng = np.random.default_rng(5)
    for _ in range(20):
        B = int(rng.integers(1, 80))
        lens = rng.integers(1, 9000, size=B).astype(np.int32)
        ql = np.where(rng.random(B) < 0.2, rng.integers(1, 300, size=B), 1).astype(np.int32)
        ql = np.minimum(ql, lens)
        nq = int(rng.integers(1, 600))
        p, _ = pkv.plan_host(lens, ql, 16, 4, 128, nq)
        ws, host = _sizes(B, int(ql.sum()), 16, 128, nq)
        assert ws >= p.workspace_bytes and host >= p.image_bytes


def _sizes(max_seqs, max_tokens, hq, d, nq):
    import ctypes

    ws, host = ctypes.c_size_t(0), ctypes.c_size_t(0)
    st = pkv.lib().paged_attn_workspace_size(max_seqs, max_tokens, hq, d, nq, ctypes.byref(ws), ctypes.byref(host))
    assert st == 0
    return ws.value, host.value


def test_plan_host_rejects_bad_lengths_and_shapes():
    with pytest.raises(pkv.PkvError) as e:
        pkv.plan_host([5, 3], [1, 4], 8, 2, 64, 4)          # q_len > context_len
    assert e.value.status == _abi.PKV_ERR_SHAPE
    with pytest.raises(pkv.PkvError) as e:
        pkv.plan_host([5, -1], None, 8, 2, 64, 4)
    assert e.value.status == _abi.PKV_ERR_SHAPE
    with pytest.raises(pkv.PkvError) as e:
        pkv.plan_host([5], None, 6, 4, 64, 4)               # Hq % H_kv != 0
    assert e.value.status == _abi.PKV_ERR_SHAPE
    with pytest.raises(pkv.PkvError) as e:
        pkv.plan_host([5], None, 8, 2, 64, 0)               # no queues
    assert e.value.status == _abi.PKV_ERR_SHAPE
    p, image = pkv.plan_host([], None, 8, 2, 64, 3)          # empty batch is fine
    assert p.num_units == 0 and p.num_tokens == 0


# ---------------------------------------------------------------------------
# argument checks that return before any launch (dummy addresses, CPU only)
# ---------------------------------------------------------------------------

A = 1 << 20  # a 1 MiB-aligned dummy address; never dereferenced by these calls


def _write(**kw):
    args = dict(k_new=A, v_new=A, new_dtype=1, stride=1024, slots=A, T=4, kc=A, vc=A, cache_dtype=1, nb=8, bs=16,
                hkv=8, d=128, ks=1.0, vs=1.0, stream=None)
    args.update(kw)
    return pkv.lib().paged_kv_write(*args.values())


@cpu_only
def test_write_argument_checks():
    assert _write(new_dtype=7) == _abi.PKV_ERR_DTYPE
    assert _write(new_dtype=2) == _abi.PKV_ERR_DTYPE          # fp8 is a cache dtype only
    assert _write(new_dtype=1, cache_dtype=0) == _abi.PKV_ERR_UNSUPPORTED  # bf16 -> f32 not offered
    assert _write(d=12) == _abi.PKV_ERR_SHAPE
    assert _write(stride=1000) == _abi.PKV_ERR_SHAPE           # < H_kv * D
    assert _write(bs=0) == _abi.PKV_ERR_SHAPE
    assert _write(cache_dtype=2, ks=0.0) == _abi.PKV_ERR_SHAPE
    assert _write(cache_dtype=2, vs=float("nan")) == _abi.PKV_ERR_SHAPE
    assert _write(k_new=None) == _abi.PKV_ERR_NULL
    assert _write(slots=None) == _abi.PKV_ERR_NULL
    assert _write(k_new=A + 4) == _abi.PKV_ERR_SHAPE           # misaligned
    assert _write(T=0, k_new=None, slots=None) == _abi.PKV_OK   # nothing to do


def _decode(the_plan, **kw):
    import ctypes

    args = dict(out=A, q=A, q_dtype=1, q_stride=4096, kc=A, vc=A, kv_dtype=1, tables=A, max_blocks=64,
                ctx=A, B=4, hq=32, hkv=8, d=128, nb=1000, bs=16, scale=0.088, ks=1.0, vs=1.0,
                plan=ctypes.byref(the_plan), ws=A, ws_bytes=1 << 30, stream=None)
    args.update(kw)
    return pkv.lib().paged_attn_decode(*args.values())


@cpu_only
def test_decode_argument_checks():
    import ctypes

    p, _ = pkv.plan_host([100, 200, 300, 400], None, 32, 8, 128, 16)
    assert _decode(p, q_dtype=2) == _abi.PKV_ERR_DTYPE
    assert _decode(p, kv_dtype=9) == _abi.PKV_ERR_DTYPE
    assert _decode(p, d=96) == _abi.PKV_ERR_UNSUPPORTED
    assert _decode(p, hkv=3) == _abi.PKV_ERR_SHAPE
    assert _decode(p, hq=48, hkv=3) == _abi.PKV_ERR_UNSUPPORTED   # group 16
    assert _decode(p, q_dtype=0) == _abi.PKV_ERR_UNSUPPORTED      # f32 q with bf16 cache
    assert _decode(p, kv_dtype=2, ks=-1.0) == _abi.PKV_ERR_SHAPE
    assert _decode(p, q_stride=100) == _abi.PKV_ERR_SHAPE
    assert _decode(p, plan=None) == _abi.PKV_ERR_NULL
    assert _decode(p, B=5) == _abi.PKV_ERR_PLAN                   # plan made for 4 sequences
    assert _decode(p, hq=16) == _abi.PKV_ERR_PLAN
    assert _decode(p, ws_bytes=16) == _abi.PKV_ERR_WORKSPACE
    assert _decode(p, out=None) == _abi.PKV_ERR_NULL
    assert _decode(p, q=A + 2) == _abi.PKV_ERR_SHAPE
    stale = _abi.PkvPlan()
    assert _decode(p, plan=ctypes.byref(stale)) == _abi.PKV_ERR_PLAN
    pm, _ = pkv.plan_host([100, 200, 300, 400], [1, 1, 1, 50], 32, 8, 128, 16)
    assert _decode(pm, B=4) == _abi.PKV_ERR_PLAN                  # a mixed plan is not a decode plan


def _prefill_queue_costs(lens, ql, nq=256):
    p, image = pkv.plan_host(lens, ql, 32, 8, 128, nq)
    units, qoff, _ = pkv.decode_plan_image(p, image)
    Q, P = p.num_queues, p.num_prefill_queues

    def pairs(u):
        seq, kb, ke, row0, nrows, pos0 = (int(x) for x in u[:6])
        return sum(max(0, min(ke - 1, pos0 + r) - kb + 1) for r in range(nrows))

    return np.array([sum(pairs(u) for u in units[qoff[q]:qoff[q + 1]]) for q in range(Q, Q + P)])


def test_prefill_units_are_balanced():
    """The prefill queues' visible (row, key) pairs stay within 15 % of their
    mean for a 512-row chunk over 2560 keys, and within 10 % for 64
    sequences of 8 rows over U[512, 4096] keys (32 pairs per kv head, past
    the few-row rule): chunk row blocks are cut to the nearest count of queue
    shares, small row blocks 3x finer, and the units are placed largest first
    by their exact flops."""
    import workloads

    st = workloads.structure_only("mixed", "page16")
    chunk = st["q_lens"] > 1
    c = _prefill_queue_costs(st["context_lens"][chunk], st["q_lens"][chunk])
    assert c.max() <= 1.15 * c.mean(), c.max() / c.mean()
    lens = workloads.structure_only("decode", "page16")["context_lens"]
    c = _prefill_queue_costs(lens, np.full(lens.shape[0], 8, np.int32))
    assert c.max() <= 1.1 * c.mean(), c.max() / c.mean()


def test_mixed_plan_tails_balance_decode_and_prefill_queues():
    """A step with decode rows and chunks: each prefill queue holds one piece
    of the chunk, their flops within 2 % of each other, and each decode
    queue's tail holds prefill pieces that bring the decode queue's work
    (its tiles at the planner's rate of 42 prefill flops per byte of K/V, a
    tile per unit of set-up) plus the tail's flops (and a tile of set-up per
    piece) to at most 10 % over a prefill queue's."""
    import workloads

    st = workloads.structure_only("mixed", "page16")
    lens, ql = st["context_lens"], st["q_lens"]
    hkv, d, nq = 8, 128, 256
    p, image = pkv.plan_host(lens, ql, 32, hkv, d, nq)
    units, qoff, _ = pkv.decode_plan_image(p, image)
    assert p.num_tail_queues == nq and p.num_prefill_queues == 2 * nq
    tile = 42 * 2 * 2 * 16 * hkv * d
    fpp = 4 * (32 // hkv) * d

    def flops(u):
        seq, kb, ke, row0, nrows, pos0 = (int(x) for x in u[:6])
        return sum(max(0, min(ke - 1, pos0 + r) - kb + 1) for r in range(nrows)) * fpp + tile

    main = np.array([sum(flops(u) for u in units[qoff[q]:qoff[q + 1]]) for q in range(nq, 2 * nq)], float)
    assert all(qoff[q + 1] - qoff[q] == 1 for q in range(nq, 2 * nq))
    assert main.max() <= 1.02 * main.min(), (main.max(), main.min())
    both = np.array([sum(((int(u[2]) - int(u[1]) + 15) // 16 + 1) * tile for u in units[qoff[q]:qoff[q + 1]]) +
                     sum(flops(u) for u in units[qoff[2 * nq + q]:qoff[2 * nq + q + 1]]) for q in range(nq)], float)
    assert both.max() <= 1.1 * main.mean(), both.max() / main.mean()
    # every tail piece is a chunk unit
    tails = units[qoff[2 * nq]:qoff[3 * nq]]
    assert len(tails) > 0 and np.all(tails[:, 7] >= 1)


@pytest.mark.parametrize("group,rows", [(4, 4), (1, 16), (8, 2), (2, 8), (4, 3)])
def test_few_row_step_is_planned_as_decode_rows(group, rows):
    """A step whose longest chunk holds at most 16 (row, q head) pairs per kv
    head (a speculative verify step) is cut and placed as decode rows are:
    its decode queues equal the oracle's split-KV plan over the sequences'
    keys, each unit holds all rows of its sequence and every kv head, and a
    cut sequence of several rows merges as a row block with piece c's rows at
    prow0 + c * rows.  Past 16 pairs the chunks are planned as chunk units.""" 
    import workloads

    lens = workloads.structure_only("decode", "page16")["context_lens"]
    hkv, nq = 8, 256
    ql = np.full(lens.shape[0], rows, np.int32)
    ql[::5] = 1  # plain decode rows among them
    p, image = pkv.plan_host(lens, ql, hkv * group, hkv, 128, nq)
    assert p.num_prefill_units == 0 and p.num_prefill_queues == 0 and p.max_q_len == rows
    units, qoff, merges = pkv.decode_plan_image(p, image)
    got = [[(int(u[0]), int(u[1]), int(u[2])) for u in units[qoff[q]:qoff[q + 1]]] for q in range(nq)]
    assert got == split_kv_plan(lens.tolist(), nq, unit_cost=1)
    cu = np.concatenate([[0], np.cumsum(ql)])
    for seq, kb, ke, row0, nrows, pos0, prow, kind in units.tolist():
        assert kind == 0 and nrows == ql[seq] and row0 == cu[seq] and pos0 == lens[seq] - ql[seq]
    for row0, nrows, prow0, parts in merges.tolist():
        seq = int(np.searchsorted(cu, row0, side="right") - 1)
        assert nrows == ql[seq]
        mine = units[units[:, 0] == seq]
        assert sorted(mine[:, 6].tolist()) == [prow0 + c * nrows for c in range(parts)]
    past = np.where(ql > 1, 16 // group + 1, 1).astype(np.int32)
    assert pkv.plan_host(lens, past, hkv * group, hkv, 128, nq)[0].num_prefill_units > 0
