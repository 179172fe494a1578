"""GPU parity of paged_attn_decode (with its write) against the fp64 oracle.

Tolerances (max-abs error against the oracle): 1e-4 for fp32 K/V, 2e-2 for
bf16 K/V, 6e-2 for an fp8 cache.  Each case prints its name before it runs.
Unused pool slots and table entries past a sequence are poisoned (NaN / -1),
so a stray read shows up as NaN.
"""

import numpy as np
import pytest

import workloads
from gpu_helpers import (TOL, DeviceCase, as_f64, check_close, log, max_err, oracle_attention, oracle_caches,
                         to_dev, to_host)

pytestmark = pytest.mark.gpu


def _run(case, gpu, num_queues=0, seqs=None):
    dc = DeviceCase(case, gpu)
    dc.write()
    plan = dc.plan(num_queues)
    out = as_f64(dc.decode(plan))
    kr, vr = oracle_caches(case, inplace=True)  # the device holds its own copy
    assert np.array_equal(to_host(dc.kc).view(np.uint8), kr.view(np.uint8)), "cache after write differs"
    ref, _ = oracle_attention(case, kr, vr, seqs=seqs)
    rows = np.arange(case.num_tokens) if seqs is None else np.asarray(seqs)
    return out[rows], ref[rows], plan, dc


@pytest.mark.parametrize("num_queues", [0, 1, 3, 4, 12, 1000])
def test_tiny_fp32(gpu, num_queues):
    log(f"tiny fp32 queues={num_queues}")
    case = workloads.make_case("tiny")
    got, ref, plan, _ = _run(case, gpu, num_queues)
    check_close(got, ref, "f32", f"tiny merges={plan.desc.num_merges}")


def test_decode_workload_full_size(gpu):
    """64 x U[512, 4096] at 32/8/128 bf16, default queues (the benchmark's launch)."""
    log("decode full size")
    case = workloads.make_case("decode")
    got, ref, plan, _ = _run(case, gpu)
    check_close(got, ref, "bf16", f"decode units={plan.desc.num_units} merges={plan.desc.num_merges}")


@pytest.mark.parametrize("bs", [1, 2, 3, 4, 7, 8, 16, 32, 48, 64])
@pytest.mark.parametrize("num_queues", [1, 9, 0])
def test_block_sizes(gpu, bs, num_queues):
    log(f"block size {bs} queues={num_queues}")
    lens = [1, 17, 100, 250, 513, 64]
    case = workloads.build_case(f"bs{bs}", 40 + bs, lens, [1] * len(lens), num_q_heads=16, num_kv_heads=4,
                                head_dim=128, block_size=bs)
    got, ref, _, _ = _run(case, gpu, num_queues)
    check_close(got, ref, "bf16", f"bs={bs}")


@pytest.mark.parametrize("bs", [16, 1, 4])
@pytest.mark.parametrize("hq,hkv,d", [(8, 8, 128), (8, 1, 128), (16, 8, 64), (32, 4, 128), (64, 8, 128),
                                      (4, 2, 64)])
def test_head_shapes(gpu, hq, hkv, d, bs):
    """Every group size and head_dim on each page kind: whole 16-token tiles,
    one-token pages, groups of 4 tokens."""
    log(f"heads {hq}/{hkv} d={d} bs={bs}")
    lens = [5, 300, 77, 1024]
    case = workloads.build_case("heads", 50, lens, [1] * 4, num_q_heads=hq, num_kv_heads=hkv, head_dim=d,
                                block_size=bs)
    got, ref, _, _ = _run(case, gpu, 7)
    check_close(got, ref, "bf16", f"heads {hq}/{hkv} d={d} bs={bs}")


def test_permutation_and_sharing_are_bit_identical(gpu):
    """Same logical K/V under another table permutation, and with a shared prefix
    against private copies: byte-identical outputs (arithmetic follows logical
    positions only; the plan follows lengths only)."""
    import paged_kv_attention_write_amd as pkv
    from paging import page_out

    rng = np.random.default_rng(8)
    hkv, d = 4, 128
    prefix = workloads.to_storage(rng.standard_normal((96, hkv, d)).astype(np.float32), "bf16")
    prefv = workloads.to_storage(rng.standard_normal((96, hkv, d)).astype(np.float32), "bf16")
    K, V = [], []
    for n in (40, 400, 17, 96):
        K.append(np.concatenate([prefix, workloads.to_storage(rng.standard_normal((n, hkv, d)).astype(np.float32), "bf16")]))
        V.append(np.concatenate([prefv, workloads.to_storage(rng.standard_normal((n, hkv, d)).astype(np.float32), "bf16")]))
    lens = np.array([k.shape[0] for k in K], np.int32)
    q = workloads.to_storage(rng.standard_normal((4, 16, d)).astype(np.float32), "bf16")
    qd = to_dev(q, gpu)
    plan = pkv.Plan(lens, num_q_heads=16, num_kv_heads=hkv, head_dim=d, device=gpu, num_queues=11)
    outs = []
    for layout in (dict(perm_seed=None), dict(perm_seed=3, extra_blocks=9), dict(perm_seed=5, shared_prefix_blocks=6)):
        kp, vp, tab = page_out(K, V, 16, **layout)
        o = to_dev(np.zeros_like(q), gpu)
        pkv.paged_attn_decode(o, qd, to_dev(kp, gpu), to_dev(vp, gpu), to_dev(tab, gpu), to_dev(lens, gpu),
                              0.08838834764831845, plan)
        outs.append(to_host(o))
    assert np.array_equal(outs[0], outs[1]) and np.array_equal(outs[0], outs[2])


def test_neighbour_independence(gpu):
    """A sequence batched with others gets its oracle answer whatever the others are."""
    base = [300, 1000, 20]
    for extra in ([], [4000, 4000], [1] * 30):
        lens = base + extra
        case = workloads.build_case("nb", 60, lens, [1] * len(lens), num_q_heads=8, num_kv_heads=2, head_dim=128,
                                    block_size=16)
        got, ref, _, _ = _run(case, gpu, 0)
        check_close(got, ref, "bf16", f"neighbours {len(extra)}")


def test_invalid_block_id_gives_nan_rows_only_for_that_sequence(gpu):
    """A table entry outside the pool is never dereferenced; its sequence's rows
    come out NaN and the other sequences are unaffected."""
    import paged_kv_attention_write_amd as pkv

    case = workloads.build_case("badid", 61, [50, 200, 33], [1, 1, 1], num_q_heads=8, num_kv_heads=2, head_dim=128,
                                block_size=16)
    dc = DeviceCase(case, gpu)
    dc.write()
    kr, vr = oracle_caches(case)
    ref, _ = oracle_attention(case, kr, vr)
    tables = case.block_tables.copy()
    tables[1, 5] = case.num_blocks + 1000
    dc.tables = to_dev(tables, gpu)
    out = as_f64(dc.decode(dc.plan(5)))
    assert np.all(np.isnan(out[1]))
    check_close(out[[0, 2]], ref[[0, 2]], "bf16", "neighbours of the bad sequence")


@pytest.mark.parametrize("changed", [0, 1])
def test_stale_plan_length_gives_nan_rows(gpu, changed):
    """Decode rows take their key ranges from the plan; a device length that
    differs from the length the plan was made from turns that row into NaN
    (sequence 0 is one piece, sequence 1 is cut over several queues) and
    leaves the other rows unaffected."""
    log(f"stale plan, sequence {changed}")
    case = workloads.build_case("stale", 62, [50, 900, 33], [1, 1, 1], num_q_heads=8, num_kv_heads=2,
                                head_dim=128, block_size=16)
    dc = DeviceCase(case, gpu)
    dc.write()
    kr, vr = oracle_caches(case)
    ref, _ = oracle_attention(case, kr, vr)
    plan = dc.plan(5)  # from the case's own lengths
    import paged_kv_attention_write_amd as pkv

    hp, image = pkv.plan_host(case.context_lens, None, 8, 2, 128, 5)
    units, _, _ = pkv.decode_plan_image(hp, image)
    pieces = [int((units[:, 0] == s).sum()) for s in range(3)]
    assert pieces[0] == 1 and pieces[1] > 1, pieces  # sequence 0 whole, sequence 1 cut
    ctx = case.context_lens.copy()
    ctx[changed] -= 1
    dc.ctx = to_dev(ctx, gpu)
    out = as_f64(dc.decode(plan))
    assert np.all(np.isnan(out[changed]))
    others = [s for s in range(3) if s != changed]
    check_close(out[others], ref[others], "bf16", "rows of the unchanged sequences")


@pytest.mark.parametrize("layout", ["page1", "page16", "contig"])
def test_long_context_layouts_sampled(gpu, layout):
    """16 x 32768 at page 1 (shuffled), page 16 (shuffled) or a contiguous slab;
    3 sampled sequences against the oracle."""
    log(f"long {layout}")
    case = workloads.make_case("long", layout)
    got, ref, plan, _ = _run(case, gpu, seqs=[0, 2, 7, 9, 15])
    check_close(got, ref, "bf16", f"long {layout} units={plan.desc.num_units}")


def test_fp8_prefix_shared_full_size(gpu):
    """128 sequences sharing 256 blocks, fp8 cache filled by the quantising write."""
    log("fp8 prefix")
    case = workloads.make_case("fp8prefix")
    got, ref, plan, _ = _run(case, gpu, seqs=list(range(0, 128, 9)))
    check_close(got, ref, "fp8", "fp8 prefix")


@pytest.mark.parametrize("bs", [16, 1, 4])
@pytest.mark.parametrize("d", [64, 128])
def test_fp8_small(gpu, d, bs):
    case = workloads.build_case("fp8s", 62, [3, 70, 500, 16], [1] * 4, num_q_heads=16, num_kv_heads=4, head_dim=d,
                                block_size=bs, kv_dtype="fp8")
    got, ref, _, _ = _run(case, gpu, 6)
    check_close(got, ref, "fp8", f"fp8 d={d} bs={bs}")


def test_q_token_stride(gpu):
    """q taken from a fused projection output with a token stride."""
    import torch

    import paged_kv_attention_write_amd as pkv

    case = workloads.build_case("qs", 63, [40, 300], [1, 1], num_q_heads=8, num_kv_heads=2, head_dim=128,
                                block_size=16)
    dc = DeviceCase(case, gpu)
    dc.write()
    wide = torch.zeros((2, 12 * 128), dtype=torch.bfloat16, device=gpu)
    wide[:, :8 * 128] = dc.q.view(2, -1)
    qv = wide[:, :8 * 128].view(2, 8, 128)
    assert not qv.is_contiguous()
    out = torch.empty((2, 8, 128), dtype=torch.bfloat16, device=gpu)
    pkv.paged_attn_decode(out, qv, dc.kc, dc.vc, dc.tables, dc.ctx, case.scale, dc.plan(3))
    kr, vr = oracle_caches(case)
    ref, _ = oracle_attention(case, kr, vr)
    check_close(as_f64(out), ref, "bf16", "q stride")


def test_plan_reused_across_layers(gpu):
    """One plan, several layers with their own pools and queries (the pages' step)."""
    lens = [100, 900, 2000]
    plan = None
    for layer in range(3):
        case = workloads.build_case("layer", 70 + layer, lens, [1, 1, 1], num_q_heads=8, num_kv_heads=2,
                                    head_dim=128, block_size=16)
        dc = DeviceCase(case, gpu)
        dc.write()
        if plan is None:
            plan = dc.plan(4)
        got = as_f64(dc.decode(plan))
        kr, vr = oracle_caches(case)
        ref, _ = oracle_attention(case, kr, vr)
        check_close(got, ref, "bf16", f"layer {layer}")


@pytest.mark.parametrize("mix", workloads.SKEW_MIXES)
@pytest.mark.parametrize("batch", [4, 16, 64])
def test_skew_mixes(gpu, mix, batch):
    """The load-balance study's length mixes (equal total tokens: uniform, one
    sequence holding half, Pareto-tailed) at a reduced total of 24576 tokens;
    default queues split the long sequences into many pieces."""
    log(f"skew {mix} batch={batch}")
    lens = workloads.skew_lengths(mix, batch, total=24576)
    case = workloads.build_case(f"skew-{mix}-{batch}", 60 + batch, lens, [1] * batch, num_q_heads=32,
                                num_kv_heads=8, head_dim=128, block_size=16)
    got, ref, plan, _ = _run(case, gpu)
    check_close(got, ref, "bf16", f"skew {mix} B={batch} units={plan.desc.num_units} merges={plan.desc.num_merges}")


def test_invalid_block_id_in_a_wide_merge(gpu):
    """A long sequence cut into many pieces (a wide merge record, its parts
    split over several waves per head) with one table entry outside the pool:
    its row comes out NaN, the short neighbours are unaffected."""
    import paged_kv_attention_write_amd as pkv

    case = workloads.build_case("badwide", 62, [40, 3000, 70], [1, 1, 1], num_q_heads=8, num_kv_heads=2,
                                head_dim=128, block_size=16)
    dc = DeviceCase(case, gpu)
    dc.write()
    kr, vr = oracle_caches(case)
    ref, _ = oracle_attention(case, kr, vr)
    plan = dc.plan(24)
    assert plan.desc.num_wide_merges >= 1
    out = as_f64(dc.decode(plan))
    check_close(out, ref, "bf16", f"wide merge wide={plan.desc.num_wide_merges}")
    tables = case.block_tables.copy()
    tables[1, 100] = case.num_blocks + 7
    dc.tables = to_dev(tables, gpu)
    out = as_f64(dc.decode(plan))
    assert np.all(np.isnan(out[1]))
    check_close(out[[0, 2]], ref[[0, 2]], "bf16", "neighbours of the bad wide row")
