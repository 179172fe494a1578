"""GPU parity of paged_attn_mixed (with this step's write) against the fp64 oracle.

A mixed step packs sequences with several new rows (a prefill chunk over its
cached prefix, causal, bottom-right aligned) and sequences with one row
(decode) into one [T] batch.  Chunk rows run on the matrix-core tile (P is
rounded to bf16 before the P V product), decode rows on the decode unit.
Tolerances as for decode: max-abs 2e-2 for bf16 K/V and 6e-2 for fp8 against
the oracle, and the scale-aware bound of gpu_helpers.check_close.
"""

import numpy as np
import pytest

import workloads
from gpu_helpers import DeviceCase, as_f64, check_close, log, oracle_attention, oracle_caches, to_dev, to_host

pytestmark = pytest.mark.gpu


def _run(case, gpu, num_queues=0, rows=None):
    dc = DeviceCase(case, gpu)
    dc.write()
    plan = dc.plan(num_queues, mixed=True)
    out = as_f64(dc.mixed(plan))
    kr, vr = oracle_caches(case, inplace=True)
    assert np.array_equal(to_host(dc.kc).view(np.uint8), kr.view(np.uint8)), "cache after write differs"
    ref, _ = oracle_attention(case, kr, vr)
    if rows is not None:
        out, ref = out[rows], ref[rows]
    return out, ref, plan


def test_mixed_workload_full_size(gpu):
    """63 decodes (context U[256, 2048]) + one 512-row chunk over 2048 cached
    tokens, 32/8/128 bf16 page 16, default queues (the benchmark's launch)."""
    log("mixed full size")
    case = workloads.make_case("mixed")
    out, ref, plan = _run(case, gpu)
    chunk = case.q_lens > 1
    cu = case.cu_seqlens
    crow = np.concatenate([np.arange(cu[s], cu[s + 1]) for s in np.nonzero(chunk)[0]])
    drow = np.concatenate([np.arange(cu[s], cu[s + 1]) for s in np.nonzero(~chunk)[0]])
    check_close(out[crow], ref[crow], "bf16", f"mixed chunk rows units={plan.desc.num_units}")
    check_close(out[drow], ref[drow], "bf16", "mixed decode rows")


@pytest.mark.parametrize("bs", [1, 3, 4, 16, 32, 48, 64])
@pytest.mark.parametrize("num_queues", [1, 7, 0])
def test_mixed_chunks_and_decodes(gpu, bs, num_queues):
    """Chunks of 2 .. 300 rows (ragged tails of the 32-row blocks and 32-key
    tiles), a chunk that is the whole context, and decodes, on several pages."""
    log(f"mixed bs={bs} queues={num_queues}")
    lens = [40, 1, 300, 77, 129, 700, 33, 2]
    ql = [1, 1, 300, 17, 65, 130, 1, 2]
    case = workloads.build_case(f"mx{bs}", 80 + bs, lens, ql, num_q_heads=16, num_kv_heads=4, head_dim=128,
                                block_size=bs)
    out, ref, _ = _run(case, gpu, num_queues)
    check_close(out, ref, "bf16", f"mixed bs={bs}")


@pytest.mark.parametrize("hq,hkv,d", [(8, 8, 128), (8, 1, 128), (16, 8, 64), (32, 4, 128), (64, 8, 128),
                                      (4, 2, 64)])
def test_mixed_head_shapes(gpu, hq, hkv, d):
    log(f"mixed heads {hq}/{hkv} d={d}")
    lens = [200, 90, 1000, 5]
    ql = [200, 1, 97, 1]
    case = workloads.build_case("mxh", 90, lens, ql, num_q_heads=hq, num_kv_heads=hkv, head_dim=d, block_size=16)
    out, ref, _ = _run(case, gpu, 11)
    check_close(out, ref, "bf16", f"mixed heads {hq}/{hkv} d={d}")


@pytest.mark.parametrize("d", [64, 128])
def test_mixed_fp8_cache(gpu, d):
    """fp8 E4M3 cache: chunk keys are widened to bf16 when staged."""
    lens = [300, 50, 700]
    ql = [120, 1, 33]
    case = workloads.build_case("mx8", 91, lens, ql, num_q_heads=16, num_kv_heads=4, head_dim=d, block_size=16,
                                kv_dtype="fp8")
    out, ref, _ = _run(case, gpu, 5)
    check_close(out, ref, "fp8", f"mixed fp8 d={d}")


@pytest.mark.parametrize("scale", [-0.07, 0.0, 0.3])
def test_mixed_scale_sign_and_zero(gpu, scale):
    """A negative score factor (carried by the sign of q in the chunk tile), a
    zero factor (uniform weights over the visible keys) and a large one."""
    lens = [300, 40, 520]
    ql = [100, 1, 37]
    case = workloads.build_case("mxs", 96, lens, ql, num_q_heads=16, num_kv_heads=4, head_dim=128, block_size=16,
                                scale=scale)
    out, ref, _ = _run(case, gpu, 5)
    check_close(out, ref, "bf16", f"mixed scale={scale}")


def test_mixed_packing_order(gpu):
    """The chunk first or last in [T]: each sequence's rows match the oracle either way."""
    for order in ("chunk-last", "chunk-first"):
        lens = [500, 800, 60, 2000]
        ql = [1, 1, 1, 400]
        if order == "chunk-first":
            lens, ql = lens[::-1], ql[::-1]
        case = workloads.build_case("mxo", 92, lens, ql, num_q_heads=32, num_kv_heads=8, head_dim=128,
                                    block_size=16)
        out, ref, _ = _run(case, gpu, 0)
        check_close(out, ref, "bf16", order)


def test_mixed_decode_only_plan_matches_decode(gpu):
    """A mixed call whose plan has one row per sequence is the decode call: byte-identical."""
    import paged_kv_attention_write_amd as pkv

    lens = [100, 900, 33]
    case = workloads.build_case("mxd", 93, lens, [1, 1, 1], num_q_heads=8, num_kv_heads=2, head_dim=128,
                                block_size=16)
    dc = DeviceCase(case, gpu)
    dc.write()
    plan = dc.plan(5)
    a = to_host(dc.decode(plan))
    b = to_host(dc.mixed(plan))
    assert np.array_equal(a, b)


def test_mixed_invalid_block_id_gives_nan_rows(gpu):
    """A chunk whose table lists a block outside the pool: every row that sees
    that block comes out NaN (rows sharing a unit with them may too); the
    other sequences are unaffected."""
    lens = [300, 50, 90]
    ql = [100, 1, 1]
    case = workloads.build_case("mxbad", 94, lens, ql, num_q_heads=8, num_kv_heads=2, head_dim=128, block_size=16)
    dc = DeviceCase(case, gpu)
    dc.write()
    kr, vr = oracle_caches(case)
    ref, _ = oracle_attention(case, kr, vr)
    tables = case.block_tables.copy()
    tables[0, 15] = case.num_blocks + 7  # keys 240 .. 255
    dc.tables = to_dev(tables, gpu)
    out = as_f64(dc.mixed(dc.plan(4, mixed=True)))
    cu = case.cu_seqlens
    first_seeing = 240 - (lens[0] - ql[0])  # row at position 240
    assert np.all(np.isnan(out[first_seeing:cu[1]]))
    check_close(out[cu[1]:], ref[cu[1]:], "bf16", "neighbours of the bad chunk")


def test_mixed_fp32_chunks_are_unsupported(gpu):
    """The prefill tile is a bf16 product: fp32 q with chunk rows is refused before any launch."""
    import paged_kv_attention_write_amd as pkv

    case = workloads.build_case("mx32", 95, [40, 20], [8, 1], num_q_heads=4, num_kv_heads=2, head_dim=64,
                                block_size=16, q_dtype="f32", kv_dtype="f32")
    dc = DeviceCase(case, gpu)
    dc.write()
    with pytest.raises(pkv.PkvError) as e:
        dc.mixed(dc.plan(2, mixed=True))
    assert e.value.status == pkv._abi.PKV_ERR_UNSUPPORTED


@pytest.mark.parametrize("q_len", [2, 4, 8])
def test_speculative_verify_rows(gpu, q_len):
    """Every sequence brings a few new rows at once (a speculative verify
    step), next to plain decode rows: all of them through the mixed path."""
    log(f"speculative verify q_len={q_len}")
    rng = np.random.default_rng(170 + q_len)
    lens = rng.integers(100, 1500, size=18).astype(np.int32)
    ql = np.full(18, q_len, np.int32)
    ql[[3, 11]] = 1
    case = workloads.build_case(f"spec{q_len}", 170 + q_len, lens.tolist(), ql.tolist(), num_q_heads=32,
                                num_kv_heads=8, head_dim=128, block_size=16)
    out, ref, plan = _run(case, gpu)
    check_close(out, ref, "bf16", f"spec q_len={q_len} units={plan.desc.num_units} merges={plan.desc.num_merges}")


@pytest.mark.parametrize("bs", [16, 3])
def test_cu_seqlens_other_than_the_plan_gives_nan_rows(gpu, bs):
    """cu_seqlens must be the prefix sums of the q_lens the plan was made
    from.  Offsets that differ (here sequence 1 given two rows and sequence
    2 none) turn the rows the plan gives those sequences into NaN, and leave
    the chunk and the last decode row as the oracle has them; a shift of
    every offset turns every row NaN.  Page 16 runs the one-launch mixed
    kernel, page 3 the decode and prefill kernels one after the other."""
    log(f"cu_seqlens mismatch bs={bs}")
    lens, ql = [300, 50, 90, 70], [100, 1, 1, 1]
    case = workloads.build_case("mxcu", 97, lens, ql, num_q_heads=8, num_kv_heads=2, head_dim=128, block_size=bs)
    dc = DeviceCase(case, gpu)
    dc.write()
    kr, vr = oracle_caches(case)
    ref, _ = oracle_attention(case, kr, vr)
    plan = dc.plan(5, mixed=True)
    good = as_f64(dc.mixed(plan))
    check_close(good, ref, "bf16", "matching cu_seqlens")
    assert list(case.cu_seqlens) == [0, 100, 101, 102, 103]
    dc.cu = to_dev(np.array([0, 100, 102, 102, 103], np.int32), gpu)
    out = as_f64(dc.mixed(plan))
    assert np.all(np.isnan(out[100:102]))
    check_close(out[np.r_[0:100, 102]], ref[np.r_[0:100, 102]], "bf16", "rows of the matching sequences")
    dc.cu = to_dev(np.array([1, 101, 102, 103, 104], np.int32), gpu)
    out = as_f64(dc.mixed(plan))
    assert np.all(np.isnan(out))


@pytest.mark.parametrize("bs", [16, 3])
@pytest.mark.parametrize("change", [-1, 1])
def test_stale_plan_length_gives_nan_chunk_rows(gpu, bs, change):
    """A chunk's key ranges and positions come from the plan; a device length
    other than the plan's (a stale plan) turns every row of the chunk into
    NaN, as it does for decode rows, and leaves the other rows unaffected."""
    log(f"stale chunk plan bs={bs} change={change}")
    lens, ql = [700, 60, 1200], [130, 1, 1]
    case = workloads.build_case("mxstale", 98, lens, ql, num_q_heads=16, num_kv_heads=4, head_dim=128,
                                block_size=bs)
    dc = DeviceCase(case, gpu)
    dc.write()
    kr, vr = oracle_caches(case)
    ref, _ = oracle_attention(case, kr, vr)
    plan = dc.plan(6, mixed=True)
    ctx = case.context_lens.copy()
    ctx[0] += change
    dc.ctx = to_dev(ctx, gpu)
    out = as_f64(dc.mixed(plan))
    assert np.all(np.isnan(out[:130]))
    check_close(out[130:], ref[130:], "bf16", "rows of the unchanged sequences")


@pytest.mark.parametrize("lens,ql", [([4000], [33]), ([4000, 3000], [33, 1]), ([4500, 900, 2500], [65, 1, 97])])
def test_single_row_chunk_block_over_a_long_prefix(gpu, lens, ql):
    """Chunks whose last row block holds one row (q_len = 1 mod 32 at 32/8
    heads) over >= 4K keys, at the default queue count: that block is cut into
    pieces and merged as a row block."""
    log(f"single-row chunk block {lens} {ql}")
    case = workloads.build_case("mx1row", 99, lens, ql, num_q_heads=32, num_kv_heads=8, head_dim=128,
                                block_size=16)
    out, ref, plan = _run(case, gpu)
    assert plan.desc.num_block_merges >= 1
    check_close(out, ref, "bf16", f"single-row block merges={plan.desc.num_merges}")
