"""GPU parity of steps that hold prefill chunks and no decode row, against the
fp64 oracle.

Such a step runs the prefill kernel alone ("nanoserve", packed batches and
chunked prefill: the chunks of a step go to a prefill path).  For bf16 K/V at
D = 128 on pages of a power of two >= 16 tokens its form follows the longest
chunk: units of at least 64 (row, q head) pairs take the wide form (4 waves
of 32 pairs, each K and V operand read from LDS feeding two matrix
products), others the 8-wave ring; other caches and pages take the 8-wave
register-staged form.  A step whose chunks all hold at most 16 pairs per kv
head (a speculative verify step) is planned as decode rows are and runs the
few-row kernel: one wave per kv head of a unit, K straight into the matrix
operands, V through the wave's own LDS tile.  Cases cover every group size, ragged chunks (row
blocks and 32-key tiles cut short), chunks that are the whole context, the
soft-cap and window variants, score factors of either sign, stale plans, few
rows beside decode rows, and the 512-row chunk of the mixed workload and the
speculative verify workload at their full sizes.  Tolerances as for the
mixed step.
"""

import numpy as np
import pytest

import oracle
import workloads
from gpu_helpers import DeviceCase, as_f64, check_close, log, oracle_attention, oracle_caches, to_dev

pytestmark = pytest.mark.gpu

LENS = [300, 1000, 77, 2100, 45]
QL = [300, 129, 40, 513, 45]


def _run(case, gpu, num_queues=0, soft_cap=0.0, window=0, few=False):
    import paged_kv_attention_write_amd as pkv

    dc = DeviceCase(case, gpu)
    dc.write()
    plan = pkv.Plan(case.context_lens, case.q_lens, num_q_heads=case.num_q_heads, num_kv_heads=case.num_kv_heads,
                    head_dim=case.head_dim, device=gpu, num_queues=num_queues, soft_cap=soft_cap, window=window)
    if few:  # every sequence's rows in decode-queue units
        assert plan.desc.num_prefill_units == 0 and plan.desc.max_q_len > 1, "a few-row step"
    else:
        assert plan.desc.num_units == plan.desc.num_prefill_units, "chunks only"
    out = as_f64(dc.mixed(plan))
    kr, vr = oracle_caches(case)
    ref, _ = oracle.paged_attention(case.q, case.q_dtype, kr, vr, case.kv_dtype, case.block_tables,
                                    case.context_lens, case.cu_seqlens, case.scale, case.k_scale, case.v_scale,
                                    soft_cap=soft_cap, window=window)
    return out, ref, plan


@pytest.mark.parametrize("hq,hkv", [(8, 8), (16, 8), (32, 8), (64, 8)])
@pytest.mark.parametrize("bs", [16, 64])
@pytest.mark.parametrize("num_queues", [0, 7])
def test_chunk_only_groups_and_pages(gpu, hq, hkv, bs, num_queues):
    log(f"chunks only hq={hq} hkv={hkv} bs={bs} queues={num_queues}")
    case = workloads.build_case(f"pf{hq}", 300 + hq + bs, LENS, QL, num_q_heads=hq, num_kv_heads=hkv,
                                head_dim=128, block_size=bs)
    out, ref, plan = _run(case, gpu, num_queues)
    check_close(out, ref, "bf16", f"chunks only G={hq // hkv} bs={bs} units={plan.desc.num_units}")


@pytest.mark.parametrize("bs,kv_dtype,d", [(3, "bf16", 128), (48, "bf16", 128), (16, "fp8", 128),
                                           (16, "bf16", 64), (32, "fp8", 64)])
def test_chunk_only_register_path(gpu, bs, kv_dtype, d):
    """Pages that are not a power of two >= 16, fp8 caches and D = 64 stage
    K/V through registers (8 waves of 16 pairs)."""
    log(f"chunks only register path bs={bs} {kv_dtype} d={d}")
    case = workloads.build_case("pfr", 320 + bs + d, LENS, QL, num_q_heads=32, num_kv_heads=8, head_dim=d,
                                block_size=bs, kv_dtype=kv_dtype)
    out, ref, _ = _run(case, gpu, 0)
    check_close(out, ref, kv_dtype, f"chunks only bs={bs} {kv_dtype} d={d}")


@pytest.mark.parametrize("bs", [16, 32])
@pytest.mark.parametrize("soft_cap,window", [(0.0, 1), (0.0, 40), (0.0, 300), (10.0, 0), (10.0, 129)])
def test_chunk_only_variants(gpu, bs, soft_cap, window):
    log(f"chunks only variants bs={bs} cap={soft_cap} W={window}")
    case = workloads.build_case("pfv", 340 + bs, LENS, QL, num_q_heads=32, num_kv_heads=8, head_dim=128,
                                block_size=bs, scale=0.3)
    out, ref, _ = _run(case, gpu, 13, soft_cap=soft_cap, window=window)
    check_close(out, ref, "bf16", f"chunks only bs={bs} cap={soft_cap} W={window}")


@pytest.mark.parametrize("scale", [-0.07, 0.0, 0.3])
def test_chunk_only_scale_sign_and_zero(gpu, scale):
    case = workloads.build_case("pfs", 350, LENS, QL, num_q_heads=32, num_kv_heads=8, head_dim=128, block_size=16,
                                scale=scale)
    out, ref, _ = _run(case, gpu, 0)
    check_close(out, ref, "bf16", f"chunks only scale={scale}")


def test_chunk_only_full_size(gpu):
    """The 512-row chunk of the mixed workload alone: rows at positions
    2048 .. 2559 over 2560 keys, 32/8/128 bf16, page 16, default queues (the
    launch the benchmark times for this chunk)."""
    log("chunk 512 over 2560 keys")
    case = workloads.build_case("pf512", 360, [2560], [512], num_q_heads=32, num_kv_heads=8, head_dim=128,
                                block_size=16)
    out, ref, plan = _run(case, gpu, 0)
    check_close(out, ref, "bf16", f"chunk 512 units={plan.desc.num_units} merges={plan.desc.num_merges}")


@pytest.mark.parametrize("change", [-1, 1])
def test_chunk_only_stale_plan_gives_nan_rows(gpu, change):
    """A device length other than the plan's turns that chunk's rows into NaN
    and leaves the other chunks as the oracle has them."""
    case = workloads.build_case("pfst", 370, [700, 300], [130, 64], num_q_heads=32, num_kv_heads=8, head_dim=128,
                                block_size=16)
    dc = DeviceCase(case, gpu)
    dc.write()
    kr, vr = oracle_caches(case)
    ref, _ = oracle_attention(case, kr, vr)
    plan = dc.plan(0, mixed=True)
    ctx = case.context_lens.copy()
    ctx[0] += change
    dc.ctx = to_dev(ctx, gpu)
    out = as_f64(dc.mixed(plan))
    assert np.all(np.isnan(out[:130]))
    check_close(out[130:], ref[130:], "bf16", "rows of the unchanged chunk")


def _few_rows(seed, n, max_q, min_len=100, max_len=3000, decode_every=0):
    """n sequences with 2 .. max_q new rows each (a speculative verify step),
    every decode_every-th one a plain decode row instead."""
    rng = np.random.default_rng(seed)
    lens = rng.integers(min_len, max_len, size=n).astype(np.int32)
    ql = rng.integers(2, max_q + 1, size=n).astype(np.int32)
    ql[0] = max_q
    if decode_every:
        ql[1::decode_every] = 1
    return lens.tolist(), ql.tolist()


@pytest.mark.parametrize("hq,hkv,max_q", [(8, 8, 16), (8, 8, 5), (16, 8, 8), (32, 8, 4), (32, 8, 3), (64, 8, 2),
                                          (16, 4, 4)])
@pytest.mark.parametrize("bs", [16, 64])
def test_few_row_units(gpu, hq, hkv, max_q, bs):
    """Units of at most 16 (row, q head) pairs: the workgroup's waves take
    turns over the unit's tiles and combine their states at its end."""
    log(f"few rows hq={hq} hkv={hkv} max_q={max_q} bs={bs}")
    lens, ql = _few_rows(400 + hq + max_q + bs, 24, max_q)
    case = workloads.build_case("pffr", 400 + hq + max_q + bs, lens, ql, num_q_heads=hq, num_kv_heads=hkv,
                                head_dim=128, block_size=bs)
    out, ref, plan = _run(case, gpu, 0, few=True)
    check_close(out, ref, "bf16", f"few rows G={hq // hkv} q<={max_q} bs={bs} units={plan.desc.num_units}")


@pytest.mark.parametrize("lens,ql", [([2, 31, 32, 33, 63, 64, 65, 127, 129, 200], [2, 3, 4, 2, 3, 4, 2, 3, 4, 2]),
                                     ([4, 4, 4], [4, 3, 2]), ([5000, 17], [4, 4])])
def test_few_row_short_and_ragged(gpu, lens, ql):
    """Units shorter than one tile per wave, ragged last tiles, chunks that
    are the whole context, at the default queue count and at one queue
    (32/8 heads: at most 4 rows per sequence)."""
    for nq in (0, 1):
        case = workloads.build_case("pffs", 450 + len(lens), lens, ql, num_q_heads=32, num_kv_heads=8,
                                    head_dim=128, block_size=16)
        dc = DeviceCase(case, gpu)
        dc.write()
        plan = dc.plan(nq, mixed=True)
        out = as_f64(dc.mixed(plan))
        kr, vr = oracle_caches(case)
        ref, _ = oracle_attention(case, kr, vr)
        check_close(out, ref, "bf16", f"few rows short lens={lens} queues={nq}")


@pytest.mark.parametrize("hq,hkv", [(8, 8), (64, 8), (32, 8), (8, 2)])
def test_few_row_units_beside_decode_rows(gpu, hq, hkv):
    """Speculative rows next to plain decode rows: the whole step runs the
    few-row kernel (a decode row is a unit of one row); 2 kv heads leave six
    of its eight waves idle."""
    g = hq // hkv
    lens, ql = _few_rows(470 + hq, 20, max(2, 16 // g), decode_every=4)
    case = workloads.build_case("pffd", 470 + hq, lens, ql, num_q_heads=hq, num_kv_heads=hkv, head_dim=128,
                                block_size=16)
    dc = DeviceCase(case, gpu)
    dc.write()
    plan = dc.plan(0, mixed=True)
    out = as_f64(dc.mixed(plan))
    kr, vr = oracle_caches(case)
    ref, _ = oracle_attention(case, kr, vr)
    check_close(out, ref, "bf16", f"few rows beside decodes G={g}")


@pytest.mark.parametrize("bs,kv_dtype,d,hkv", [(48, "bf16", 128, 8), (3, "bf16", 128, 8), (16, "fp8", 128, 8),
                                               (16, "bf16", 64, 8), (7, "fp8", 64, 4), (16, "bf16", 128, 16)])
def test_few_row_register_path(gpu, bs, kv_dtype, d, hkv):
    """Few-row steps the few-row kernel does not serve (pages that are not a
    power of two >= 16, fp8 caches, D = 64) run the register-staged prefill
    tile over the decode queues, one kv head of a unit after the other; 16
    kv heads take the few-row kernel with two heads per wave."""
    lens, ql = _few_rows(480 + bs + d, 16, 4)
    case = workloads.build_case("pffr2", 480 + bs + d, lens, ql, num_q_heads=4 * hkv, num_kv_heads=hkv,
                                head_dim=d, block_size=bs, kv_dtype=kv_dtype)
    out, ref, _ = _run(case, gpu, 0, few=True)
    check_close(out, ref, kv_dtype, f"few rows bs={bs} {kv_dtype} d={d} hkv={hkv}")


@pytest.mark.parametrize("soft_cap,window", [(0.0, 1), (0.0, 40), (0.0, 300), (10.0, 0), (10.0, 129)])
def test_few_row_variants(gpu, soft_cap, window):
    lens, ql = _few_rows(490, 16, 4)
    case = workloads.build_case("pffv", 490, lens, ql, num_q_heads=32, num_kv_heads=8, head_dim=128, block_size=16,
                                scale=0.3)
    out, ref, _ = _run(case, gpu, 0, soft_cap=soft_cap, window=window, few=True)
    check_close(out, ref, "bf16", f"few rows cap={soft_cap} W={window}")


def test_few_row_full_size(gpu):
    """The speculative verify workload at its full size: 64 sequences of
    U[512, 4096] keys with 4 new rows each, 32/8/128 bf16, page 16, default
    queues (the launch the benchmark times)."""
    lens = workloads.structure_only("decode", "page16")["context_lens"]
    case = workloads.build_case("pffull", 495, lens.tolist(), [4] * len(lens), num_q_heads=32, num_kv_heads=8,
                                head_dim=128, block_size=16)
    out, ref, plan = _run(case, gpu, 0, few=True)
    check_close(out, ref, "bf16", f"specverify full size units={plan.desc.num_units}")


@pytest.mark.parametrize("change", [-1, 1])
def test_few_row_stale_plan_gives_nan_rows(gpu, change):
    case = workloads.build_case("pffst", 497, [700, 300, 1500], [4, 3, 4], num_q_heads=32, num_kv_heads=8,
                                head_dim=128, block_size=16)
    dc = DeviceCase(case, gpu)
    dc.write()
    kr, vr = oracle_caches(case)
    ref, _ = oracle_attention(case, kr, vr)
    plan = dc.plan(0, mixed=True)
    ctx = case.context_lens.copy()
    ctx[1] += change
    dc.ctx = to_dev(ctx, gpu)
    out = as_f64(dc.mixed(plan))
    assert np.all(np.isnan(out[4:7]))
    check_close(out[np.r_[0:4, 7:11]], ref[np.r_[0:4, 7:11]], "bf16", "rows of the unchanged sequences")
