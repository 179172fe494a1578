"""GPU parity of the attention variants a plan can carry, the logit soft-cap
(scores through c * tanh(s / c)) and the sliding window (a row at position p
sees keys p - W < j <= p), against the fp64 oracle's variants.

"How Easy Is It to Start Serving LLMs?", Phase 4 §2 names soft-capping and
sliding windows among the attention variants one kernel template serves;
here they are run-time switches of the same decode, prefill, mixed and merge
kernels, so every path is checked: whole-tile pages (the direct-to-LDS
prefill ring and the one-launch mixed kernel), odd page sizes (the register
path, per-token page loads), fp8 and fp32 caches, head dims 64 and 128,
every group size, split rows merged from many pieces, and windows that end
inside a tile, on a tile edge, inside one page, or past the whole context.
"""

import numpy as np
import pytest

import oracle
import workloads
from gpu_helpers import DeviceCase, as_f64, check_close, log, oracle_caches, to_dev

pytestmark = pytest.mark.gpu


def _plan(case, gpu, mixed, soft_cap, window, num_queues=0, capacity=None):
    import paged_kv_attention_write_amd as pkv

    return pkv.Plan(case.context_lens, case.q_lens if mixed else None, num_q_heads=case.num_q_heads,
                    num_kv_heads=case.num_kv_heads, head_dim=case.head_dim, device=gpu, num_queues=num_queues,
                    soft_cap=soft_cap, window=window, capacity=capacity)


def _run(case, gpu, mixed, soft_cap=0.0, window=0, num_queues=0):
    import torch

    dc = DeviceCase(case, gpu)
    dc.write()
    plan = _plan(case, gpu, mixed, soft_cap, window, num_queues)
    assert plan.desc.window_left == window
    out = dc.mixed(plan) if mixed else dc.decode(plan)
    torch.cuda.synchronize()
    kr, vr = oracle_caches(case)
    ref, _ = oracle.paged_attention(case.q, case.q_dtype, kr, vr, case.kv_dtype, case.block_tables,
                                    case.context_lens, case.cu_seqlens, case.scale, case.k_scale, case.v_scale,
                                    soft_cap=soft_cap, window=window)
    return as_f64(out), ref, plan


DECODE_LENS = [1, 15, 16, 17, 100, 250, 513, 64, 2000, 4500]


@pytest.mark.parametrize("soft_cap,scale", [(1.0, 0.4), (5.0, 0.4), (30.0, 1.0), (50.0, None)])
def test_soft_cap_decode(gpu, soft_cap, scale):
    """Scores well past the cap (scale 0.4 to 1 on unit-variance q and k
    gives |s| up to ~20-40) saturate; the split rows merge capped pieces."""
    log(f"soft-cap decode c={soft_cap} scale={scale}")
    case = workloads.build_case("cap", 150, DECODE_LENS, [1] * len(DECODE_LENS), num_q_heads=32, num_kv_heads=8,
                                head_dim=128, block_size=16, scale=scale)
    got, ref, plan = _run(case, gpu, mixed=False, soft_cap=soft_cap, num_queues=23)
    assert plan.desc.num_merges > 0
    check_close(got, ref, "bf16", f"soft-cap {soft_cap}")


@pytest.mark.parametrize("window", [1, 15, 16, 17, 100, 1000, 4499, 4500, 10000])
def test_window_decode(gpu, window):
    log(f"window decode W={window}")
    case = workloads.build_case("win", 151, DECODE_LENS, [1] * len(DECODE_LENS), num_q_heads=32, num_kv_heads=8,
                                head_dim=128, block_size=16)
    got, ref, _ = _run(case, gpu, mixed=False, window=window, num_queues=23)
    check_close(got, ref, "bf16", f"window {window}")


@pytest.mark.parametrize("bs", [1, 3, 4, 32, 48, 64])
@pytest.mark.parametrize("hq,hkv,d", [(16, 4, 128), (8, 8, 64), (16, 2, 64)])
def test_variants_decode_pages_and_groups(gpu, bs, hq, hkv, d):
    log(f"variants decode bs={bs} hq={hq} hkv={hkv} d={d}")
    lens = [1, 17, 100, 250, 513, 64, 2000]
    case = workloads.build_case(f"vpg{bs}", 152 + bs, lens, [1] * len(lens), num_q_heads=hq, num_kv_heads=hkv,
                                head_dim=d, block_size=bs, scale=0.3)
    got, ref, _ = _run(case, gpu, mixed=False, soft_cap=8.0, window=77, num_queues=9)
    check_close(got, ref, "bf16", f"cap 8 window 77 bs={bs}")


@pytest.mark.parametrize("q_dtype,kv_dtype,tol", [("f32", "f32", "f32"), ("bf16", "fp8", "fp8")])
def test_variants_decode_dtypes(gpu, q_dtype, kv_dtype, tol):
    log(f"variants decode {q_dtype}/{kv_dtype}")
    lens = [1, 17, 100, 250, 513, 64, 2000]
    case = workloads.build_case(f"vdt{kv_dtype}", 160, lens, [1] * len(lens), num_q_heads=16, num_kv_heads=4,
                                head_dim=128, block_size=16, q_dtype=q_dtype, kv_dtype=kv_dtype, scale=0.3)
    got, ref, _ = _run(case, gpu, mixed=False, soft_cap=6.0, window=300, num_queues=9)
    check_close(got, ref, tol, f"cap 6 window 300 {q_dtype}/{kv_dtype}")


MIXED_LENS = [700, 1300, 2560, 130, 900, 45, 3000, 260]
MIXED_Q = [1, 1, 512, 65, 1, 45, 4, 1]


@pytest.mark.parametrize("bs", [16, 32, 3, 48, 64])
@pytest.mark.parametrize("soft_cap,window", [(0.0, 1), (0.0, 64), (0.0, 300), (0.0, 2000), (10.0, 0), (10.0, 129)])
def test_variants_mixed(gpu, bs, soft_cap, window):
    """Chunks, a whole-prompt prefill (45 of 45), a speculative-verify row
    block (4 rows) and decode rows in one step; page 16/32 take the ring
    prefill and the one-launch mixed kernel, page 3 the register path."""
    log(f"variants mixed bs={bs} cap={soft_cap} W={window}")
    case = workloads.build_case(f"vmx{bs}", 170 + bs, MIXED_LENS, MIXED_Q, num_q_heads=32, num_kv_heads=8,
                                head_dim=128, block_size=bs, scale=0.3)
    got, ref, _ = _run(case, gpu, mixed=True, soft_cap=soft_cap, window=window, num_queues=17)
    check_close(got, ref, "bf16", f"mixed bs={bs} cap={soft_cap} W={window}")


@pytest.mark.parametrize("hq,hkv,d", [(16, 16, 128), (16, 8, 64), (32, 4, 64), (64, 8, 128)])
def test_variants_mixed_groups(gpu, hq, hkv, d):
    log(f"variants mixed hq={hq} hkv={hkv} d={d}")
    case = workloads.build_case("vmg", 180 + hq + d, MIXED_LENS, MIXED_Q, num_q_heads=hq, num_kv_heads=hkv,
                                head_dim=d, block_size=16, scale=0.3)
    got, ref, _ = _run(case, gpu, mixed=True, soft_cap=12.0, window=200, num_queues=17)
    check_close(got, ref, "bf16", f"mixed cap 12 W 200 hq={hq} hkv={hkv} d={d}")


def test_variants_mixed_fp8(gpu):
    log("variants mixed fp8")
    case = workloads.build_case("vmf", 190, MIXED_LENS, MIXED_Q, num_q_heads=32, num_kv_heads=8, head_dim=128,
                                block_size=16, kv_dtype="fp8", scale=0.3)
    got, ref, _ = _run(case, gpu, mixed=True, soft_cap=7.0, window=450, num_queues=17)
    check_close(got, ref, "fp8", "mixed fp8 cap 7 W 450")


def test_variants_decode_full_size(gpu):
    """The 64-sequence decode batch (lengths 512-4096, 32 q / 8 kv heads,
    D 128, page 16) with a 1024-key window and a soft-cap of 50."""
    log("variants decode full size")
    case = workloads.make_case("decode")
    got, ref, _ = _run(case, gpu, mixed=False, soft_cap=50.0, window=1024)
    check_close(got, ref, "bf16", "decode cap 50 W 1024")


def test_variant_capacity_plan_matches_compact_plan(gpu):
    """A variant plan laid out at a capacity (for captured steps) computes
    the same bits as the compact variant plan."""
    import torch

    log("variant capacity plan")
    case = workloads.build_case("vcap", 195, MIXED_LENS, MIXED_Q, num_q_heads=32, num_kv_heads=8, head_dim=128,
                                block_size=16, scale=0.3)
    dc = DeviceCase(case, gpu)
    dc.write()
    a = dc.mixed(_plan(case, gpu, True, 9.0, 333, 17))
    b = dc.mixed(_plan(case, gpu, True, 9.0, 333, 17, capacity=(16, 4096)))
    torch.cuda.synchronize()
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))


def test_no_variant_is_the_plain_call(gpu):
    """soft_cap 0 and a window past every context give the plain plan's bits."""
    import torch

    log("variant off equals plain")
    case = workloads.build_case("voff", 196, MIXED_LENS, MIXED_Q, num_q_heads=32, num_kv_heads=8, head_dim=128,
                                block_size=16, scale=0.3)
    dc = DeviceCase(case, gpu)
    dc.write()
    plain = dc.mixed(dc.plan(17, mixed=True))
    wide = dc.mixed(_plan(case, gpu, True, 0.0, 10 ** 6, 17))
    torch.cuda.synchronize()
    assert torch.equal(plain.view(torch.int16), wide.view(torch.int16))


def test_variants_through_csr_tables(gpu):
    """The CSR entry points with a variant plan give the dense calls' bits."""
    import torch
    import paged_kv_attention_write_amd as pkv

    log("variants through CSR tables")
    case = workloads.build_case("vcsr", 197, MIXED_LENS, MIXED_Q, num_q_heads=32, num_kv_heads=8, head_dim=128,
                                block_size=16, scale=0.3)
    dc = DeviceCase(case, gpu)
    dc.write()
    plan = _plan(case, gpu, True, 11.0, 250, 17)
    dense = dc.mixed(plan)
    rows = [case.block_tables[s, :-(-int(n) // 16)] for s, n in enumerate(case.context_lens)]
    indptr = np.concatenate([[0], np.cumsum([len(r) for r in rows])]).astype(np.int32)
    indices = np.concatenate(rows).astype(np.int32)
    out = torch.empty_like(dc.q)
    pkv.paged_attn_mixed_csr(out, dc.q, dc.kc, dc.vc, to_dev(indptr, gpu), to_dev(indices, gpu), dc.cu, dc.ctx,
                             case.scale, plan, case.k_scale, case.v_scale)
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16), dense.view(torch.int16))


def test_variant_decode_in_a_graph(gpu):
    """A decode call with a soft-cap and window plan of fixed capacity,
    captured once and replayed after re-plans of the same lengths, with
    eager work between replays: every replay equals the eager call."""
    import torch
    import paged_kv_attention_write_amd as pkv

    log("variant decode in a graph")
    case = workloads.build_case("vgr", 198, DECODE_LENS, [1] * len(DECODE_LENS), num_q_heads=32, num_kv_heads=8,
                                head_dim=128, block_size=16, scale=0.4)
    dc = DeviceCase(case, gpu)
    dc.write()
    B = len(DECODE_LENS)
    plan = _plan(case, gpu, False, 20.0, 700, 0, capacity=(B, B))
    eager = dc.decode(plan).clone()
    out = torch.empty_like(dc.q)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        dc.decode(plan, out)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        dc.decode(plan, out)
    torch.cuda.synchronize()
    for _ in range(3):
        out.zero_()
        plan.update(case.context_lens)
        g.replay()
        x = torch.randn(1 << 20, device=gpu)
        float((x * 2.0).sum())
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), eager.view(torch.int16))
    kr, vr = oracle_caches(case)
    ref, _ = oracle.paged_attention(case.q, case.q_dtype, kr, vr, case.kv_dtype, case.block_tables,
                                    case.context_lens, case.cu_seqlens, case.scale, case.k_scale, case.v_scale,
                                    soft_cap=20.0, window=700)
    check_close(as_f64(out), ref, "bf16", "graph decode cap 20 W 700")
