"""GPU parity of paged_attn_decode_write: a decode step's write and attention
in one call, against the fp64 oracle of the write followed by attention, and
byte for byte against the two separate calls (paged_kv_write then
paged_attn_decode) on a copy of the same pools.

The slots the new tokens go to are poisoned with NaN before the call (see
workloads), so a key read before its write lands shows up as a NaN row.
Tolerances as in test_gpu_decode.py.  Each case prints its name first.
"""

import numpy as np
import pytest

import workloads
from gpu_helpers import DeviceCase, as_f64, check_close, log, oracle_attention, oracle_caches, to_dev, to_host

pytestmark = pytest.mark.gpu


def _fused(dc, plan, slots=None):
    import torch

    import paged_kv_attention_write_amd as pkv

    c = dc.case
    out = torch.empty_like(dc.q)
    pkv.paged_attn_decode_write(out, dc.q, dc.k_new, dc.v_new, dc.slots if slots is None else slots, dc.kc, dc.vc,
                                dc.tables, dc.ctx, c.scale, plan, c.k_scale, c.v_scale)
    return out


def _both(case, gpu, num_queues):
    """(fused output, fused pools, two-call output, two-call pools, plan)."""
    d1, d2 = DeviceCase(case, gpu), DeviceCase(case, gpu)
    plan = d1.plan(num_queues)
    out1 = _fused(d1, plan)
    d2.write()
    out2 = d2.decode(plan)
    return out1, d1, out2, d2, plan


@pytest.mark.parametrize("num_queues", [0, 1, 5, 24])
def test_fused_write_matches_the_two_calls(gpu, num_queues):
    """bf16 pools, page 16, sequences cut into pieces at most queue counts: the
    fused call writes the same bytes as paged_kv_write and returns the same
    output as paged_attn_decode after it, within tolerance of the oracle."""
    log(f"decode+write bf16 queues={num_queues}")
    case = workloads.build_case("dw", 81, [1, 17, 100, 513, 2047, 3000, 64, 900], [1] * 8, num_q_heads=32,
                                num_kv_heads=8, head_dim=128, block_size=16)
    out1, d1, out2, d2, plan = _both(case, gpu, num_queues)
    assert np.array_equal(to_host(d1.kc).view(np.uint16), to_host(d2.kc).view(np.uint16))
    assert np.array_equal(to_host(d1.vc).view(np.uint16), to_host(d2.vc).view(np.uint16))
    assert np.array_equal(to_host(out1).view(np.uint16), to_host(out2).view(np.uint16))
    kr, vr = oracle_caches(case)
    assert np.array_equal(to_host(d1.kc).view(np.uint16), kr.view(np.uint16))
    ref, _ = oracle_attention(case, kr, vr)
    check_close(as_f64(out1), ref, "bf16", f"fused write merges={plan.desc.num_merges}")


@pytest.mark.parametrize("bs", [1, 3, 16, 48])
@pytest.mark.parametrize("hq,hkv,d", [(16, 4, 128), (8, 8, 64), (8, 1, 128), (12, 3, 64), (128, 16, 128)])
def test_fused_write_shapes(gpu, bs, hq, hkv, d):
    """Pages of whole 16-token tiles (16, 48: one launch) and others (1, 3: the
    write kernel, then the decode call), head shapes, default queues and
    three queues (pieces)."""
    log(f"decode+write bs={bs} {hq}/{hkv}/{d}")
    case = workloads.build_case(f"dw{bs}", 82 + bs, [1, 30, 257, 1000], [1] * 4, num_q_heads=hq,
                                num_kv_heads=hkv, head_dim=d, block_size=bs)
    for nq in (0, 3):
        out1, d1, out2, d2, _ = _both(case, gpu, nq)
        assert np.array_equal(to_host(d1.kc).view(np.uint16), to_host(d2.kc).view(np.uint16))
        assert np.array_equal(to_host(out1).view(np.uint16), to_host(out2).view(np.uint16))
    kr, vr = oracle_caches(case)
    ref, _ = oracle_attention(case, kr, vr)
    check_close(as_f64(out1), ref, "bf16", f"bs={bs}")


def test_fused_write_fp32(gpu):
    """fp32 q and pools take the two launches."""
    log("decode+write fp32 tiny")
    case = workloads.make_case("tiny")
    for nq in (1, 3, 12):
        out1, d1, out2, d2, _ = _both(case, gpu, nq)
        assert np.array_equal(to_host(d1.kc), to_host(d2.kc), equal_nan=True)
        assert np.array_equal(to_host(out1), to_host(out2))
    kr, vr = oracle_caches(case)
    ref, _ = oracle_attention(case, kr, vr)
    check_close(as_f64(out1), ref, "f32", "fused write fp32")


def test_fused_write_fp8_cache_takes_the_two_launches(gpu):
    """An fp8 cache (bf16 tokens converted by the write): the write kernel then
    the decode call, the same bytes and output as the two calls."""
    log("decode+write fp8")
    case = workloads.build_case("dw8", 90, [40, 700, 1500], [1, 1, 1], num_q_heads=16, num_kv_heads=4,
                                head_dim=128, block_size=16, kv_dtype="fp8")
    out1, d1, out2, d2, _ = _both(case, gpu, 0)
    assert np.array_equal(to_host(d1.kc), to_host(d2.kc))
    assert np.array_equal(to_host(out1).view(np.uint16), to_host(out2).view(np.uint16))
    kr, vr = oracle_caches(case)
    ref, _ = oracle_attention(case, kr, vr)
    check_close(as_f64(out1), ref, "fp8", "fused write fp8")


def test_negative_slot_writes_nothing(gpu):
    """slot_mapping[s] < 0: nothing is written for s, and its row is attention
    over the pool as it is (here the poisoned slot: NaN), as the two calls give."""
    import torch

    import paged_kv_attention_write_amd as pkv

    log("decode+write negative slot")
    case = workloads.build_case("dwneg", 91, [50, 600, 1200], [1, 1, 1], num_q_heads=16, num_kv_heads=4,
                                head_dim=128, block_size=16)
    slots = case.slot_mapping.copy()
    slots[1] = -1
    d1, d2 = DeviceCase(case, gpu), DeviceCase(case, gpu)
    plan = d1.plan(3)
    out1 = _fused(d1, plan, to_dev(slots, gpu))
    pkv.paged_kv_write(d2.k_new, d2.v_new, to_dev(slots, gpu), d2.kc, d2.vc)
    out2 = d2.decode(plan)
    torch.cuda.synchronize()
    assert np.array_equal(to_host(d1.kc).view(np.uint16), to_host(d2.kc).view(np.uint16))
    assert np.array_equal(to_host(out1).view(np.uint16), to_host(out2).view(np.uint16))
    o = as_f64(out1)
    assert np.all(np.isnan(o[1])) and not np.any(np.isnan(o[[0, 2]]))


def test_slot_other_than_the_key_gives_nan_row_and_no_write(gpu):
    """slot_mapping[s] naming another slot than key context_lens[s] - 1: in the
    one-launch path the row comes out NaN and nothing is written for it; the
    other rows match the oracle."""
    log("decode+write wrong slot")
    case = workloads.build_case("dwbad", 92, [50, 600, 1200], [1, 1, 1], num_q_heads=16, num_kv_heads=4,
                                head_dim=128, block_size=16)
    slots = case.slot_mapping.copy()
    other = int(case.block_tables[1, 0]) * 16 + 3  # key 3 of sequence 1
    slots[1] = other
    d1 = DeviceCase(case, gpu)
    before = to_host(d1.kc).copy()
    plan = d1.plan(3)
    out1 = as_f64(_fused(d1, plan, to_dev(slots, gpu)))
    after = to_host(d1.kc)
    nb, bs = after.shape[0], after.shape[1]
    flat_b, flat_a = before.reshape(nb * bs, -1), after.reshape(nb * bs, -1)
    assert np.array_equal(flat_a[other].view(np.uint16), flat_b[other].view(np.uint16))
    assert np.array_equal(flat_a[case.slot_mapping[1]].view(np.uint16), flat_b[case.slot_mapping[1]].view(np.uint16))
    assert np.all(np.isnan(out1[1]))
    kr, vr = oracle_caches(case)
    ref, _ = oracle_attention(case, kr, vr)
    check_close(out1[[0, 2]], ref[[0, 2]], "bf16", "rows beside the wrong slot")


def test_fused_write_full_decode_workload(gpu):
    """64 x U[512, 4096] at 32/8/128, default queues: the benchmark's step."""
    log("decode+write full size")
    case = workloads.make_case("decode")
    out1, d1, out2, d2, plan = _both(case, gpu, 0)
    assert np.array_equal(to_host(out1).view(np.uint16), to_host(out2).view(np.uint16))
    assert np.array_equal(to_host(d1.kc).view(np.uint16), to_host(d2.kc).view(np.uint16))
    kr, vr = oracle_caches(case, inplace=True)
    ref, _ = oracle_attention(case, kr, vr)
    check_close(as_f64(out1), ref, "bf16", f"full decode+write units={plan.desc.num_units}")
