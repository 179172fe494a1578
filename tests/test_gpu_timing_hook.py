"""GPU test of the timing hook pkv_set_split_event: while it is set, decode
and mixed calls record the event between their attention kernel and their
merge kernel, and their outputs stay byte for byte those of calls made
without it.  Each case prints its name first."""

import numpy as np
import pytest

import workloads
from gpu_helpers import DeviceCase, log, to_host

pytestmark = pytest.mark.gpu


def test_split_event_falls_between_the_call_events(gpu):
    import torch

    import paged_kv_attention_write_amd as pkv

    log("split event: decode and decode+write calls")
    case = workloads.build_case("split", 91, [1, 17, 100, 513, 2047, 3000, 64, 900], [1] * 8, num_q_heads=32,
                                num_kv_heads=8, head_dim=128, block_size=16)
    d = DeviceCase(case, gpu)
    d.write()
    plan = d.plan(5)  # pieces, so that the merge kernel runs
    ref = to_host(d.decode(plan))
    stream = torch.cuda.current_stream()
    e0, em, e1 = (torch.cuda.Event(enable_timing=True) for _ in range(3))
    em.record(stream)  # gives the event its HIP handle
    c = case
    try:
        pkv.set_split_event(em)
        out = torch.empty_like(d.q)
        e0.record(stream)
        pkv.paged_attn_decode(out, d.q, d.kc, d.vc, d.tables, d.ctx, c.scale, plan, c.k_scale, c.v_scale)
        e1.record(stream)
    finally:
        pkv.set_split_event(None)
    torch.cuda.synchronize()
    kern, call = e0.elapsed_time(em), e0.elapsed_time(e1)
    assert 0.0 < kern <= call, (kern, call)
    assert np.array_equal(to_host(out).view(np.uint16), ref.view(np.uint16))
    # unset: a later call does not record it
    before = e0.elapsed_time(em)
    out2 = torch.empty_like(d.q)
    pkv.paged_attn_decode(out2, d.q, d.kc, d.vc, d.tables, d.ctx, c.scale, plan, c.k_scale, c.v_scale)
    torch.cuda.synchronize()
    assert e0.elapsed_time(em) == before
    assert np.array_equal(to_host(out2).view(np.uint16), ref.view(np.uint16))


def test_split_event_on_a_mixed_call(gpu):
    import torch

    import paged_kv_attention_write_amd as pkv

    log("split event: mixed call")
    case = workloads.build_case("splitm", 92, [700, 40, 1500, 2600], [1, 1, 1, 200], num_q_heads=32,
                                num_kv_heads=8, head_dim=128, block_size=16)
    d = DeviceCase(case, gpu)
    d.write()
    plan = d.plan(0, mixed=True)
    ref = to_host(d.mixed(plan))
    stream = torch.cuda.current_stream()
    e0, em, e1 = (torch.cuda.Event(enable_timing=True) for _ in range(3))
    em.record(stream)
    try:
        pkv.set_split_event(em)
        e0.record(stream)
        out = d.mixed(plan)
        e1.record(stream)
    finally:
        pkv.set_split_event(None)
    torch.cuda.synchronize()
    assert 0.0 < e0.elapsed_time(em) <= e0.elapsed_time(e1)
    assert np.array_equal(to_host(out).view(np.uint16), ref.view(np.uint16))
