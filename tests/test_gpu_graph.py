"""Attention calls captured into a HIP graph (torch.cuda.CUDAGraph) and
replayed: a multi-layer step of write + decode, and decode / mixed calls whose
lengths change between replays (plans of one capacity made into the same
workspace, lengths updated in place).

Every replay is compared with eager calls on the same inputs, bit for bit
(same kernels, same plan content), and with the fp64 oracle.  Replays are
interleaved with eager work and synchronisations, several times over.
"""

import numpy as np
import pytest

import workloads
from gpu_helpers import DeviceCase, as_f64, check_close, log, oracle_attention, oracle_caches, to_dev

pytestmark = pytest.mark.gpu


def _graph(torch, fn):
    """Warm fn up eagerly on a side stream, then capture it."""
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        fn()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    torch.cuda.synchronize()
    return g


def _eager_noise(torch, gpu):
    x = torch.randn(1 << 20, device=gpu)
    y = (x * 2.0 + 1.0).sum()
    torch.cuda.synchronize()
    return float(y)


def test_graph_multi_layer_write_and_decode(gpu):
    """Three layers of (write + decode), each over its own pool, in one graph."""
    import torch
    import paged_kv_attention_write_amd as pkv

    log("graph: 3 layers of write + decode")
    lens = [50, 900, 33, 1500, 17, 3000]
    B = len(lens)
    layers = []
    for l in range(3):
        case = workloads.build_case(f"g{l}", 120 + l, lens, [1] * B, num_q_heads=32, num_kv_heads=8, head_dim=128,
                                    block_size=16)
        layers.append((case, DeviceCase(case, gpu)))
    c0 = layers[0][0]
    plan = pkv.Plan(c0.context_lens, None, num_q_heads=32, num_kv_heads=8, head_dim=128, device=gpu,
                    capacity=(B, B))
    outs = [torch.empty_like(dc.q) for _, dc in layers]

    def step():
        for (case, dc), out in zip(layers, outs):
            dc.write()
            dc.decode(plan, out)

    step()
    torch.cuda.synchronize()
    eager = [o.clone() for o in outs]
    g = _graph(torch, step)
    for rep in range(3):
        for o in outs:
            o.fill_(float("nan"))
        _eager_noise(torch, gpu)
        g.replay()
        torch.cuda.synchronize()
        for l, o in enumerate(outs):
            assert torch.equal(o.view(torch.int16), eager[l].view(torch.int16)), f"replay {rep} layer {l}"
    for (case, dc), o in zip(layers, outs):
        kr, vr = oracle_caches(case)
        ref, _ = oracle_attention(case, kr, vr)
        check_close(as_f64(o), ref, "bf16", "graph layer")


@pytest.mark.parametrize("kind", ["decode", "mixed"])
def test_graph_replay_across_length_changes(gpu, kind):
    import torch
    import paged_kv_attention_write_amd as pkv

    log(f"graph: {kind} across length changes")
    if kind == "decode":
        sets = [[50, 900, 33, 1500, 17, 3000], [51, 901, 34, 1501, 18, 3001], [700, 20, 2600, 64, 1200, 5]]
        ql = [1] * 6
    else:
        sets = [[40, 900, 600, 1300], [41, 901, 700, 1400], [300, 64, 560, 1200]]
        ql = [1, 1, 96, 1]
    top = np.max(np.asarray(sets), axis=0)
    case = workloads.build_case(f"glen-{kind}", 130, top.tolist(), ql, num_q_heads=32, num_kv_heads=8,
                                head_dim=128, block_size=16)
    dc = DeviceCase(case, gpu)
    dc.write()  # the newest keys of the longest set (poisoned until written)
    kr, vr = oracle_caches(case)
    B, T = len(ql), int(np.sum(ql))
    mixed = kind == "mixed"
    qls = np.asarray(ql, np.int32) if mixed else None
    plan = pkv.Plan(np.asarray(sets[0], np.int32), qls, num_q_heads=32, num_kv_heads=8, head_dim=128, device=gpu,
                    capacity=(B, T))
    out = torch.empty_like(dc.q)

    def call(p, o):
        (dc.mixed if mixed else dc.decode)(p, o)

    dc.ctx.copy_(to_dev(np.asarray(sets[0], np.int32), gpu))
    g = _graph(torch, lambda: call(plan, out))
    for rep in range(2):
        for i, lens in enumerate(sets):
            lens = np.asarray(lens, np.int32)
            plan.update(lens, qls)
            dc.ctx.copy_(to_dev(lens, gpu))
            out.fill_(float("nan"))
            _eager_noise(torch, gpu)
            g.replay()
            torch.cuda.synchronize()
            # eager call with a compact plan for the same lengths
            ref_plan = pkv.Plan(lens, qls, num_q_heads=32, num_kv_heads=8, head_dim=128, device=gpu)
            eager = torch.empty_like(out)
            call(ref_plan, eager)
            torch.cuda.synchronize()
            assert torch.equal(out.view(torch.int16), eager.view(torch.int16)), f"replay {rep} set {i}"
            log(f"  set {i}: merges {plan.desc.num_merges} wide {plan.desc.num_wide_merges} "
                f"(room {plan.desc.max_row_merges} rows, {plan.desc.max_block_merges} blocks)")
            if rep == 0:
                import oracle
                ref, _ = oracle.paged_attention(case.q, case.q_dtype, kr, vr, case.kv_dtype, case.block_tables,
                                                lens, case.cu_seqlens, case.scale, case.k_scale, case.v_scale)
                check_close(as_f64(out), ref, "bf16", f"{kind} set {i}")
