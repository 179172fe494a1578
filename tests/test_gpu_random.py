"""Seeded random batches through paged_attn_mixed against the fp64 oracle:
random lengths (including whole-prompt chunks and single keys), query rows,
page sizes (1, 3, 4, 16, 32, 48, 64), head shapes, bf16 or fp8 caches, and the
soft-cap / sliding-window variants, with a small queue count so that rows
are cut and merged."""

import numpy as np
import pytest

import oracle
import workloads
from gpu_helpers import DeviceCase, as_f64, check_close, log, oracle_caches

pytestmark = pytest.mark.gpu


def _draw(seed):
    rng = np.random.default_rng(5000 + seed)
    B = int(rng.integers(1, 12))
    lens = rng.integers(1, 3000, size=B)
    ql = np.where(rng.random(B) < 0.4, rng.integers(2, 200, size=B), 1)
    ql = np.minimum(ql, lens)
    whole = (rng.random(B) < 0.15) & (lens < 400)
    ql[whole] = lens[whole]
    hq, hkv, d = [(32, 8, 128), (16, 4, 64), (8, 8, 128), (16, 8, 64)][int(rng.integers(0, 4))]
    bs = int(rng.choice([1, 3, 4, 16, 32, 48, 64]))
    kv = "fp8" if rng.random() < 0.25 else "bf16"
    cap = float(rng.choice([0.0, 0.0, 8.0]))
    window = int(rng.choice([0, 0, 33, 500]))
    nq = int(rng.integers(3, 40))
    return lens.astype(int), ql.astype(int), hq, hkv, d, bs, kv, cap, window, nq


@pytest.mark.parametrize("seed", range(10))
def test_random_mixed_batches(gpu, seed):
    import paged_kv_attention_write_amd as pkv

    lens, ql, hq, hkv, d, bs, kv, cap, window, nq = _draw(seed)
    log(f"random seed {seed}: B={len(lens)} T={int(ql.sum())} {hq}/{hkv}/{d} bs={bs} {kv} cap={cap} W={window} "
        f"queues={nq}")
    case = workloads.build_case(f"rnd{seed}", 300 + seed, lens, ql, num_q_heads=hq, num_kv_heads=hkv, head_dim=d,
                                block_size=bs, kv_dtype=kv, scale=0.2)
    dc = DeviceCase(case, gpu)
    dc.write()
    plan = pkv.Plan(case.context_lens, case.q_lens, num_q_heads=hq, num_kv_heads=hkv, head_dim=d, device=gpu,
                    num_queues=nq, soft_cap=cap, window=window)
    out = as_f64(dc.mixed(plan))
    kr, vr = oracle_caches(case)
    ref, _ = oracle.paged_attention(case.q, case.q_dtype, kr, vr, case.kv_dtype, case.block_tables,
                                    case.context_lens, case.cu_seqlens, case.scale, case.k_scale, case.v_scale,
                                    soft_cap=cap, window=window)
    check_close(out, ref, kv, f"random seed {seed}")
